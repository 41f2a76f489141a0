// Device helpers shared by the library's HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bs_internal.h"

namespace bs {

// Native 4 x 32-bit vector (global_load_dwordx4), usable with the
// non-temporal load builtin.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint8_t *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Launch a kernel and map any launch error to BS_E_HIP.
#define BS_LAUNCH_CHECK()                                   \
    do {                                                    \
        if (hipGetLastError() != hipSuccess) return BS_E_HIP; \
    } while (0)

// Bit planes of 128 int8 activations: w[b][d] holds bit b (two's complement,
// bit 7 has weight -128) of positions 32d..32d+31, position 32d+i in bit i.
// Built with wavefront ballots, so every value is uniform across the wave
// and lives in scalar registers.
struct XPlanes {
    uint32_t w[8][4];
};

__device__ __forceinline__ void ballot_planes(const int8_t *__restrict__ xg, XPlanes &xp) {
    const int lane = threadIdx.x & 63;
    const int v0 = xg[lane];
    const int v1 = xg[64 + lane];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint64_t m0 = __ballot((v0 >> b) & 1);
        const uint64_t m1 = __ballot((v1 >> b) & 1);
        xp.w[b][0] = (uint32_t)m0;
        xp.w[b][1] = (uint32_t)(m0 >> 32);
        xp.w[b][2] = (uint32_t)m1;
        xp.w[b][3] = (uint32_t)(m1 >> 32);
    }
}

// Signed sum of one 128-weight group against bit-planed activations:
//   sum_i t_i x_i = sum_b w_b (popcount(nz & X_b) - 2 popcount(neg & X_b)),
// w_b = 2^b for b < 7 and -128 for b = 7 (t_i = nz_i - 2 neg_i).
__device__ __forceinline__ int group_dot(const uint32_t nz[4], const uint32_t ng[4],
                                         const XPlanes &xp) {
    int s = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        int cn = 0, cg = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            cn += __builtin_popcount(nz[d] & xp.w[b][d]);
            cg += __builtin_popcount(ng[d] & xp.w[b][d]);
        }
        const int t = cn - 2 * cg;
        s += (b == 7) ? -t * 128 : t * (1 << b);
    }
    return s;
}

// Uniform broadcast of lane `i`'s value (v_readlane with a scalar index).
__device__ __forceinline__ int lane_value(int v, int i) {
    return __builtin_amdgcn_readlane(v, i);
}

}  // namespace bs
