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

// Bit planes of one group's 128 int8 activations, uniform across the
// wavefront: w[b][d] holds bit b (two's complement, bit 7 has weight -128) of
// positions 32d..32d+31, position 32d+i in bit i.  Lane l supplies positions
// l (xa) and 64 + l (xb), sign-extended; sixteen ballots build the planes in
// scalar registers.
struct XPlanes {
    uint32_t w[8][4];
};

__device__ __forceinline__ void ballot_planes(int xa, int xb, XPlanes &xp) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint64_t m0 = __ballot(b == 7 ? xa < 0 : (xa & (1 << b)) != 0);
        const uint64_t m1 = __ballot(b == 7 ? xb < 0 : (xb & (1 << b)) != 0);
        xp.w[b][0] = (uint32_t)m0;
        xp.w[b][1] = (uint32_t)(m0 >> 32);
        xp.w[b][2] = (uint32_t)m1;
        xp.w[b][3] = (uint32_t)(m1 >> 32);
    }
}

// Uniform broadcast of lane `i`'s value (v_readlane with a scalar index).
__device__ __forceinline__ int lane_value(int v, int i) {
    return __builtin_amdgcn_readlane(v, i);
}

}  // namespace bs
