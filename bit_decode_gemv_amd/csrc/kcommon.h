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
// scalar registers.  Both bytes sit at the top of the two 16-bit halves of
// one register, so each plane costs one packed 16-bit shift and two 16-bit
// sign tests (the upper half's through a sub-dword operand select).
struct XPlanes {
    uint32_t w[8][4];
};

typedef short short2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void ballot_planes(int xa, int xb, XPlanes &xp) {
    short2v p;
    p.x = (short)((uint32_t)xa << 8);   // the byte's bit 7 at the 16-bit sign
    p.y = (short)((uint32_t)xb << 8);
#pragma unroll
    for (int b = 7; b >= 0; --b) {
        const uint64_t m0 = __ballot(p.x < 0);
        const uint64_t m1 = __ballot(p.y < 0);
        xp.w[b][0] = (uint32_t)m0;
        xp.w[b][1] = (uint32_t)(m0 >> 32);
        xp.w[b][2] = (uint32_t)m1;
        xp.w[b][3] = (uint32_t)(m1 >> 32);
        p = p << (short)1;
    }
}

// popcount(v) + acc as one v_bcnt_u32_b32, whose second operand is an
// addend.  Written as inline assembly so that a chain of counts stays one
// chain: the compiler would otherwise re-associate the sums into separate
// counts and three-operand adds, one more instruction per four counts.
__device__ __forceinline__ int bcnt_add(uint32_t v, int acc) {
    int r;
    asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(acc));
    return r;
}

// Raw buffer resource over `bytes` bytes at base (gfx9-family descriptor
// word 3).  A load through it takes a per-lane offset in a vector register
// and a wavefront-uniform one in a scalar register, so a loop that steps a
// uniform offset keeps its address arithmetic on the scalar unit; offsets at
// or past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes, non-temporal (cache policy bit 1), at voff + soff.
__device__ __forceinline__ uint4 buffer_load_stream16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                      uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bits, sign-extended, non-temporal.
__device__ __forceinline__ int buffer_load_stream_i16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                      uint32_t soff) {
    return (int)(int16_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 2);
}

__device__ __forceinline__ int buffer_load_i8(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
    return (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

__device__ __forceinline__ int buffer_load_i16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    return (int)(int16_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Uniform broadcast of lane `i`'s value (v_readlane with a scalar index).
__device__ __forceinline__ int lane_value(int v, int i) {
    return __builtin_amdgcn_readlane(v, i);
}

}  // namespace bs
