// Wavefront and workgroup maxima of 64-bit values by DPP lane moves (no LDS
// round trip per step); gfx950, wave64.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bs {

// v against its DPP-moved copy (CTRL: the data-parallel-primitive lane
// pattern; ROWS: the 16-lane rows written), per 32-bit half; lanes the
// pattern gives no source keep their own value.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWS, 0xF, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWS, 0xF, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

// The largest v of the wavefront, in lane 63: row shifts by 1, 2, 4 and 8,
// then lane 15 broadcast into the next row and lane 31 into the upper two.
__device__ __forceinline__ uint64_t wave_max_u64_lane63(uint64_t v) {
    v = dpp_max_u64<0x111, 0xF>(v);   // row_shr:1
    v = dpp_max_u64<0x112, 0xF>(v);   // row_shr:2
    v = dpp_max_u64<0x114, 0xF>(v);   // row_shr:4
    v = dpp_max_u64<0x118, 0xF>(v);   // row_shr:8
    v = dpp_max_u64<0x142, 0xA>(v);   // row_bcast:15, rows 1 and 3
    v = dpp_max_u64<0x143, 0xC>(v);   // row_bcast:31, rows 2 and 3
    return v;
}

// The workgroup maximum of v (workgroups of up to 16 wavefronts), in every
// thread: each wavefront's by DPP moves, its lane 63 writing a slot;
// wavefront 0 folds the slots in one 16-lane row and every thread reads the
// result (a fold in every thread would repeat the same VALU work in all of
// the workgroup's wavefronts).  Every thread calls; red[16] and fin[1] in
// LDS, reusable after the next barrier.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t *red, uint64_t *fin) {
    v = wave_max_u64_lane63(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    if (lane == 63) red[wave] = v;
    __syncthreads();
    if (wave == 0) {
        uint64_t x = lane < nw ? red[lane < 16 ? lane : 0] : 0;
        x = dpp_max_u64<0x111, 0xF>(x);   // row_shr:1
        x = dpp_max_u64<0x112, 0xF>(x);   // row_shr:2
        x = dpp_max_u64<0x114, 0xF>(x);   // row_shr:4
        x = dpp_max_u64<0x118, 0xF>(x);   // row_shr:8
        if (lane == 15) *fin = x;
    }
    __syncthreads();
    return *fin;
}

}  // namespace bs
