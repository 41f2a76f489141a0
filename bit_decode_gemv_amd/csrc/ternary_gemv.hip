// bs_ternary_gemv: exact batch-1 ternary GEMV on gfx950.
//
// Computes, per row r, y[r] = sum_g floor(scale[r][g] * s[r][g] / 2^frac)
// with s the masked signed sum of the ternary row against int8 activations
// ("A standalone deterministic integer inference engine for BitNet-style
// LLMs", section 4.2; the W_nonzero / W_negative planes of "BitState / HSDR
// PoC Technical Brief - v0.5", section 4).
//
// Mappings.  Up to K = 16384 (128 groups) both GEMVs run the pipelined
// mapping (ternary_pipe_kernel): a workgroup owns R = 8, 16 or 32 rows of one
// 64-row tile and all of K; its wavefronts are split into 64/R slices of R
// lanes (lane = row) that take interleaved 128-weight groups.  The workgroup
// reads x once, transposes it into eight bit planes per group in LDS (8x8
// bit transposes; one barrier), and every lane streams its row's 16-byte
// plane fields of its groups through buffer resources bounded at the tile,
// so loads past K read zero and none is predicated.  The inner loop works on
// the signed population of the brief's section 4 through the identity
// t*m = nz*(m xor neg) - neg (t = nz - 2 neg): per 32 weights and activation
// bit plane, one AND-XOR (v_bitop3) and one popcount chained through its
// addend.  Slices meet by lane permutations, wavefronts in LDS; integer sums
// make the result independent of that order (integer-engine page, section
// 3.2), and each row is stored once.
//
// Beyond 128 groups, the row-block mapping (per-wavefront LDS staging, no
// workgroup barrier).  bs_ternary_gemv_acc (y += W x, the residual-stream
// update of a decoder layer) runs the tile mapping (one workgroup per 64-row
// tile and run of groups, activation bit planes from sixteen ballots into
// scalar registers), each workgroup adding its rows' partial sums to y with
// int64 atomics.
//
// bs_q1_gemv runs the same kernels on Q1_0 weights (integer-engine page,
// section 4.1): one sign bit per weight (1 = +1, 0 = -1) in the layout of the
// ternary W_nonzero plane, signed_sum = 2 * pos_sum - block_total, where
// block_total (the group's sum of x, shared by every row) is reduced across
// the group's 16 staging lanes and kept beside the group's bit planes in LDS,
// and pos_sum = sum_b 2^b popcount(bits & M_b) (-128 for b = 7).
#include "kcommon.h"

namespace bs {
namespace {

constexpr int kPlaneStride = 9;   // uint4 per group in LDS: 8 planes + 1 pad

__device__ __forceinline__ uint64_t transpose8x8(uint64_t q) {
    // byte i of q = activation of position i; afterwards byte b holds bit b
    // of the eight positions, position i in bit i
    uint64_t t;
    t = (q ^ (q >> 7)) & 0x00AA00AA00AA00AAull;
    q = q ^ t ^ (t << 7);
    t = (q ^ (q >> 14)) & 0x0000CCCC0000CCCCull;
    q = q ^ t ^ (t << 14);
    t = (q ^ (q >> 28)) & 0x00000000F0F0F0F0ull;
    q = q ^ t ^ (t << 28);
    return q;
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// sum_b w_b sum_d popcount(f(b, d)) with plane weights w_b = 2^b for b < 7
// and -128 for b = 7, as a Horner scheme from the top plane down: the running
// sum doubles between planes and the four counts of a plane chain into it
// through the count instruction's addend (plane 7 enters as -2 * its count,
// which the six doublings that follow bring to -128).  One count per 32
// weights and plane, plus one doubling per plane.
template <typename F>
__device__ __forceinline__ int weighted_plane_count(F f) {
    int q = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) q = bcnt_add(f(7, d), q);
    int s = -2 * q;
#pragma unroll
    for (int b = 6; b >= 0; --b) {
#pragma unroll
        for (int d = 0; d < 4; ++d) s = bcnt_add(f(b, d), s);
        if (b > 0) s *= 2;
    }
    return s;
}

// sum_i t_i x_i over one group, from the two weight planes of this lane and
// the group's activation planes (bit b of the 128 activations, position i at
// bit i%32 of word i/32).  With t_i = nz_i - 2 neg_i (neg a subset of nz)
// every lane satisfies t_i * m_i = nz_i (m_i xor neg_i) - neg_i, so for
// activation bit plane b
//   sum_i t_i m_bi = popcount(nz & (M_b ^ neg)) - popcount(neg);
// over the plane weights w_b (2^b, and -128 for bit 7, summing to -1) the
// popcount(neg) terms add up to + popcount(neg).  xg[b] holds plane b (LDS
// staging of the row-block kernel).
__device__ __forceinline__ int group_dot(const uint4 &nz, const uint4 &ng,
                                         const uint4 *__restrict__ xg) {
    int s = weighted_plane_count(
        [&](int b, int d) { return word(nz, d) & (word(xg[b], d) ^ word(ng, d)); });
#pragma unroll
    for (int d = 0; d < 4; ++d) s = bcnt_add(word(ng, d), s);
    return s;
}

// Q1_0: 2 * pos_sum - block_total for one group; xg[8].x holds block_total.
__device__ __forceinline__ int q1_group_dot(const uint4 &bits, const uint4 *__restrict__ xg) {
    const int pos =
        weighted_plane_count([&](int b, int d) { return word(bits, d) & word(xg[b], d); });
    return 2 * pos - (int)xg[8].x;
}

// The same two sums against scalar-register activation planes (tile
// mapping): xp.w[b][d] is uniform across the wavefront.
__device__ __forceinline__ int tile_dot(const uint4 &nz, const uint4 &ng, const XPlanes &xp) {
    int s = weighted_plane_count(
        [&](int b, int d) { return word(nz, d) & (xp.w[b][d] ^ word(ng, d)); });
#pragma unroll
    for (int d = 0; d < 4; ++d) s = bcnt_add(word(ng, d), s);
    return s;
}

// v summed with the lane 16 (SWAP32 false) or 32 (true) apart, in every lane:
// the gfx950 permlane swaps exchange 16-lane rows (odd rows of one operand
// with even rows of the other) or 32-lane halves at VALU rate; with both
// operands v, the two results are v and its partner, whose sum is wanted.
// int64 goes as two 32-bit halves.
template <bool SWAP32>
__device__ __forceinline__ int64_t add_partner(int64_t v) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)((uint64_t)v >> 32);
    uint32_t l0, l1, h0, h1;
    if constexpr (SWAP32) {
        const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        l0 = l[0]; l1 = l[1]; h0 = h[0]; h1 = h[1];
    } else {
        const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        l0 = l[0]; l1 = l[1]; h0 = h[0]; h1 = h[1];
    }
    return (int64_t)(((uint64_t)h0 << 32) | l0) + (int64_t)(((uint64_t)h1 << 32) | l1);
}

// Wait for this wavefront's LDS writes (or reads) to complete; the slot is
// private to the wavefront, so no workgroup barrier is involved.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_wave_barrier();
}

// R rows per block, up to MAXG groups per slice in flight per round.  The
// wavefront's LDS slot holds the planes of its (64/R) * MAXG round groups,
// local index li = q * (64/R) + (slice within the wavefront).
template <int R, int MAXG, bool Q1>
__global__ void ternary_rows_kernel(const uint8_t *__restrict__ planes,
                                    const int16_t *__restrict__ pscales,
                                    const int8_t *__restrict__ x, int rows, int groups,
                                    int shift, int64_t *__restrict__ y) {
    constexpr int S = 64 / R;                 // slices per wavefront
    constexpr int LG = S * MAXG;              // groups per wavefront per round
    constexpr int PASSES = (LG * 16 + 63) / 64;
    __shared__ uint4 xpl[16][LG * kPlaneStride];
    __shared__ int64_t part[16][R];
    const int nwaves = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = lane % R, sl = lane / R;
    const int nslices = nwaves * S;
    const int slice0 = wave * S;             // first slice of this wavefront
    const int row = blockIdx.x * R + rr;
    const int tile = row >> 6, j = row & 63;
    const bool live = row < rows;
    uint4 *const slot = xpl[wave];
    uint8_t *const slot8 = reinterpret_cast<uint8_t *>(slot);

    int64_t acc = 0;
    for (int r0 = 0; slice0 + r0 * nslices < groups; r0 += MAXG) {
        // activations of this wavefront's round groups: task = 8 positions
        uint2 act[PASSES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int task = lane + 64 * p;
            const int li = task >> 4;
            const int g = slice0 + (li % S) + (r0 + li / S) * nslices;
            if (task < LG * 16 && g < groups)
                act[p] = *reinterpret_cast<const uint2 *>(x + (size_t)g * 128 + 8 * (task & 15));
        }
        uint4 wnz[MAXG], wng[MAXG];
        int sc[MAXG];
#pragma unroll
        for (int q = 0; q < MAXG; ++q) {
            const int g = slice0 + sl + (r0 + q) * nslices;
            if (live && g < groups) {
                const size_t blk = (size_t)tile * groups + g;
                if constexpr (Q1) {
                    wnz[q] = load_stream16(planes + blk * 1024 + 16 * j);
                } else {
                    wnz[q] = load_stream16(planes + blk * 2048 + 16 * j);
                    wng[q] = load_stream16(planes + blk * 2048 + 1024 + 16 * j);
                }
                sc[q] = pscales[((size_t)(row >> 4) * groups + g) * 16 + (row & 15)];
            }
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int task = lane + 64 * p;
            const int li = task >> 4;
            const int g = slice0 + (li % S) + (r0 + li / S) * nslices;
            const bool valid = task < LG * 16 && g < groups;
            if (valid) {
                const uint64_t t8 = transpose8x8((uint64_t)act[p].x | ((uint64_t)act[p].y << 32));
                const int piece = task & 15, d = piece >> 2, o = piece & 3;
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    slot8[((li * kPlaneStride + b) * 4 + d) * 4 + o] = (uint8_t)(t8 >> (8 * b));
            }
            if constexpr (Q1) {
                // block_total: the 16 lanes of a group (task & 15 = lane & 15)
                int sum8 = 0;
                if (valid) {
                    const uint64_t raw = (uint64_t)act[p].x | ((uint64_t)act[p].y << 32);
#pragma unroll
                    for (int i = 0; i < 8; ++i) sum8 += (int)(int8_t)(raw >> (8 * i));
                }
#pragma unroll
                for (int m = 8; m >= 1; m >>= 1) sum8 += __shfl_xor(sum8, m, 16);
                if (valid && (task & 15) == 0)
                    reinterpret_cast<int *>(slot + li * kPlaneStride + 8)[0] = sum8;
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int q = 0; q < MAXG; ++q) {
            const int g = slice0 + sl + (r0 + q) * nslices;
            if (live && g < groups) {
                const uint4 *xg = slot + (q * S + sl) * kPlaneStride;
                int s;
                if constexpr (Q1) s = q1_group_dot(wnz[q], xg);
                else s = group_dot(wnz[q], wng[q], xg);
                acc += (int64_t)((s * sc[q]) >> shift);   // arithmetic shift = floor
            }
        }
        wave_lds_fence();   // the next round overwrites the slot
    }
    // slices of one wavefront: lanes rr, rr+R, rr+2R, ...
    if constexpr (R == 16) acc = add_partner<false>(acc);
    if constexpr (R <= 32) acc = add_partner<true>(acc);
    if (lane < R) part[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < R) {
        int64_t tot = 0;
        for (int w = 0; w < nwaves; ++w) tot += part[w][threadIdx.x];
        const int r = blockIdx.x * R + threadIdx.x;
        if (r < rows) y[r] = tot;
    }
}

// One workgroup per (64-row tile, run of cg groups), W wavefronts (W <= 16),
// lane l of each serving row 64*tile + l; wavefront w takes the run's groups
// w, w + W, ... with one group's loads in flight at a time (more wavefronts,
// not deeper per-wavefront queues, measured faster).  The W partial sums per
// row meet in LDS; then the row's sum is stored (ACC false: one run covers
// all of K) or added to y with one int64 atomic per row and workgroup (ACC
// true: y += W x; the runs of a tile add in any order, exactly, since
// integer addition is associative).  Rows past `rows` (the tile's zero
// padding) are computed like the others and not stored.
__global__ void ternary_acc_kernel(const uint8_t *__restrict__ planes,
                                   const int16_t *__restrict__ pscales,
                                   const int8_t *__restrict__ x, int rows, int groups, int cg,
                                   int nruns, int shift, int64_t *__restrict__ y) {
    __shared__ int64_t part[16][64];
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int tile = (int)blockIdx.x / nruns;
    const int g0 = ((int)blockIdx.x - tile * nruns) * cg;
    const int g1 = min(groups, g0 + cg);
    const int row = tile * 64 + lane;
    const bool live = row < rows;
    // this tile's planes, its four 16-row scale blocks, and x: the group
    // steps a uniform (scalar) offset, the lane's part is fixed
    const __amdgpu_buffer_rsrc_t rp =
        buffer_rsrc(planes + (size_t)tile * groups * 2048, (uint32_t)groups * 2048);
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(pscales + (size_t)tile * 64 * groups, (uint32_t)groups * 128);
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x, (uint32_t)groups * 128);
    const uint32_t sc_off = (uint32_t)(((lane >> 4) * groups * 16 + (lane & 15)) * 2);
    int64_t acc = 0;
    for (int g = g0 + wave; g < g1; g += nwaves) {
        // padding rows (lane >= rows - 64 * tile) read the tile's zero rows
        const int xa = buffer_load_i8(rx, lane, g * 128);
        const int xb = buffer_load_i8(rx, 64 + lane, g * 128);
        const uint4 nz = buffer_load_stream16(rp, 16 * lane, g * 2048);
        const uint4 ng = buffer_load_stream16(rp, 1024 + 16 * lane, g * 2048);
        const int sc = buffer_load_i16(rs, sc_off, g * 32);
        XPlanes xp;
        ballot_planes(xa, xb, xp);
        const int s = tile_dot(nz, ng, xp);
        acc += (int64_t)(__mul24(s, sc) >> shift);   // |s * sc| <= 2^29; >> = floor
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < 64) {
        int64_t tot = 0;
        for (int w = 0; w < nwaves; ++w) tot += part[w][threadIdx.x];
        if (live) atomicAdd(reinterpret_cast<unsigned long long *>(y + row), (unsigned long long)tot);
    }
}

// v summed with the lane 8 apart within each 16-lane row (DPP row rotate by
// 8: lane i of a row reads lane (i + 8) mod 16, its xor-8 partner).
__device__ __forceinline__ int64_t add_partner8(int64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)((uint64_t)v >> 32);
    const uint32_t l = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, false);
    const uint32_t h = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, false);
    return v + (int64_t)(((uint64_t)h << 32) | l);
}

__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
    return make_uint2(v.x, v.y);
}

// Pipelined mapping.  A workgroup owns R rows of one 64-row tile (R = 8, 16,
// 32 or 64) and all of K; its NW wavefronts hold S = 64/R slices each, lane l of
// wavefront w serving row (l mod R) in slice w*S + l/R, and slice s takes the
// groups s, s + NW*S, ... (NG of them).  Phases:
//   1. every lane loads its share of x (8 bytes per chunk) and then the
//      weights of its first D groups: vmcnt retires loads in order, so the
//      activations can be used while the weights are still in flight;
//   2. the workgroup turns x into bit planes in LDS (one 8x8 bit transpose
//      per 8 positions; group g's plane b at xpl[g*9 + b], position i of the
//      group at bit i%32 of word i/32), then one barrier;
//   3. group q of the slice is computed while the loads of groups q+1..q+D
//      are in flight.
// Every load is unconditional: the buffer resources bound each one to its
// tile, its scale block and x, and a load past the end reads zero, so the
// wait counts are static and a padding slot contributes 0.  Slices of a
// wavefront meet by lane permutations, wavefronts in LDS.
template <int R, int NW, int NG, int D, bool Q1>
__global__ __launch_bounds__(NW * 64) void ternary_pipe_kernel(
    const uint8_t *__restrict__ planes, const int16_t *__restrict__ pscales,
    const int8_t *__restrict__ x, int rows, int groups, int shift, int64_t *__restrict__ y) {
    constexpr int S = 64 / R, NS = NW * S, NT = NW * 64;
    constexpr int MAXG = NS * NG;                    // groups the slots cover
    constexpr int XP = (MAXG * 16 + NT - 1) / NT;    // 8-position chunks per thread
    static_assert(R == 8 || R == 16 || R == 32 || R == 64, "row block");
    static_assert(D >= 1 && D <= NG, "pipeline depth");
    __shared__ uint4 xpl[(MAXG + 1) * kPlaneStride];  // + one slot for chunks past K
    __shared__ int64_t part[NW][R];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int sl = wave * S + lane / R;
    const int row0 = (int)blockIdx.x * R;
    const int tile = row0 >> 6;
    const int j = (row0 & 63) + lane % R;            // row within the tile
    constexpr uint32_t kBlk = Q1 ? 1024 : 2048;   // plane bytes per (tile, group)
    const __amdgpu_buffer_rsrc_t rp =
        buffer_rsrc(planes + (size_t)tile * groups * kBlk, (uint32_t)groups * kBlk);
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(pscales + (size_t)tile * 64 * groups, (uint32_t)groups * 128);
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x, (uint32_t)groups * 128);
    const uint32_t w_off = 16u * j;
    const uint32_t sc_off = (uint32_t)(((j >> 4) * groups * 16 + (j & 15)) * 2);

    // Scale loads: with several groups per slice non-temporal, like the
    // planes (0.13 to 0.3 us less per launch on the tall shapes); a lone
    // group per slice keeps the default policy (non-temporal measured slower
    // there: the two workgroups of a 16-row block share each scale line)
    auto load_scale = [&](uint32_t off) {
        return NG == 1 ? buffer_load_i16(rs, off, 0) : buffer_load_stream_i16(rs, off, 0);
    };
    uint2 xv[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) xv[p] = buffer_load8(rx, 8u * (threadIdx.x + p * NT));
    __builtin_amdgcn_sched_barrier(0);
    // the first D groups: scales, then planes (the compiler schedules a lone
    // scale load, NG = 1, after the barrier below; issuing it first measured
    // no faster)
    uint4 nz[NG], ng[NG];
    int sc[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        if (q < D) sc[q] = load_scale(sc_off + (uint32_t)(sl + q * NS) * 32u);
    }
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        if (q < D) {
            const uint32_t g = (uint32_t)(sl + q * NS);
            nz[q] = buffer_load_stream16(rp, g * kBlk + w_off, 0);
            if constexpr (!Q1) ng[q] = buffer_load_stream16(rp, g * kBlk + 1024u + w_off, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int c = threadIdx.x + p * NT;
        const uint64_t t8 = transpose8x8((uint64_t)xv[p].x | ((uint64_t)xv[p].y << 32));
        const int gi = c < groups * 16 ? (c >> 4) : MAXG;
        uint8_t *dst = reinterpret_cast<uint8_t *>(xpl + gi * kPlaneStride) + (c & 15);
#pragma unroll
        for (int b = 0; b < 8; ++b) dst[b * 16] = (uint8_t)(t8 >> (8 * b));
        if constexpr (Q1) {
            // block_total of the group in its padding slot: the group's 16
            // chunks are 16 consecutive lanes (NT is a multiple of 16)
            const uint64_t raw = (uint64_t)xv[p].x | ((uint64_t)xv[p].y << 32);
            int sum8 = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum8 += (int)(int8_t)(raw >> (8 * i));
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) sum8 += __shfl_xor(sum8, m, 16);
            if ((c & 15) == 0) reinterpret_cast<int *>(xpl + gi * kPlaneStride + 8)[0] = sum8;
        }
    }
    __syncthreads();
    int64_t acc = 0;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        if (q + D < NG) {
            const uint32_t g = (uint32_t)(sl + (q + D) * NS);
            nz[q + D] = buffer_load_stream16(rp, g * kBlk + w_off, 0);
            if constexpr (!Q1) ng[q + D] = buffer_load_stream16(rp, g * kBlk + 1024u + w_off, 0);
            sc[q + D] = load_scale(sc_off + g * 32u);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int g = sl + q * NS;
        const uint4 *xg = xpl + (g < groups ? g : 0) * kPlaneStride;   // padding: any group
        uint4 xr[Q1 ? 9 : 8];             // all eight planes (and Q1's total) in flight
#pragma unroll
        for (int b = 0; b < (Q1 ? 9 : 8); ++b) xr[b] = xg[b];
        int s;
        if constexpr (Q1) {
            // a padding slice's zero bits still give -block_total: its scale
            // is forced to 0 (the ternary form's zero planes give s = 0)
            s = g < groups ? q1_group_dot(nz[q], xr) : 0;
        } else {
            s = group_dot(nz[q], ng[q], xr);
        }
        acc += (int64_t)(__mul24(s, sc[q]) >> shift);   // |s * sc| <= 2^29; >> = floor
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (S == 8) acc = add_partner8(acc);
    if constexpr (S >= 4) acc = add_partner<false>(acc);
    if constexpr (S >= 2) acc = add_partner<true>(acc);
    if (lane < R) part[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < R) {
        int64_t tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += part[w][threadIdx.x];
        const int r = row0 + (int)threadIdx.x;
        if (r < rows) y[r] = tot;
    }
}

// Launch shape of the pipelined kernel: R rows per block, NW wavefronts,
// NG groups per slice, D groups in flight ahead of the one being computed.
// From sweeps on MI355X with cold weights (every (R, NW) with the fewest NG
// covering K, D = 1 to 3; each configuration checked bit-exact), the winners
// per K and row range:
//   K <= 3072:  under 2048 rows 8-row blocks, 1 group per slice; to 4096
//               rows 16-row blocks, to 10240 32-row blocks, both with 2
//               groups per slice and D = 1; taller 64-row blocks (a whole
//               tile) of 4 wavefronts;
//   K <= 5120:  from 10240 rows whole tiles of 8 wavefronts; 6400 to 10240
//               rows 32-row blocks of 4; else 16-row blocks, 2 per slice;
//   K <= 8192:  16-row blocks, 2 groups per slice, D = 1;
//   K <= 12288: 16-row blocks of 8 wavefronts, 3 groups per slice, D = 1;
//   K <= 16384: 32-row blocks of 8 wavefronts, 7 or 8 groups per slice.
// Per launch (events, back-to-back, cold weights, interleaved medians) against
// the previous table: 2560x2560 2.63 -> 2.53 us, 6912x2560 3.13 -> 3.08,
// 13824x2560 4.07 -> 3.81, 11008x4096 4.43 -> 4.21, 13824x5120 5.25 -> 5.22,
// 2560x6912 3.18 -> 3.09, 4096x11008 4.41 -> 4.34, 5120x13824 6.60 -> 6.07;
// 640x2560 unchanged (2.42).  Fewer, longer wavefronts won at long K (8 of 7
// groups beat 9 of 6), and whole-tile blocks on tall short-K matrices: one
// wavefront's 64 lanes then read a group's 1 KiB plane block as one run.
struct PipeCfg {
    int R, NW, NG, D;
};

constexpr int kPipeMaxGroups = 128;   // K <= 16384; larger K takes the row-block kernel

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
static inline int imin(int a, int b) { return a < b ? a : b; }

static PipeCfg choose_pipe(int64_t rows, int64_t groups) {
    if (groups <= 24) {
        if (rows < 2048) return {8, cdiv(groups, 8), 1, 1};
        if (rows <= 4096) return {16, cdiv(groups, 8), 2, 1};
        if (rows < 10240) return {32, cdiv(groups, 4), 2, 1};
        const int ng = cdiv(groups, 4);
        return {64, 4, ng, imin(ng, 2)};
    }
    if (groups <= 40) {
        if (rows >= 10240) return {64, 8, cdiv(groups, 8), 2};
        if (rows >= 6400) return {32, 4, cdiv(groups, 8), 2};
        return {16, cdiv(groups, 8), 2, 1};
    }
    if (groups <= 64) return {16, cdiv(groups, 8), 2, 1};
    if (groups <= 96) return {16, 8, 3, 1};
    return {32, 8, cdiv(groups, 16), 2};
}

// Q1_0 (half the plane bytes per group), from the same sweep: up to K = 3072
// 16-row blocks with two groups per slice (D = 2) up to 4096 rows, whole
// tiles of 4 wavefronts from 10240 (D up to 3), 32-row blocks of 4 between;
// up to K = 5120 from 10240 rows the ternary table's whole tiles; elsewhere
// the ternary table's blocks with D = 2 (one group in flight measured slower
// for Q1_0: 2560x6912 3.04 us against 3.16).  Per launch: 2560x2560 2.47 us,
// 13824x2560 3.52 -> 3.34, 2560x6912 3.04, 13824x5120 4.87 -> 4.34.
static PipeCfg choose_pipe_q1(int64_t rows, int64_t groups) {
    if (groups <= 24) {
        const int ng = cdiv(groups, 8);
        if (rows <= 4096) return {16, ng, 2, 2};
        if (rows >= 10240) return {64, 4, cdiv(groups, 4), imin(cdiv(groups, 4), 3)};
        return {32, 4, ng, imin(ng, 2)};
    }
    PipeCfg c = choose_pipe(rows, groups);
    c.D = imin(c.NG, 2);
    return c;
}

template <int R, int NW, int NG, int D, bool Q1>
static void launch_pipe1(hipStream_t st, const uint8_t *planes, const int16_t *scales,
                         const int8_t *x, int rows, int groups, int shift, int64_t *y) {
    const unsigned nblk = (unsigned)((rows + R - 1) / R);
    hipLaunchKernelGGL((ternary_pipe_kernel<R, NW, NG, D, Q1>), dim3(nblk), dim3(NW * 64), 0, st,
                       planes, scales, x, rows, groups, shift, y);
}

// The instantiated configurations (R, NW, NG, D): every one the two tables
// above can return for 1 to 128 groups.
#define BS_PIPE_CONFIGS(X)                                                                     \
    X(8, 1, 1, 1) X(8, 2, 1, 1) X(8, 3, 1, 1)                                                  \
    X(16, 1, 2, 1) X(16, 2, 2, 1) X(16, 3, 2, 1) X(16, 4, 2, 1)                                \
    X(16, 5, 2, 1) X(16, 6, 2, 1) X(16, 7, 2, 1) X(16, 8, 2, 1)                                \
    X(16, 1, 2, 2) X(16, 2, 2, 2) X(16, 3, 2, 2) X(16, 4, 2, 2)                                \
    X(16, 5, 2, 2) X(16, 6, 2, 2) X(16, 7, 2, 2) X(16, 8, 2, 2)                                \
    X(16, 8, 3, 1) X(16, 8, 3, 2)                                                              \
    X(32, 1, 2, 1) X(32, 2, 2, 1) X(32, 3, 2, 1) X(32, 4, 2, 1) X(32, 5, 2, 1) X(32, 6, 2, 1) \
    X(32, 4, 1, 1) X(32, 4, 2, 2) X(32, 4, 3, 2) X(32, 4, 4, 2) X(32, 4, 5, 2)                 \
    X(32, 8, 7, 2) X(32, 8, 8, 2)                                                              \
    X(64, 4, 1, 1) X(64, 4, 2, 2) X(64, 4, 3, 2) X(64, 4, 4, 2) X(64, 4, 5, 2) X(64, 4, 6, 2) \
    X(64, 4, 3, 3) X(64, 4, 4, 3) X(64, 4, 5, 3) X(64, 4, 6, 3)                                \
    X(64, 8, 4, 2) X(64, 8, 5, 2)

// Launches the configuration c, which must cover every group ((64 / R) * NW
// * NG >= groups: the LDS staging has a slot for each); false (no launch)
// for a configuration outside the instantiated set.
template <bool Q1>
static bool launch_pipe(const PipeCfg &c, hipStream_t st, const uint8_t *p, const int16_t *s,
                        const int8_t *x, int rows, int groups, int shift, int64_t *y) {
    if (c.R <= 0 || c.NW <= 0 || c.NG <= 0 || (64 / c.R) * c.NW * c.NG < groups) return false;
#define BS_PIPE_CASE(R_, NW_, NG_, D_)                                                         \
    if (c.R == R_ && c.NW == NW_ && c.NG == NG_ && c.D == D_) {                                \
        launch_pipe1<R_, NW_, NG_, D_, Q1>(st, p, s, x, rows, groups, shift, y);               \
        return true;                                                                           \
    }
    BS_PIPE_CONFIGS(BS_PIPE_CASE)
#undef BS_PIPE_CASE
    return false;
}

struct TernaryCfg {
    int rows_per_block;   // R: 32 or 16
    int waves;            // wavefronts per block, 1..16
    int maxg;             // groups per slice and round held in registers: 1 or 2
};

template <int R, int G, bool Q1>
static void launch_rg(int waves, hipStream_t st, const uint8_t *planes, const int16_t *scales,
                      const int8_t *x, int rows, int groups, int shift, int64_t *y) {
    const unsigned nblk = (unsigned)((rows + R - 1) / R);
    hipLaunchKernelGGL((ternary_rows_kernel<R, G, Q1>), dim3(nblk), dim3(waves * 64), 0, st,
                       planes, scales, x, rows, groups, shift, y);
}

template <int R, bool Q1>
static bool launch_r(int maxg, int waves, hipStream_t st, const uint8_t *planes,
                     const int16_t *scales, const int8_t *x, int rows, int groups, int shift,
                     int64_t *y) {
    switch (maxg) {
    case 1: launch_rg<R, 1, Q1>(waves, st, planes, scales, x, rows, groups, shift, y); return true;
    case 2: launch_rg<R, 2, Q1>(waves, st, planes, scales, x, rows, groups, shift, y); return true;
    default: return false;
    }
}

template <bool Q1>
static int32_t launch_ternary(const TernaryCfg &c, const uint8_t *planes, const int16_t *scales,
                              const int8_t *x, int64_t rows, int64_t k, int32_t frac, int64_t *y,
                              hipStream_t st) {
    if (c.waves < 1 || c.waves > 16) return BS_E_RANGE;
    const int groups = (int)(k / kGroup);
    const int shift = frac > 31 ? 31 : frac;   // |scale*s| < 2^31: shift 31 is floor
    const int n = (int)rows;
    bool ok;
    switch (c.rows_per_block) {
    case 32: ok = launch_r<32, Q1>(c.maxg, c.waves, st, planes, scales, x, n, groups, shift, y); break;
    case 16: ok = launch_r<16, Q1>(c.maxg, c.waves, st, planes, scales, x, n, groups, shift, y); break;
    default: ok = false;
    }
    if (!ok) return BS_E_RANGE;
    BS_LAUNCH_CHECK();
    return BS_OK;
}

// Launch shape of the row-block kernel, which takes K > 16384 (more than the
// pipelined kernel's 128 groups), from sweeps on MI355X with cold weights:
// one group per slice and round (more rounds measured faster than more
// groups in flight per round), 32-row blocks of 16 wavefronts from 5000 rows
// (Q1_0, whose group is half the bytes: two groups per slice and round),
// else 16-row blocks of 16.
static TernaryCfg choose_cfg(int64_t rows, bool q1) {
    TernaryCfg c;
    if (rows >= 5000) {
        c.rows_per_block = 32;
        c.waves = 16;
        c.maxg = q1 ? 2 : 1;
    } else {
        c.rows_per_block = 16;
        c.waves = 16;
        c.maxg = 1;
    }
    return c;
}

// y += W x: the tile mapping, split over runs of cg groups per workgroup.
// Tall matrices with few groups keep one run per tile (cg = K/128);
// otherwise runs of four groups, four
// wavefronts (one group each), when that still gives 150+ workgroups, else
// runs of one group and one wavefront (sweeps on MI355X: 2560x2560 2.70 us,
// 2560x6912 3.48 us, 6912x2560 3.32 us, against 2.96 / 3.85 / 3.55 us for the
// storing kernel).  Runs grow so the grid stays below 2^24 workgroups.
static int32_t launch_acc(const uint8_t *planes, const int16_t *scales, const int8_t *x,
                          int64_t rows, int64_t k, int32_t frac, int64_t *y, hipStream_t st) {
    const int64_t groups = k / kGroup, tiles = pad64(rows) / 64;
    const int shift = frac > 31 ? 31 : frac;
    int64_t cg, waves;
    if (tiles >= 150 && groups <= 48 && (groups <= 24 || tiles >= 200)) {
        cg = groups;
        waves = groups < 16 ? groups : 16;
    } else {
        cg = tiles * ((groups + 3) / 4) >= 150 ? 4 : 1;
        const int64_t min_cg = (tiles * groups + ((int64_t)1 << 24) - 1) >> 24;
        if (cg < min_cg) cg = min_cg;
        waves = cg < 16 ? cg : 16;
    }
    const int64_t nruns = (groups + cg - 1) / cg;
    hipLaunchKernelGGL(ternary_acc_kernel, dim3((unsigned)(tiles * nruns)),
                       dim3((unsigned)waves * 64), 0, st, planes, scales, x, (int)rows,
                       (int)groups, (int)cg, (int)nruns, shift, y);
    BS_LAUNCH_CHECK();
    return BS_OK;
}

}  // namespace
}  // namespace bs

using namespace bs;

static int32_t gemv_check(const uint8_t *planes, const int16_t *scales, const int8_t *x,
                          int64_t rows, int64_t k, int32_t frac, const int64_t *y) {
    if (!planes || !scales || !x || !y) return BS_E_NULL;
    if (int32_t st = check_rows_k(rows, k, (int64_t)1 << 24)) return st;
    if (frac < 0 || frac > 62) return BS_E_RANGE;
    if (((uintptr_t)planes & 15) || ((uintptr_t)scales & 1) || ((uintptr_t)x & 7) ||
        ((uintptr_t)y & 7))
        return BS_E_ALIGN;
    return BS_OK;
}

extern "C" int32_t bs_ternary_gemv(const uint8_t *planes, const int16_t *scales,
                                   const int8_t *x, int64_t rows, int64_t k, int32_t frac,
                                   int64_t *y, void *stream) {
    if (int32_t st = gemv_check(planes, scales, x, rows, k, frac, y)) return st;
    const int64_t groups = k / kGroup;
    if (groups <= kPipeMaxGroups) {
        const int shift = frac > 31 ? 31 : frac;   // |scale*s| < 2^31: shift 31 is floor
        if (!launch_pipe<false>(choose_pipe(rows, groups), (hipStream_t)stream, planes, scales,
                                x, (int)rows, (int)groups, shift, y))
            return BS_E_RANGE;
        BS_LAUNCH_CHECK();
        return BS_OK;
    }
    return launch_ternary<false>(choose_cfg(rows, false), planes, scales, x, rows, k, frac, y,
                                 (hipStream_t)stream);
}

extern "C" int32_t bs_q1_gemv(const uint8_t *bits, const int16_t *scales, const int8_t *x,
                              int64_t rows, int64_t k, int32_t frac, int64_t *y, void *stream) {
    if (int32_t st = gemv_check(bits, scales, x, rows, k, frac, y)) return st;
    const int64_t groups = k / kGroup;
    if (groups <= kPipeMaxGroups) {
        const int shift = frac > 31 ? 31 : frac;
        if (!launch_pipe<true>(choose_pipe_q1(rows, groups), (hipStream_t)stream, bits, scales,
                               x, (int)rows, (int)groups, shift, y))
            return BS_E_RANGE;
        BS_LAUNCH_CHECK();
        return BS_OK;
    }
    return launch_ternary<true>(choose_cfg(rows, true), bits, scales, x, rows, k, frac, y,
                                (hipStream_t)stream);
}

extern "C" int32_t bs_ternary_gemv_acc(const uint8_t *planes, const int16_t *scales,
                                       const int8_t *x, int64_t rows, int64_t k, int32_t frac,
                                       int64_t *y, void *stream) {
    if (int32_t st = gemv_check(planes, scales, x, rows, k, frac, y)) return st;
    return launch_acc(planes, scales, x, rows, k, frac, y, (hipStream_t)stream);
}
