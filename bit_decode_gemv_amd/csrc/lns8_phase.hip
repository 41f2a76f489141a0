// bs_lns8_phase_gemv: the BitState LNS8 eight-phase GEMV on gfx950
// ("BitState / HSDR PoC Technical Brief - v0.5", sections 3, 3.1 and 4).
//
// Weights are ternary bitplanes (the tiled layout of bs_ternary_gemv), the
// activations LNS8 bytes S1|E4|L3.  A ternary weight has log offset 0, so a
// product keeps the activation code and takes the sign S1 XOR [t < 0].  Each
// product adds +-(1 << E4) to one of eight int32 accumulators A[L3]; the row
// result S = 2^-9 * sum_p A[p] * F[p] is materialised once per row.
//
// Three reductions, identical in result:
//   DIRECT   -- per product position, route +-(1 << E4) to A[L3];
//   POPCOUNT -- per state s (a code 1..127: the positions holding it), the
//               signed count C_s of the row's nonzero weights there, added
//               as C_s << band into A[phase]: the histogram H[phase][band]
//               folded into A as it is produced;
//   MATRIX   -- the direct routing as a contraction of the row's signed
//               trits with a 16-column matrix of the activations (one column
//               per phase and band half), on the int8 matrix instructions.
//
// DIRECT mapping: a workgroup owns one 64-row tile (lane j of every
// wavefront = row 64*tile + j, so the activation codes are uniform across a
// wavefront) and a run of 64-position units, one or more per wavefront.  The
// wavefronts' A[8] meet in LDS (integer addition is associative, so the
// order is free).  When K is split over several workgroups per tile (64
// tiles alone would leave most of the GPU idle), each workgroup writes its
// partial A to the workspace with agent-scope stores (coherent across the
// XCDs' L2s: written through, as the compiler implements agent-scope atomic
// stores), waits for them to complete, and counts itself done on the tile's
// counter with an agent-scope atomic add; the workgroup that finds itself
// last reads the partials with agent-scope loads, sums them, writes A and S
// and returns the counter and the partials to zero for the next call.  One
// launch, no spin, and no L2 write-back or invalidate: a release/acquire
// pair on the counter (buffer_wbl2 + buffer_inv) measured 19.5 us per call
// instead of 10-11.
//
// POPCOUNT mapping (lns8_pc_kernel below): a workgroup owns 16 rows and all
// of K, with the state sets built once per workgroup in LDS; no workspace.
// MATRIX mapping (lns8_mx_kernel below): the same 16 rows and all of K, the
// activations staged once per workgroup in LDS; no workspace.
#include "kcommon.h"

namespace bs {
namespace {

// F[p] = 2^((p-2)/8), p = 0..7, correctly rounded to binary64.
__device__ constexpr double kF[8] = {
    0x1.ae89f995ad3adp-1, 0x1.d5818dcfba487p-1, 0x1.0000000000000p+0, 0x1.172b83c7d517bp+0,
    0x1.306fe0a31b715p+0, 0x1.4bfdad5362a27p+0, 0x1.6a09e667f3bcdp+0, 0x1.8ace5422aa0dbp+0};

// S = 2^-9 * sum_p A[p] F[p], evaluated exactly and rounded once: every F[p]
// is an integer multiple of 2^-53 (F[p] < 2), so the sum is the integer
// t = sum_p A[p] * (F[p] * 2^53) (below 2^88) times 2^-62.  With F[p] * 2^53 =
// Fh * 2^27 + Fl (both below 2^27) the two int64 sums h = sum A Fh and l =
// sum A Fl (each below 2^61) give t = h * 2^27 + l exactly; regrouped as
// t = a + b with a = (g >> 26) * 2^53 and b < 2^53, g = h + (l >> 27), both
// are exact doubles, so the one rounded addition a + b is t rounded to nearest
// even.  The power-of-two scaling is exact (|t| >= 1 or t = 0).
__device__ __forceinline__ double materialize(const int A[8]) {
    int64_t h = 0, l = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t f = (int64_t)(kF[p] * 9007199254740992.0);
        h += (int64_t)A[p] * (int)(f >> 27);
        l += (int64_t)A[p] * (int)(f & ((1 << 27) - 1));
    }
    const int64_t g = h + (l >> 27);
    const double a = (double)(g >> 26) * 9007199254740992.0;
    const double b = (double)(((g & ((1 << 26) - 1)) << 27) | (l & ((1 << 27) - 1)));
    return ldexp(a + b, -62);
}

// One unit of work of DIRECT: 64 positions (half h of group g) for the
// wavefront's 64 rows.  Lane j holds row j's W_nonzero / W_negative bits of
// those positions (bit i = position 64h + i) and, for the ballots, the
// activation byte of position 64h + j.
__device__ __forceinline__ void lns8_unit(const uint8_t *__restrict__ planes,
                                          const uint8_t *__restrict__ x, int tile, int groups,
                                          int u, int lane, int A[8]) {
    const int g = u >> 1, h = u & 1;
    const size_t blk = (size_t)tile * groups + g;
    const uint2 nzv = *reinterpret_cast<const uint2 *>(planes + blk * 2048 + 16 * lane + 8 * h);
    const uint2 ngv = *reinterpret_cast<const uint2 *>(planes + blk * 2048 + 1024 + 16 * lane + 8 * h);
    const int b = x[(size_t)g * 128 + 64 * h + lane];
    const int code = b & 0x7F;
    // Every product is routed on its own.  Lane j first turns position
    // j's byte into its signed weight w_j = (-1)^S1 * 2^E4 (0 for code
    // 0); then for each phase p the positions with phase p (a ballot
    // mask) are walked one by one, and position i adds w_i * t_i to A[p]
    // of every row, t_i = nz_i - 2 neg_i the row's trit there (so the
    // product sign is S1 xor [t < 0]).  The walk takes positions 0..31 and
    // 32..63 from the two 32-bit words in turn.
    const int mag = code ? 1 << (code >> 3) : 0;
    const int wv = (b & 0x80) ? -mag : mag;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint64_t m = __ballot(code != 0 && (code & 7) == p);
        int anz = 0, ang = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t nzw = half ? nzv.y : nzv.x, ngw = half ? ngv.y : ngv.x;
            uint32_t mh = (uint32_t)(m >> (32 * half));
            while (mh) {
                const int i = __builtin_ctz(mh);
                mh &= mh - 1;
                const int w = __builtin_amdgcn_readlane(wv, 32 * half + i);
                // bit * w with a 24-bit multiply-add (|w| <= 2^15)
                anz = __mul24((int)__builtin_amdgcn_ubfe(nzw, i, 1), w) + anz;
                ang = __mul24((int)__builtin_amdgcn_ubfe(ngw, i, 1), w) + ang;
            }
        }
        A[p] += anz - 2 * ang;
    }
}

// The end of a (tile, split) workgroup of the split-K mappings.  red[w][p][j]
// holds wavefront w's A[p] of row j of the tile (the first nw wavefronts);
// the wavefronts are summed, the splits of the tile meet through the
// workspace (the last to arrive sums them), and A and S are stored.  Every
// thread of the workgroup calls it.
template <int MAXW>
__device__ __forceinline__ void tile_finish(int (&red)[MAXW][8][64], int &last, int nw, int tile,
                                            int split, int nsplit, int rows,
                                            int32_t *__restrict__ acc_out,
                                            double *__restrict__ s_out,
                                            int *__restrict__ counters,
                                            int *__restrict__ partial) {
    // pair (p, j) sums phase p of row j over the wavefronts; the 512 pairs
    // are shared out over however many threads the workgroup has
    for (int idx = threadIdx.x; idx < 512; idx += blockDim.x) {
        const int p = idx >> 6, j = idx & 63;
        // all the reads in flight at once; wavefronts past nw (whose slots
        // were never written) are masked out
        int t = 0;
#pragma unroll
        for (int w = 0; w < MAXW; ++w) t += red[w][p][j] & -(int)(w < nw);
        red[0][p][j] = t;   // wavefront 0's entry of this pair is read only here
    }
    __syncthreads();
    if (nsplit > 1) {
        // this split's partial, then the tile's counter
        const size_t padded_rows = (size_t)(gridDim.x / nsplit) * 64;
        for (int idx = threadIdx.x; idx < 512; idx += blockDim.x) {
            const int p = idx >> 6, j = idx & 63;
            __hip_atomic_store(partial + ((size_t)split * padded_rows + tile * 64 + j) * 8 + p,
                               red[0][p][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are done
        __syncthreads();
        if (threadIdx.x == 0)
            last = __hip_atomic_fetch_add(counters + tile, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
        __syncthreads();
        if (!last) return;                     // uniform
        // sum the partials and clear them: every call leaves the whole
        // workspace zero, so the counters of a later call with more tiles
        // never land on stale partials
        for (int idx = threadIdx.x; idx < 512; idx += blockDim.x) {
            const int p = idx >> 6, j = idx & 63;
            int *src = partial + ((size_t)tile * 64 + j) * 8 + p;
            const size_t stride = padded_rows * 8;
            int t = 0;
            // every load in flight at once, then the clearing stores (a load
            // and a store to one address in turn would wait for each load)
            for (int sp = 0; sp < nsplit; ++sp)
                t += __hip_atomic_load(src + sp * stride, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            for (int sp = 0; sp < nsplit; ++sp) src[sp * stride] = 0;
            red[0][p][j] = t;   // only this thread reads or writes pair (p, j) here
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
    }
    if (threadIdx.x < 64) {
        const int row = tile * 64 + threadIdx.x;
        if (row < rows) {
            int T[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) T[p] = red[0][p][threadIdx.x];
            int4 *dst = reinterpret_cast<int4 *>(acc_out + (size_t)row * 8);
            dst[0] = make_int4(T[0], T[1], T[2], T[3]);
            dst[1] = make_int4(T[4], T[5], T[6], T[7]);
            if (s_out) s_out[row] = materialize(T);
        }
    }
}

// One workgroup per (64-row tile, split): wavefront w takes the units (64
// positions each, two per group) [(split * W + w) * upw, ... + upw).
__global__ __launch_bounds__(1024) void lns8_kernel(
    const uint8_t *__restrict__ planes, const uint8_t *__restrict__ x, int rows, int groups,
    int upw, int nsplit, int32_t *__restrict__ acc_out, double *__restrict__ s_out,
    int *__restrict__ counters, int *__restrict__ partial) {
    __shared__ int red[16][8][64];
    __shared__ int last;
    const int tile = blockIdx.x / nsplit;
    const int split = blockIdx.x - tile * nsplit;
    const int nw = blockDim.x >> 6;
    // uniform: the activation bytes of DIRECT then come through scalar loads
    // and the phase routing is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int u0 = (split * nw + wave) * upw;
    const int u1 = min(2 * groups, u0 + upw);

    int A[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int u = u0; u < u1; ++u) lns8_unit(planes, x, tile, groups, u, lane, A);
#pragma unroll
    for (int p = 0; p < 8; ++p) red[wave][p][lane] = A[p];
    __syncthreads();
    tile_finish<16>(red, last, nw, tile, split, nsplit, rows, acc_out, s_out, counters, partial);
}

// POPCOUNT without a split of K.  A workgroup owns 16 rows and all of K: in
// wavefront w, quarter q (lanes 16q..16q+15, lane = row 16 * block + (lane &
// 15)) takes unit 4w + q of every chunk of 4 * NW units.  The state sets
// depend on the activations alone, so per chunk the workgroup builds them
// once in LDS: for every code 1..127 and unit of the chunk the 64-bit mask of
// the unit's positions holding that code (code 0 is an exact zero and has no
// state), and every unit's S1 mask.  A wavefront then walks, phase by phase,
// the codes present in any of its four units; each lane reads its own
// unit's mask of the code and adds C_s << band to A[phase].  With pneg =
// nz & (S1 ^ neg), the positions whose product sign is negative, the product
// signs are t' = nz - 2 pneg, and over any position mask M
//   sum_{i in M} t'_i = popcount(nz & (M ^ pneg)) - popcount(pneg)
// (per position t' m = nz (m ^ pneg) - pneg, the ternary GEMV's identity), so
// a state costs one bitop3 and one count per 32 positions; a phase's
// -popcount(pneg) terms add up to -popcount(pneg) * sum_s 2^band(s), and a
// state the lane's unit lacks (M = 0) adds popcount(pneg) - popcount(pneg)
// = 0.  The quarters meet by lane swaps, the wavefronts in LDS, and one lane
// per row stores A and S: no workspace, no second round trip through memory.
//
// The mask table's rows are the states in phase-major order (row 16 * phase
// + band for code 8 * band + phase), each holding the chunk's units plus one
// padding slot: the presence step, where lane i reads row i, then spreads
// its lanes over the LDS banks (rows of a whole number of bank widths would
// put all 64 lanes on the same four banks).
constexpr int kPcRows = 16;                 // rows per workgroup
constexpr int kPcMaxUnits = 64;             // units per chunk at 16 wavefronts
constexpr int kPcTabSlots = 128 * (kPcMaxUnits + 1);   // 64-bit slots

__device__ __forceinline__ int add_quarters(int v) {
    // the gfx950 lane swaps return v and the value of the partner lane
    // (32 lanes apart, then 16), whose sum is wanted
    const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    v = (int)a[0] + (int)a[1];
    const auto b = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    return (int)b[0] + (int)b[1];
}

__global__ __launch_bounds__(1024) void lns8_pc_kernel(
    const uint8_t *__restrict__ planes, const uint8_t *__restrict__ x, int rows, int groups,
    int32_t *__restrict__ acc_out, double *__restrict__ s_out) {
    // tab[(row * (cu + 1) + unit) * 2 + half]: the mask of the unit's
    // positions 32 * half .. 32 * half + 31 holding the code of state row
    __shared__ __align__(16) uint32_t tab[kPcTabSlots * 2];
    __shared__ uint32_t sgn[kPcMaxUnits * 2];
    __shared__ int red[8][kPcRows];          // A[p] of the 16 rows, summed with ds_add
    const int nw = blockDim.x >> 6;
    const int cu = 4 * nw;                   // units per chunk
    const int rs = cu + 1;                   // table row stride, 64-bit slots
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ul = 4 * wave + (lane >> 4);   // this lane's unit within a chunk
    const int row = blockIdx.x * kPcRows + (lane & 15);   // < the padded row count
    const int tile = row >> 6, rit = row & 63;
    const int units = 2 * groups;
    const int k = groups * 128;

    for (int i = threadIdx.x; i < 8 * kPcRows; i += blockDim.x) (&red[0][0])[i] = 0;   // before the first barrier
    int A[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c0 = 0; c0 < units; c0 += cu) {
        // this lane's weights and this thread's four activation bytes (the
        // fill's: positions 4t .. 4t+3 of the chunk, unit t / 16), in flight
        // while the table is cleared
        const int u = c0 + ul;
        uint2 nzv = make_uint2(0, 0), ngv = make_uint2(0, 0);
        if (u < units) {
            const size_t off = ((size_t)tile * groups + (u >> 1)) * 2048 + 16 * rit + 8 * (u & 1);
            nzv = *reinterpret_cast<const uint2 *>(planes + off);
            ngv = *reinterpret_cast<const uint2 *>(planes + off + 1024);
        }
        const int pos = c0 * 64 + 4 * (int)threadIdx.x;
        const uint32_t v = pos < k ? *reinterpret_cast<const uint32_t *>(x + pos) : 0u;
        if (c0) __syncthreads();             // the previous chunk's reads are done
        // clear the chunk's table (128 rows of cu + 1 slots: 256 * nw + 64
        // 16-byte stores) and masks
        uint4 *t4 = reinterpret_cast<uint4 *>(tab);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int j = threadIdx.x + i * blockDim.x;
            if (j < 64 * rs) t4[j] = make_uint4(0, 0, 0, 0);
        }
        if ((int)threadIdx.x < 2 * cu) sgn[threadIdx.x] = 0;
        __syncthreads();
        // thread t: positions 4t .. 4t+3 of the chunk (unit t / 16); bytes
        // past K read as 0 (code 0, no state)
        {
            const int t = threadIdx.x;
            const int ut = t >> 4, bit = 4 * (t & 15);   // bit of the unit's first position
            const int half = bit >> 5, sh = bit & 31;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int code = (v >> (8 * i)) & 0x7F;
                const int sr = 16 * (code & 7) + (code >> 3);   // state row
                if (code) atomicOr(&tab[(sr * rs + ut) * 2 + half], 1u << (sh + i));
            }
            const uint32_t sb = ((v >> 7) & 1) | ((v >> 14) & 2) | ((v >> 21) & 4) | ((v >> 28) & 8);
            if (sb) atomicOr(&sgn[ut * 2 + half], sb << sh);
        }
        __syncthreads();
        // the states present in the wavefront's four units, phase-major: bit
        // 16 (p & 3) + band of pres[p >> 2]; lane i looks at row i (then
        // 64 + i)
        const uint2 *tab2 = reinterpret_cast<const uint2 *>(tab);
        uint64_t pres[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint2 *r = tab2 + (64 * hh + lane) * rs + 4 * wave;
            const uint2 a = r[0], b = r[1], c = r[2], d = r[3];
            pres[hh] = __ballot((a.x | a.y | b.x | b.y | c.x | c.y | d.x | d.y) != 0);
        }
        const uint32_t sg0 = sgn[ul * 2], sg1 = sgn[ul * 2 + 1];
        // pneg; kept opaque to the compiler, which would otherwise fold the
        // nz & into nz & (M ^ S1 ^ neg) and spend an xor and an and per word
        // instead of one bitop3
        uint32_t pn0 = nzv.x & (sg0 ^ ngv.x), pn1 = nzv.y & (sg1 ^ ngv.y);
        asm volatile("" : "+v"(pn0));
        asm volatile("" : "+v"(pn1));
        const int npn = bcnt_add(pn1, bcnt_add(pn0, 0));
        // the state loop is bound by instruction issue (one scalar and one
        // vector instruction per cycle per CU): the row stride multiplies on
        // the vector unit (a per-lane copy of it), the scalar unit keeps only
        // the band search, the bit clear and the loop test
        const uint8_t *mrow = reinterpret_cast<const uint8_t *>(tab2 + ul);
        int rs8v = rs * 8;
        asm volatile("" : "+v"(rs8v));
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint32_t bm = (uint32_t)(pres[p >> 2] >> (16 * (p & 3))) & 0xFFFFu;   // uniform
            // sum over the phase's states of 2^band: the band mask itself
            const int wsum = (int)bm;
            const uint8_t *pb = mrow + 16 * p * rs * 8;
            int sum = 0;
            while (bm) {
                const int band = __builtin_ctz(bm);
                asm("s_bitset0_b32 %0, %1" : "+s"(bm) : "s"(band));
                const uint2 m = *reinterpret_cast<const uint2 *>(pb + __mul24(band, rs8v));
                // two counts chained through the count-and-add instruction
                const int c = __builtin_popcount(nzv.y & (m.y ^ pn1)) +
                              __builtin_popcount(nzv.x & (m.x ^ pn0));
                sum += c << band;
            }
            // |sum|, npn * wsum <= 64 * 2^16
            A[p] += sum - __mul24(npn, wsum);
        }
    }
    // the quarters by lane swaps, the wavefronts by LDS atomic adds
    // (integer addition: the order is free)
#pragma unroll
    for (int p = 0; p < 8; ++p) A[p] = add_quarters(A[p]);
    if (lane < kPcRows) {
#pragma unroll
        for (int p = 0; p < 8; ++p) atomicAdd(&red[p][lane], A[p]);
    }
    __syncthreads();
    if ((int)threadIdx.x < kPcRows) {
        const int rr = blockIdx.x * kPcRows + threadIdx.x;
        if (rr < rows) {
            int T[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) T[p] = red[p][threadIdx.x];
            int4 *dst = reinterpret_cast<int4 *>(acc_out + (size_t)rr * 8);
            dst[0] = make_int4(T[0], T[1], T[2], T[3]);
            dst[1] = make_int4(T[4], T[5], T[6], T[7]);
            if (s_out) s_out[rr] = materialize(T);
        }
    }
}

// MATRIX: the direct routing written as a contraction.  Over the columns
// (p, h) of a 16-column matrix X, X[k][(p, h)] = 2^(E4 & 7) when position k
// has phase p, E4 >> 3 = h and a nonzero code, else 0, and
//   A[p] = sum_k t'_k X[k][(p, 0)] + 256 * sum_k t'_k X[k][(p, 1)]
// with t' = nz - 2 pneg the signed trits (pneg = nz & (S1 ^ neg), as in
// POPCOUNT): each product lands in exactly one column, its phase's, scaled
// by the band's low three bits.  The contraction runs on the int8 matrix
// instruction of 16 rows x 16 columns x 64 positions.  X's entries reach
// 128, one past int8, so the matrix holds X - 1 (0..127 where the code
// matches the column, -1 elsewhere) and the row's trit sum U = sum_k t'_k,
// subtracted from every column, is added back: A[p] = C[(p, 0)] + 256 *
// C[(p, 1)] + 257 * U.
//
// Mapping: like POPCOUNT, one workgroup per 16 rows (one slice of a tile)
// and all of K, so no workspace and no second pass; its wavefronts take
// whole groups of 128 positions in turn and meet in LDS.  Lane l of a
// wavefront holds, for its lane group q = l / 16, positions 32q .. 32q+31 of
// the group: as A operand the trits of row l % 16, as B operand the entries
// of column l % 16 (the instruction pairs A's and B's bytes by lane group
// and byte, so any assignment of positions to them serves if both use it;
// here byte b of step h is position 32q + 16h + b).
//
// The activations are staged once per workgroup in LDS, a chunk of up to 64
// groups at a time: per position the byte (E4 & 7) | phase << 4 | (E4 >> 3)
// << 7, and per 64 positions the S1 mask.  A column's byte is then one
// permute of a table of 2^j - 1 indexed by that byte XOR the column's key
// (phase << 4 | half << 7): the index is E4 & 7 when phase and band half
// match and 16 or more (byte 0xFF) when they differ.  Code 0 (phase 0, band
// 0) matches column (0, 0) at index 0, where that column's table holds -1:
// no product.  The sixteen trits of a step come from the row's nz and pneg
// bits one nibble at a time: a 24-bit multiply by 0x204081 (0x408102) copies
// a nibble's bits to the low (second) bit of four bytes without overlap, and
// a byte permute maps the 2-bit pattern nz + 2 pneg to 0, 1 or 0xFF.

// int8 trits n_i - 2 m_i of bits sh .. sh+3 (m a subset of n), byte i = bit sh + i
__device__ __forceinline__ int trits4(uint32_t n, uint32_t m, int sh) {
    const uint32_t a = (__builtin_amdgcn_ubfe(n, sh, 4) * 0x204081u) & 0x01010101u;
    const uint32_t sel = ((__builtin_amdgcn_ubfe(m, sh, 4) * 0x408102u) & 0x02020202u) | a;
    return (int)__builtin_amdgcn_perm(0u, 0xFF000100u, sel);
}

// column bytes of four staged positions: table[E4 & 7] where the phase and
// band half match the column's key, else 0xFF
__device__ __forceinline__ int xcol4(uint32_t v, uint32_t key, uint32_t tlo, uint32_t thi) {
    return (int)__builtin_amdgcn_perm(thi, tlo, v ^ key);
}

// staged byte of four LNS8 codes: E4 & 7 in bits 0-2, the phase in bits 4-6,
// E4 >> 3 in bit 7 (S1 is dropped; it is staged as a mask)
__device__ __forceinline__ uint32_t mx_stage4(uint32_t w) {
    return ((w >> 3) & 0x07070707u) | ((w & 0x07070707u) << 4) | ((w << 1) & 0x80808080u);
}

typedef int mx_v4i __attribute__((ext_vector_type(4)));

constexpr int kMxRows = 16;    // rows per workgroup
constexpr int kMxChunk = 64;   // groups staged in LDS at a time (a multiple of every
                               // wavefront count the launch uses when groups >= 16)

__global__ __launch_bounds__(1024) void lns8_mx_kernel(
    const uint8_t *__restrict__ planes, const uint8_t *__restrict__ x, int rows, int groups,
    int32_t *__restrict__ acc_out, double *__restrict__ s_out) {
    __shared__ uint4 xv[kMxChunk * 8];        // staged bytes, 128 per group
    __shared__ uint64_t xs[kMxChunk * 2];     // S1 masks, 64 positions each
    __shared__ int red[8][kMxRows];           // A[p] of the 16 rows, summed with ds_add
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, q = lane >> 4;
    const int row = blockIdx.x * kMxRows + c;   // < the padded row count
    const int tile = row >> 6, rit = row & 63;
    // column (c & 7, c >> 3) of X - 1: key phase << 4 | half << 7; table[j] =
    // 2^j - 1, column (0, 0)'s entry 0 (code 0 only) -1
    const uint32_t key = (uint32_t)(((c & 7) << 4) | ((c >> 3) << 7)) * 0x01010101u;
    const uint32_t tlo = c == 0 ? 0x070301FFu : 0x07030100u, thi = 0x7F3F1F0Fu;

    for (int i = threadIdx.x; i < 8 * kMxRows; i += blockDim.x) (&red[0][0])[i] = 0;
    mx_v4i acc = {0, 0, 0, 0};
    int un = 0, ug = 0;
    // the lane's row's nz and neg words of a group (positions 32q .. 32q+31)
    const uint8_t *pt = planes + (size_t)tile * groups * 2048 + 16 * rit + 4 * q;
    auto load = [&](int g, uint32_t &n, uint32_t &ng) {
        n = *reinterpret_cast<const uint32_t *>(pt + (size_t)g * 2048);
        ng = *reinterpret_cast<const uint32_t *>(pt + (size_t)g * 2048 + 1024);
    };
    // one group of the staged chunk (index gl)
    auto work = [&](int gl, uint32_t n, uint32_t ng) {
        const uint32_t sg = reinterpret_cast<const uint32_t *>(xs)[4 * gl + q];
        const uint4 w0 = xv[8 * gl + 2 * q], w1 = xv[8 * gl + 2 * q + 1];
        const uint32_t m = n & (ng ^ sg);
        un = bcnt_add(n, un);
        ug = bcnt_add(m, ug);
        const mx_v4i xb0 = {xcol4(w0.x, key, tlo, thi), xcol4(w0.y, key, tlo, thi),
                            xcol4(w0.z, key, tlo, thi), xcol4(w0.w, key, tlo, thi)};
        const mx_v4i a0 = {trits4(n, m, 0), trits4(n, m, 4), trits4(n, m, 8),
                           trits4(n, m, 12)};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, xb0, acc, 0, 0, 0);
        const mx_v4i xb1 = {xcol4(w1.x, key, tlo, thi), xcol4(w1.y, key, tlo, thi),
                            xcol4(w1.z, key, tlo, thi), xcol4(w1.w, key, tlo, thi)};
        const mx_v4i a1 = {trits4(n, m, 16), trits4(n, m, 20), trits4(n, m, 24),
                           trits4(n, m, 28)};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, xb1, acc, 0, 0, 0);
    };
    // the wavefront's groups are wave, wave + nw, ...; two register sets
    // alternate so the next group's words load while one is computed (nw <=
    // groups, so the first exists)
    // The activations of a chunk: every byte is loaded before any is used (one
    // round trip); a chunk holds at most 8 positions per thread (blockDim is
    // 64 per group below 16 groups, else 1024, and a chunk 128 positions per
    // group, at most 64 groups).  The bounds are wavefront-uniform: i - lane
    // is a multiple of 64, and so is a chunk's position count.
    uint32_t xb[8];
    auto stage_load = [&](int c0, int npos) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = threadIdx.x + j * blockDim.x;
            xb[j] = i < npos ? x[(size_t)c0 * 128 + i] : 0u;
        }
    };
    auto stage_store = [&](int npos) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = threadIdx.x + j * blockDim.x;
            if (i < npos) {
                reinterpret_cast<uint8_t *>(xv)[i] = (uint8_t)mx_stage4(xb[j]);
                const uint64_t s1 = __ballot(xb[j] & 0x80);
                if (lane == 0) xs[i >> 6] = s1;
            }
        }
    };
    // the wavefront's groups are wave, wave + nw, ...; two register sets
    // alternate so the next group's words load while one is computed (nw <=
    // groups, so the first exists).  The first group's words are requested
    // after the first chunk's bytes, so staging waits on those bytes alone.
    uint32_t na, nga, nb = 0, ngb = 0;
    int cend = kMxChunk < groups ? kMxChunk : groups;
    stage_load(0, cend * 128);
    load(wave, na, nga);
    stage_store(cend * 128);
    __syncthreads();
    for (int c0 = 0; c0 < groups; c0 += kMxChunk) {
        cend = c0 + kMxChunk < groups ? c0 + kMxChunk : groups;
        if (c0) {
            __syncthreads();   // every wavefront is done with the last chunk
            stage_load(c0, (cend - c0) * 128);
            stage_store((cend - c0) * 128);
            __syncthreads();
        }
        // the wavefront's first group of the chunk: c0 is a multiple of nw
        // whenever there is more than one chunk (nw = 16), and the words of
        // that group are in na, nga
        for (int g = c0 + wave; g < cend; g += 2 * nw) {
            if (g + nw < groups) load(g + nw, nb, ngb);
            work(g - c0, na, nga);
            if (g + nw >= cend) {
                na = nb;
                nga = ngb;
                break;
            }
            if (g + 2 * nw < groups) load(g + 2 * nw, na, nga);
            work(g + nw - c0, nb, ngb);
        }
    }
    // lane (c, q) holds C[row 4q + v][column c]; lanes c < 8 combine columns
    // (c, 0) and (c, 1) (lane c + 8, a DPP rotate by 8 within the 16-lane row)
    // with the row's U (lane 4q + v once the lane groups' counts are summed),
    // and the wavefronts meet by LDS atomic adds (integer addition: the order
    // is free)
    const int u = add_quarters(un - 2 * ug);
    __syncthreads();   // red is zero
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int hi = __builtin_amdgcn_mov_dpp(acc[v], 0x128, 0xF, 0xF, false);
        const int ur = __shfl(u, 4 * q + v);
        // modulo 2^32 (the sum, A[p], fits int32; its terms need not)
        if (c < 8)
            atomicAdd(&red[c][4 * q + v],
                      (int)((uint32_t)acc[v] + 256u * (uint32_t)hi + 257u * (uint32_t)ur));
    }
    __syncthreads();
    if ((int)threadIdx.x < kMxRows) {
        const int rr = blockIdx.x * kMxRows + threadIdx.x;
        if (rr < rows) {
            int T[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) T[p] = red[p][threadIdx.x];
            int4 *dst = reinterpret_cast<int4 *>(acc_out + (size_t)rr * 8);
            dst[0] = make_int4(T[0], T[1], T[2], T[3]);
            dst[1] = make_int4(T[4], T[5], T[6], T[7]);
            if (s_out) s_out[rr] = materialize(T);
        }
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

// |A[p]| <= k * 2^15 must fit int32: k <= 65535, the largest multiple of 128
// below that is 65408.
static constexpr int64_t kLns8MaxK = 65408;

// Launch shape: about 4096 wavefronts in all (four per SIMD, to hide the
// scalar/vector dependency chains of the per-product loop), up to 16 per
// workgroup, each with at least one 64-position unit; K is split over
// workgroups only when one workgroup per tile cannot hold them.

struct Lns8Plan {
    int64_t tiles, groups;
    int waves, upw, nsplit;
};

static Lns8Plan lns8_plan(int64_t rows, int64_t k) {
    Lns8Plan pl;
    pl.tiles = pad64(rows) / 64;
    pl.groups = k / kGroup;
    const int64_t units = 2 * pl.groups;
    int64_t want = (4096 + pl.tiles - 1) / pl.tiles;   // wavefronts per tile
    if (want < 1) want = 1;
    if (want > units) want = units;
    pl.waves = (int)(want < 16 ? want : 16);
    int64_t nsplit = (want + pl.waves - 1) / pl.waves;
    pl.upw = (int)((units + pl.waves * nsplit - 1) / (pl.waves * nsplit));
    pl.nsplit = (int)((units + (int64_t)pl.waves * pl.upw - 1) / ((int64_t)pl.waves * pl.upw));
    return pl;
}

// Workspace, when K is split: one int32 counter per tile (256-byte
// aligned), then the partial accumulators int32[nsplit][R][8].  It must be
// zero before the first call, and every call leaves it zero (the last
// workgroup of a tile clears the tile's counter and partials).
struct Lns8Ws {
    size_t counters, partial, total;
};

static Lns8Ws lns8_ws(int64_t rows, int64_t k) {
    const Lns8Plan pl = lns8_plan(rows, k);
    Lns8Ws w;
    w.counters = 0;
    w.partial = pl.nsplit > 1 ? align_up((size_t)pl.tiles * 4, kWsAlign) : 0;
    w.total = pl.nsplit > 1 ? w.partial + (size_t)pl.nsplit * (size_t)pad64(rows) * 8 * 4
                            : kWsAlign;
    w.total = align_up(w.total, kWsAlign);
    return w;
}

static size_t lns8_ws_bytes(int64_t rows, int64_t k) { return lns8_ws(rows, k).total; }

extern "C" size_t bs_lns8_workspace_bytes(int64_t rows, int64_t k) {
    if (check_rows_k(rows, k, kLns8MaxK) != BS_OK) return 0;
    return lns8_ws_bytes(rows, k);
}

extern "C" int32_t bs_lns8_phase_gemv(const uint8_t *planes, const uint8_t *x_lns8,
                                      int64_t rows, int64_t k, int32_t path, int32_t *acc,
                                      double *s, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    if (!planes || !x_lns8 || !acc) return BS_E_NULL;
    if (int32_t st = check_rows_k(rows, k, kLns8MaxK)) return st;
    if (path != BS_LNS8_DIRECT && path != BS_LNS8_POPCOUNT && path != BS_LNS8_MATRIX)
        return BS_E_RANGE;
    if (((uintptr_t)planes & 15) || ((uintptr_t)x_lns8 & 3) || ((uintptr_t)acc & 3) ||
        ((uintptr_t)s & 7))
        return BS_E_ALIGN;
    if (!ws_ok(workspace, workspace_bytes, lns8_ws_bytes(rows, k))) return BS_E_WORKSPACE;

    hipStream_t st = (hipStream_t)stream;
    if (path == BS_LNS8_MATRIX) {
        // 16 rows and all of K per workgroup, up to 16 wavefronts taking
        // whole groups; the workspace is not touched
        const int64_t groups = k / kGroup;
        const int64_t nw = groups < 16 ? groups : 16;
        const int64_t blocks = (rows + kMxRows - 1) / kMxRows;
        hipLaunchKernelGGL(lns8_mx_kernel, dim3((unsigned)blocks), dim3((unsigned)(nw * 64)), 0,
                           st, planes, x_lns8, (int)rows, (int)groups, acc, s);
        BS_LAUNCH_CHECK();
        return BS_OK;
    }
    if (path == BS_LNS8_POPCOUNT) {
        // 16 rows and all of K per workgroup; the workspace is not touched
        const int64_t units = 2 * (k / kGroup);
        const int64_t nw = units >= 64 ? 16 : (units + 3) / 4;
        const int64_t blocks = (rows + kPcRows - 1) / kPcRows;
        hipLaunchKernelGGL(lns8_pc_kernel, dim3((unsigned)blocks), dim3((unsigned)(nw * 64)), 0,
                           st, planes, x_lns8, (int)rows, (int)(k / kGroup), acc, s);
        BS_LAUNCH_CHECK();
        return BS_OK;
    }
    const Lns8Plan pl = lns8_plan(rows, k);
    const Lns8Ws w = lns8_ws(rows, k);
    unsigned char *base = static_cast<unsigned char *>(workspace);
    int *counters = reinterpret_cast<int *>(base + w.counters);
    int *partial = reinterpret_cast<int *>(base + w.partial);
    hipLaunchKernelGGL(lns8_kernel, dim3((unsigned)(pl.tiles * pl.nsplit)), dim3(pl.waves * 64), 0, st,
                       planes, x_lns8, (int)rows, (int)pl.groups, pl.upw, pl.nsplit, acc, s,
                       counters, partial);
    BS_LAUNCH_CHECK();
    return BS_OK;
}
