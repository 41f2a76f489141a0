// bs_flns_phase_gemv: the pure fractional-LNS reduction of the BitState
// brief on gfx950 ("BitState / HSDR PoC Technical Brief - v0.5", section
// 5.2: count-to-log folding, kappa+/kappa- pair adds with exact
// cancellation, balanced trees, the log-domain scale).
//
// Values.  In registers a log-domain value is one int32, e = 2*L + s (s = 1
// for a negative value), and INT32_MIN stands for zero.  The pair add sorts
// by L, looks up one correction (same-sign table, or opposite-sign table
// behind it) and adds it to L; the sign bit rides along.  L stays far inside
// +-2^29: at most 2^f (127 + 8 log2 K + 8 log2 d) above, and each of at most
// 16 tree levels can lower it by |km[1]| < 2^(f+4) below.
//
// Mapping.  Kernel A: a workgroup of eight wavefronts per (64-row tile, run
// of eight Tile128s); lane j of every wavefront is row 64*tile + j, so the
// activation bytes of a Tile128 are uniform across the wavefront.  Per code
// c the two 64-position halves are selected by ballots (scalar masks); the
// signed population of each row is popcount(mask & positive products) -
// popcount(mask & negative products).  A code absent from the tile is dead
// for the whole wavefront, and so is every tree node whose leaves are all
// dead: those adds are skipped by scalar branches.  The sixteen bands of a
// phase reduce in registers; the eight Tile128s of the workgroup meet in
// LDS.  With more than eight Tile128s, each workgroup writes its eight phase
// partials per row to the workspace and kernel B (lanes = workgroups of one
// row, shuffles) finishes the tile tree, then the phase tree and the scale.
// The kernel boundary makes the partials visible across XCDs.
//
// Tables.  For frac_bits <= 8 the corrections are int16 and staged in LDS
// (at most 102,640 bytes); above, they are read from the device blob.
#include <limits.h>

#include <type_traits>

#include "flns_layout.h"
#include "kcommon.h"

namespace bs {
namespace {

constexpr int kZ = INT_MIN;   // encoded zero
constexpr int kTilesPerWg = 8;

// The pair add of two encoded values (zero = identity).  Symmetric in a, b.
template <typename E>
__device__ __forceinline__ int lns_add(int a, int b, const E *__restrict__ lut, int nkp,
                                       int nkm) {
    const int la = a >> 1, lb = b >> 1;
    const bool a_hi = la >= lb;
    const int hi = a_hi ? a : b;
    const int d = a_hi ? la - lb : lb - la;
    const bool same = ((a ^ b) & 1) == 0;
    const bool in = same ? d < nkp : d < nkm;
    const int corr = in ? (int)lut[same ? d : nkp + d] : 0;
    int out = hi + 2 * corr;
    out = (!same && d == 0) ? kZ : out;
    out = a == kZ ? b : out;
    out = b == kZ ? a : out;
    return out;
}

// A tree node: its per-lane value and whether any leaf below it is live
// (uniform across the wavefront).
struct Node {
    int e;
    bool live;
};

template <typename E>
__device__ __forceinline__ Node join(Node a, Node b, const E *__restrict__ lut, int nkp,
                                     int nkm) {
    if (!b.live) return a;
    if (!a.live) return b;
    return Node{lns_add(a.e, b.e, lut, nkp, nkm), true};
}

// Per-lane state of one Tile128: the two activation codes each lane holds
// (positions lane and 64 + lane) and the row's positive / negative product
// masks of the two halves.
struct TileState {
    int code0, code1;
    uint64_t pos0, neg0, pos1, neg1;
};

// Leaf of code c: the folded signed population, or dead when no position
// of the tile has code c.
__device__ __forceinline__ Node leaf(int c, int f, const TileState &ts,
                                     const int32_t *__restrict__ fold) {
    const uint64_t m0 = __ballot(ts.code0 == c);
    const uint64_t m1 = __ballot(ts.code1 == c);
    if ((m0 | m1) == 0) return Node{kZ, false};
    const int cnt = __popcll(m0 & ts.pos0) - __popcll(m0 & ts.neg0) + __popcll(m1 & ts.pos1) -
                    __popcll(m1 & ts.neg1);
    const int n = cnt < 0 ? -cnt : cnt;
    const int e = cnt == 0 ? kZ : 2 * ((c << f) + fold[n]) + (cnt < 0 ? 1 : 0);
    return Node{e, true};
}

// Final encoding: scale, then (sign, L).
__device__ __forceinline__ int2 finish(int e, int ld) {
    if (e == kZ) return make_int2(0, 0);
    e += 2 * ld;
    return make_int2((e & 1) ? -1 : 1, e >> 1);
}

// The 8 -> 4 -> 2 -> 1 tree over the phase results.
template <typename E>
__device__ __forceinline__ int phase_tree(const int v[8], const E *__restrict__ lut, int nkp,
                                          int nkm) {
    const int a = lns_add(lns_add(v[0], v[1], lut, nkp, nkm), lns_add(v[2], v[3], lut, nkp, nkm),
                          lut, nkp, nkm);
    const int b = lns_add(lns_add(v[4], v[5], lut, nkp, nkm), lns_add(v[6], v[7], lut, nkp, nkm),
                          lut, nkp, nkm);
    return lns_add(a, b, lut, nkp, nkm);
}

template <bool SMALL>
using LutT = typename std::conditional<SMALL, int16_t, int32_t>::type;

template <bool SMALL>
__global__ __launch_bounds__(512) void flns_tile_kernel(
    const uint8_t *__restrict__ planes, const uint8_t *__restrict__ x, int rows, int groups,
    int f, const uint8_t *__restrict__ table, int nkp, int nkm, int ld, int nsplit,
    int32_t *__restrict__ out, int *__restrict__ partial) {
    using E = LutT<SMALL>;
    __shared__ int32_t s_fold[kFlnsFoldSlots];
    __shared__ uint4 s_lut4[SMALL ? (kFlnsSmallMaxEntries * 2 + 15) / 16 : 1];
    __shared__ int s_x[kTilesPerWg][8][64];

    const int rtile = blockIdx.x / nsplit;
    const int q = blockIdx.x - rtile * nsplit;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;

    const int32_t *g_fold = reinterpret_cast<const int32_t *>(table + kFlnsHdrBytes);
    for (int i = threadIdx.x; i < kFlnsFoldSlots; i += blockDim.x) s_fold[i] = g_fold[i];
    if constexpr (SMALL) {
        const uint4 *src = reinterpret_cast<const uint4 *>(table + kFlnsCorrOff);
        const int n16 = ((nkp + nkm) * 2 + 15) / 16;
        for (int i = threadIdx.x; i < n16; i += blockDim.x) s_lut4[i] = src[i];
    }
    __syncthreads();
    const E *lut = SMALL ? reinterpret_cast<const E *>(s_lut4)
                         : reinterpret_cast<const E *>(table + kFlnsCorrOff);

    const int j = q * kTilesPerWg + wave;   // Tile128 = 128-weight group j
    if (j < groups) {
        const size_t blk = (size_t)rtile * groups + j;
        const uint4 nz = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 16 * lane);
        const uint4 ng = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 1024 + 16 * lane);
        const int b0 = x[(size_t)j * 128 + lane];
        const int b1 = x[(size_t)j * 128 + 64 + lane];
        const uint64_t s0 = __ballot(b0 >> 7), s1 = __ballot(b1 >> 7);
        const uint64_t nz0 = (uint64_t)nz.x | ((uint64_t)nz.y << 32);
        const uint64_t nz1 = (uint64_t)nz.z | ((uint64_t)nz.w << 32);
        const uint64_t ng0 = (uint64_t)ng.x | ((uint64_t)ng.y << 32);
        const uint64_t ng1 = (uint64_t)ng.z | ((uint64_t)ng.w << 32);
        TileState ts;
        ts.code0 = b0 & 0x7F;
        ts.code1 = b1 & 0x7F;
        // a product is negative iff S1 xor [t < 0]
        ts.neg0 = nz0 & (s0 ^ ng0);
        ts.pos0 = nz0 & ~(s0 ^ ng0);
        ts.neg1 = nz1 & (s1 ^ ng1);
        ts.pos1 = nz1 & ~(s1 ^ ng1);
#pragma unroll 1
        for (int p = 0; p < 8; ++p) {
            Node v[16];
            v[0] = p == 0 ? Node{kZ, false} : leaf(p, f, ts, s_fold);   // code 0 is zero
#pragma unroll
            for (int b = 1; b < 16; ++b) v[b] = leaf(8 * b + p, f, ts, s_fold);
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int m = 0; m < w; ++m) v[m] = join(v[2 * m], v[2 * m + 1], lut, nkp, nkm);
            s_x[wave][p][lane] = v[0].live ? v[0].e : kZ;
        }
    } else {
#pragma unroll
        for (int p = 0; p < 8; ++p) s_x[wave][p][lane] = kZ;
    }
    __syncthreads();

    // The workgroup's eight Tile128s per (phase, row): thread t takes phase
    // t / 64 of row t % 64.
    const int p = threadIdx.x >> 6;
    int v[kTilesPerWg];
#pragma unroll
    for (int w = 0; w < kTilesPerWg; ++w) v[w] = s_x[w][p][lane];
    const int r = lns_add(
        lns_add(lns_add(v[0], v[1], lut, nkp, nkm), lns_add(v[2], v[3], lut, nkp, nkm), lut, nkp,
                nkm),
        lns_add(lns_add(v[4], v[5], lut, nkp, nkm), lns_add(v[6], v[7], lut, nkp, nkm), lut, nkp,
                nkm),
        lut, nkp, nkm);
    const int row = rtile * 64 + lane;
    if (nsplit == 1) {
        __syncthreads();
        s_x[0][p][lane] = r;
        __syncthreads();
        if (threadIdx.x < 64 && row < rows) {
            int ph[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) ph[k] = s_x[0][k][lane];
            *reinterpret_cast<int2 *>(out + 2 * (size_t)row) = finish(phase_tree(ph, lut, nkp, nkm), ld);
        }
    } else {
        const size_t padded_rows = (size_t)(gridDim.x / nsplit) * 64;
        partial[((size_t)q * padded_rows + row) * 8 + p] = r;
    }
}

// Kernel B: the tile tree across the nsplit workgroups of a row, then the
// phase tree and the scale.  P (a power of two >= nsplit, <= 64) lanes per
// row, lane i holding workgroup i's eight phase partials (zero past nsplit);
// level s pairs lanes i and i ^ s, which is the balanced pairwise tree.
template <typename E>
__global__ __launch_bounds__(256) void flns_combine(const int *__restrict__ partial, int rows,
                                                   int padded_rows, int nsplit, int P,
                                                   const uint8_t *__restrict__ table, int nkp,
                                                   int nkm, int ld, int32_t *__restrict__ out) {
    const E *lut = reinterpret_cast<const E *>(table + kFlnsCorrOff);
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int row = gid / P;
    const int q = gid - row * P;
    int v[8];
    if (row < rows && q < nsplit) {
        const int4 *src = reinterpret_cast<const int4 *>(partial + ((size_t)q * padded_rows + row) * 8);
        const int4 a = src[0], b = src[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int p = 0; p < 8; ++p) v[p] = kZ;
    }
    for (int s = 1; s < P; s <<= 1) {
#pragma unroll
        for (int p = 0; p < 8; ++p) v[p] = lns_add(v[p], __shfl_xor(v[p], s), lut, nkp, nkm);
    }
    if (q == 0 && row < rows)
        *reinterpret_cast<int2 *>(out + 2 * (size_t)row) = finish(phase_tree(v, lut, nkp, nkm), ld);
}

}  // namespace
}  // namespace bs

using namespace bs;

// Same K limit as the LNS8 GEMV (k <= 65408).
static constexpr int64_t kFlnsMaxK = 65408;

static int64_t flns_nsplit(int64_t k) { return (k / kGroup + kTilesPerWg - 1) / kTilesPerWg; }

static size_t flns_ws_bytes(int64_t rows, int64_t k) {
    const int64_t ns = flns_nsplit(k);
    const size_t part = ns > 1 ? (size_t)ns * (size_t)pad64(rows) * 8 * 4 : 0;
    return align_up(part > 0 ? part : 1, kWsAlign);
}

extern "C" size_t bs_flns_workspace_bytes(int64_t rows, int64_t k) {
    if (check_rows_k(rows, k, kFlnsMaxK) != BS_OK) return 0;
    return flns_ws_bytes(rows, k);
}

extern "C" int32_t bs_flns_phase_gemv(const uint8_t *planes, const uint8_t *x_lns8, int64_t rows,
                                      int64_t k, int32_t frac_bits, uint32_t scale_d,
                                      const void *table, int64_t table_bytes, int32_t *out,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    if (!planes || !x_lns8 || !table || !out) return BS_E_NULL;
    if (int32_t st = check_rows_k(rows, k, kFlnsMaxK)) return st;
    FlnsSizes sz;
    if (!flns_sizes(frac_bits, &sz) || scale_d == 0) return BS_E_RANGE;
    if (table_bytes != sz.bytes) return BS_E_RANGE;
    int64_t ld = 0;
    if (!flns_log_scale(frac_bits, scale_d, &ld)) return BS_E_RANGE;
    if (((uintptr_t)planes & 15) || ((uintptr_t)x_lns8 & 3) || ((uintptr_t)table & 15) ||
        ((uintptr_t)out & 7))
        return BS_E_ALIGN;
    if (!ws_ok(workspace, workspace_bytes, flns_ws_bytes(rows, k))) return BS_E_WORKSPACE;
    const bool small = frac_bits <= kFlnsSmallMaxFrac;
    if (small && sz.n_kp + sz.n_km > kFlnsSmallMaxEntries) return BS_E_RANGE;

    const int64_t tiles = pad64(rows) / 64;
    const int64_t groups = k / kGroup;
    const int nsplit = (int)flns_nsplit(k);
    // both grids within the 2^32 threads of one launch
    if (tiles * nsplit * kTilesPerWg * 64 >= ((int64_t)1 << 32) ||
        rows * 64 >= ((int64_t)1 << 32))
        return BS_E_SHAPE;
    hipStream_t st = (hipStream_t)stream;
    const uint8_t *tb = static_cast<const uint8_t *>(table);
    int *partial = static_cast<int *>(workspace);
    auto kern = small ? flns_tile_kernel<true> : flns_tile_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * nsplit)), dim3(kTilesPerWg * 64), 0, st,
                       planes, x_lns8, (int)rows, (int)groups, (int)frac_bits, tb, (int)sz.n_kp,
                       (int)sz.n_km, (int)ld, nsplit, out, partial);
    BS_LAUNCH_CHECK();
    if (nsplit > 1) {
        int P = 1;
        while (P < nsplit) P <<= 1;
        const int64_t threads = rows * P;
        auto comb = small ? flns_combine<int16_t> : flns_combine<int32_t>;
        hipLaunchKernelGGL(comb, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, partial,
                           (int)rows, (int)pad64(rows), nsplit, P, tb, (int)sz.n_kp, (int)sz.n_km,
                           (int)ld, out);
        BS_LAUNCH_CHECK();
    }
    return BS_OK;
}
