// bs_flns_phase_gemv: the pure fractional-LNS reduction of the BitState
// brief on gfx950 ("BitState / HSDR PoC Technical Brief - v0.5", section
// 5.2: count-to-log folding, kappa+/kappa- pair adds with exact
// cancellation, balanced trees, the log-domain scale).
//
// Values.  In registers a log-domain value is one int32, e = 2*L + s (s = 1
// for a negative value); zero is a coordinate far below every real one (see
// kZ).  The pair add sorts by L, looks up one correction (same-sign table,
// or opposite-sign table behind it) and adds it to L; the sign bit rides
// along.  For f <= 12 a real L stays inside (-2^24, 2^22): at most
// 2^f (127 + 8 log2 K + 8 log2 d) above, and each of at most 16 tree levels
// can lower it by |km[1]| ~ N (log2 N + 0.53) < 2^(f+7) below.
//
// Mapping.  One launch, no workspace: a workgroup of sixteen wavefronts owns
// 16 rows and all of K (flns_rows_kernel below).  Every leaf, tree node and
// tree order is the one the brief's reduction fixes; the balanced tile tree
// runs first in registers, then across the wavefronts in LDS, then across
// chunks of 32 Tile128s.  Zero-valued leaves and dead subtrees enter the
// pair adds as kZ, which every pair add with a real operand returns
// unchanged.
//
// Tables.  For frac_bits <= 8 the corrections are int16 and staged in LDS
// (at most 102,656 bytes); above, they are read from the
// device blob.  Table reads never sit behind a branch: an index past the
// table reads slot 0 and the value is discarded, so reads overlap.
#include <limits.h>

#include <type_traits>

#include "flns_layout.h"
#include "kcommon.h"

namespace bs {
namespace {

// Zero is the coordinate -2^29 with sign +: every real L lies above -2^24
// (the bound above), so against a real operand D exceeds every table and
// the pair add returns the real operand unchanged, as the identity must.
// Sums of zeros stay below -2^28 (at most +N per tree level), which is how
// a result is recognised as zero at the end; only exact cancellation
// creates a new zero.
constexpr int kZ = -(1 << 30);
constexpr int kZeroBelow = -(1 << 29);   // encoded values below this are zero
constexpr int kWavesPerWg = 16;

// The pair add of two encoded values.  Symmetric in a, b.  On encoded
// values max() picks the operand of larger L (equal L: equal values, or a
// cancelling pair), and (hi|1) - (lo|1) = 2D whatever the signs.  The
// tables are two runs of S entries (same sign, then opposite sign) whose
// last slots are zero, so clamping D to S - 1 replaces the range test, and
// the byte offset of entry D of 2-byte entries is 2D itself.  a ^ b == 1
// is equal L with opposite signs: exact cancellation.  Every conditional
// selects between named values, so nothing is emitted as a branch and the
// table read stays in flight.
template <typename E>
__device__ __forceinline__ int lns_add(int a, int b, const E *__restrict__ lut, int S) {
    const int hi = max(a, b), lo = min(a, b);
    const int x = a ^ b;
    const int d2 = (hi | 1) - (lo | 1);
    const int d2c = min(d2, 2 * S - 2);
    const int run = __mul24(x & 1, 2 * S);
    const int byte = (d2c + run) * (int)(sizeof(E) / 2);
    const int corr = (int)*reinterpret_cast<const E *>(reinterpret_cast<const char *>(lut) + byte);
    const int sum = hi + 2 * corr;
    return x == 1 ? kZ : sum;
}

// Stage n 16-byte words of the table into LDS with every load of a thread
// issued before its first store.
__device__ __forceinline__ void stage16(uint4 *__restrict__ dst, const uint4 *__restrict__ src,
                                        int n) {
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
    for (int base = threadIdx.x; base < n; base += 8 * blockDim.x) {
        u32x4 t0 = {}, t1 = {}, t2 = {}, t3 = {}, t4 = {}, t5 = {}, t6 = {}, t7 = {};
        const int st = blockDim.x;
        if (base < n) t0 = s4[base];
        if (base + st < n) t1 = s4[base + st];
        if (base + 2 * st < n) t2 = s4[base + 2 * st];
        if (base + 3 * st < n) t3 = s4[base + 3 * st];
        if (base + 4 * st < n) t4 = s4[base + 4 * st];
        if (base + 5 * st < n) t5 = s4[base + 5 * st];
        if (base + 6 * st < n) t6 = s4[base + 6 * st];
        if (base + 7 * st < n) t7 = s4[base + 7 * st];
        if (base < n) d4[base] = t0;
        if (base + st < n) d4[base + st] = t1;
        if (base + 2 * st < n) d4[base + 2 * st] = t2;
        if (base + 3 * st < n) d4[base + 3 * st] = t3;
        if (base + 4 * st < n) d4[base + 4 * st] = t4;
        if (base + 5 * st < n) d4[base + 5 * st] = t5;
        if (base + 6 * st < n) d4[base + 6 * st] = t6;
        if (base + 7 * st < n) d4[base + 7 * st] = t7;
    }
}

// Final encoding: scale, then (sign, L).
__device__ __forceinline__ int2 finish(int e, int ld) {
    if (e < kZeroBelow) return make_int2(0, 0);
    e += 2 * ld;
    return make_int2((e & 1) ? -1 : 1, e >> 1);
}

// The 8 -> 4 -> 2 -> 1 tree over the phase results.
template <typename E>
__device__ __forceinline__ int phase_tree(const int v[8], const E *__restrict__ lut, int S) {
    const int a = lns_add(lns_add(v[0], v[1], lut, S), lns_add(v[2], v[3], lut, S), lut, S);
    const int b = lns_add(lns_add(v[4], v[5], lut, S), lns_add(v[6], v[7], lut, S), lut, S);
    return lns_add(a, b, lut, S);
}

template <bool SMALL>
using LutT = typename std::conditional<SMALL, int16_t, int32_t>::type;

// Split-free mapping: a workgroup owns 16 rows and all of K.  Wavefront w
// takes Tile128s 2w and 2w + 1 of every chunk of 32, one after the other, so
// all its lanes share one Tile128 at a time (the S1 ballots stay uniform);
// quarter q (lanes 16q..16q+15, lane = row 16 * block + (lane & 15)) takes
// phases q and q + 4.  Per Tile128 the wavefront builds, in its own LDS
// region, the 128-position mask of every code and the phase-major presence
// of the codes.  The band loop of a phase walks the bands live for any of
// the four phases in flight: a band the lane's phase lacks has an empty mask,
// so its population is zero and its leaf kZ, and the pair add of anything
// with kZ returns it unchanged, so the union's extra leaves and nodes leave
// every real result as the per-phase tree gives it.  The tile tree keeps its
// balanced order: Tile128s 2w and 2w + 1 in registers, the 16 wavefronts'
// nodes in LDS, then the chunks; the phase tree and the scale follow.
constexpr int kFrRows = 16;

// Wait for this wavefront's LDS operations; its masks are private to it, so
// no workgroup barrier is involved.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_wave_barrier();
}

constexpr int kFrChunkTiles = 2 * kWavesPerWg;   // 32 Tile128s per chunk
constexpr int kFrMaxChunks = 16;                  // 65408 / 128 = 511 Tile128s

template <bool SMALL>
__global__ __launch_bounds__(1024) void flns_rows_kernel(
    const uint8_t *__restrict__ planes, const uint8_t *__restrict__ x, int rows, int groups,
    int f, const uint8_t *__restrict__ table, int S, int ld, int32_t *__restrict__ out) {
    using E = LutT<SMALL>;
    __shared__ int32_t s_fold[kFlnsFoldSlots];
    __shared__ uint4 s_lut4[SMALL ? kFlnsSmallMaxEntries * 2 / 16 : 1];
    __shared__ uint4 s_mask[kWavesPerWg][128];        // per wavefront: code -> positions
    __shared__ uint32_t s_pw[kWavesPerWg][4];          // per wavefront: presence, phase-major
    __shared__ int s_l1[kWavesPerWg][8][kFrRows];      // level-1 tile nodes
    __shared__ int s_root[kFrMaxChunks][8][kFrRows];   // chunk roots
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, r = lane & 15;
    const int row = blockIdx.x * kFrRows + r;          // < the padded row count
    const int rtile = row >> 6, rit = row & 63;

    const int32_t *g_fold = reinterpret_cast<const int32_t *>(table + kFlnsHdrBytes);
    for (int i = threadIdx.x; i < kFlnsFoldSlots; i += blockDim.x) s_fold[i] = g_fold[i];
    if constexpr (SMALL)
        stage16(s_lut4, reinterpret_cast<const uint4 *>(table + kFlnsCorrOff), (2 * S * 2 + 15) / 16);
    __syncthreads();
    const E *lut = SMALL ? reinterpret_cast<const E *>(s_lut4)
                         : reinterpret_cast<const E *>(table + kFlnsCorrOff);
    uint4 *mw = s_mask[wave];
    const int nchunks = (groups + kFrChunkTiles - 1) / kFrChunkTiles;

    for (int ch = 0; ch < nchunks; ++ch) {
        // the pair's results per phase q + 4i: ra from Tile128 2w, rb from 2w + 1
        int ra[2] = {kZ, kZ}, rb[2] = {kZ, kZ};
#pragma unroll 1
        for (int tt = 0; tt < 2; ++tt) {
            const int j = ch * kFrChunkTiles + 2 * wave + tt;   // Tile128 (group) index
            if (j >= groups) break;   // uniform
            const size_t blk = (size_t)rtile * groups + j;
            const uint4 nz = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 16 * rit);
            const uint4 ng = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 1024 + 16 * rit);
            const int b0 = x[(size_t)j * 128 + lane];
            const int b1 = x[(size_t)j * 128 + 64 + lane];
            // this wavefront's masks and presence for Tile128 j
            mw[lane] = make_uint4(0, 0, 0, 0);
            mw[64 + lane] = make_uint4(0, 0, 0, 0);
            if (lane < 4) s_pw[wave][lane] = 0;
            wave_lds_sync();
            {
                const int c0 = b0 & 0x7F, c1 = b1 & 0x7F;
                uint32_t *m0 = reinterpret_cast<uint32_t *>(mw + c0);
                uint32_t *m1 = reinterpret_cast<uint32_t *>(mw + c1);
                const int r0 = 16 * (c0 & 7) + (c0 >> 3), r1 = 16 * (c1 & 7) + (c1 >> 3);
                if (c0) {
                    atomicOr(m0 + (lane >> 5), 1u << (lane & 31));
                    atomicOr(&s_pw[wave][r0 >> 5], 1u << (r0 & 31));
                }
                if (c1) {
                    atomicOr(m1 + 2 + (lane >> 5), 1u << (lane & 31));
                    atomicOr(&s_pw[wave][r1 >> 5], 1u << (r1 & 31));
                }
            }
            wave_lds_sync();
            uint32_t pres[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) pres[w] = __builtin_amdgcn_readfirstlane(s_pw[wave][w]);
            const uint64_t s0 = __ballot(b0 >> 7), s1 = __ballot(b1 >> 7);
            uint32_t nzw[4] = {nz.x, nz.y, nz.z, nz.w};
            uint32_t neg[4];
            neg[0] = nz.x & ((uint32_t)s0 ^ ng.x);
            neg[1] = nz.y & ((uint32_t)(s0 >> 32) ^ ng.y);
            neg[2] = nz.z & ((uint32_t)s1 ^ ng.z);
            neg[3] = nz.w & ((uint32_t)(s1 >> 32) ^ ng.w);
#pragma unroll
            for (int w = 0; w < 4; ++w) asm volatile("" : "+v"(neg[w]));
            const int nneg = bcnt_add(neg[3], bcnt_add(neg[2], bcnt_add(neg[1], bcnt_add(neg[0], 0))));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int p = q + 4 * i;   // this lane's phase
                // bands live for any of phases 4i .. 4i + 3 (uniform)
                const uint32_t d0 = pres[2 * i], d1 = pres[2 * i + 1];
                const uint32_t live = (d0 | (d0 >> 16) | d1 | (d1 >> 16)) & 0xFFFFu;
                const uint4 *mp = mw + p;   // + 8 * band
                int cnt[16], fv[16];
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    cnt[b] = 0;
                    fv[b] = 0;
                    if ((live >> b) & 1) {
                        const uint4 m = mp[8 * b];
                        int c = bcnt_add(nzw[0] & (m.x ^ neg[0]), 0);
                        c = bcnt_add(nzw[1] & (m.y ^ neg[1]), c);
                        c = bcnt_add(nzw[2] & (m.z ^ neg[2]), c);
                        c = bcnt_add(nzw[3] & (m.w ^ neg[3]), c);
                        cnt[b] = c - nneg;
                        fv[b] = s_fold[abs(cnt[b])];
                    }
                }
                uint32_t lv = live;
                asm volatile("" : "+s"(lv));
                int v[16];
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    v[b] = kZ;
                    if ((lv >> b) & 1) {
                        const int ng1 = cnt[b] < 0 ? 1 : 0;
                        const int val = 2 * (((8 * b + p) << f) + fv[b]) + ng1;
                        v[b] = cnt[b] == 0 ? kZ : val;
                    }
                }
                uint32_t any = lv;
#pragma unroll
                for (int w = 8, sh = 1; w >= 1; w >>= 1, sh <<= 1) {
                    const uint32_t both = any & (any >> sh);
#pragma unroll
                    for (int m = 0; m < w; ++m) {
                        const int a = v[2 * m], c = v[2 * m + 1];
                        v[m] = (both >> (2 * sh * m)) & 1 ? lns_add(a, c, lut, S) : max(a, c);
                    }
                    any |= any >> sh;
                }
                if (tt == 0)
                    ra[i] = v[0];
                else
                    rb[i] = v[0];
            }
            wave_lds_sync();   // the next Tile128 rewrites this wavefront's masks
        }
        // level 1 of the tile tree: Tile128s 2w and 2w + 1
#pragma unroll
        for (int i = 0; i < 2; ++i)
            s_l1[wave][q + 4 * i][r] = lns_add(ra[i], rb[i], lut, S);
        __syncthreads();
        // levels 2..5 over the 16 wavefronts' nodes: thread (p, r)
        if (threadIdx.x < 8 * kFrRows) {
            const int p = threadIdx.x >> 4, rr = threadIdx.x & 15;
            int v[16];
#pragma unroll
            for (int w = 0; w < 16; ++w) v[w] = s_l1[w][p][rr];
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int m = 0; m < w; ++m) v[m] = lns_add(v[2 * m], v[2 * m + 1], lut, S);
            s_root[ch][p][rr] = v[0];
        }
        __syncthreads();
    }
    // the chunk roots in a balanced tree (kZ past the last chunk), then the
    // phase tree and the scale
    if (threadIdx.x < 8 * kFrRows) {
        const int p = threadIdx.x >> 4, rr = threadIdx.x & 15;
        int v[kFrMaxChunks];
#pragma unroll
        for (int c = 0; c < kFrMaxChunks; ++c) v[c] = c < nchunks ? s_root[c][p][rr] : kZ;
        // a pair whose right child lies past the last chunk keeps its left
        // one: the pair add with an all-zero subtree, as the padding gives
#pragma unroll
        for (int sh = 1; sh < kFrMaxChunks; sh <<= 1)
#pragma unroll
            for (int m = 0; m < kFrMaxChunks; m += 2 * sh)
                if (m + sh < nchunks) v[m] = lns_add(v[m], v[m + sh], lut, S);
        s_l1[0][p][rr] = v[0];
    }
    __syncthreads();
    if (threadIdx.x < kFrRows) {
        const int grow = blockIdx.x * kFrRows + threadIdx.x;
        if (grow < rows) {
            int ph[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) ph[k] = s_l1[0][k][threadIdx.x];
            *reinterpret_cast<int2 *>(out + 2 * (size_t)grow) = finish(phase_tree(ph, lut, S), ld);
        }
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

// Same K limit as the LNS8 GEMV (k <= 65408).
static constexpr int64_t kFlnsMaxK = 65408;

// The workspace argument is kept for the interface; the reduction needs
// none, so it is never read or written.
static size_t flns_ws_bytes(int64_t, int64_t) { return kWsAlign; }

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
    if (small && 2 * sz.stride > kFlnsSmallMaxEntries) return BS_E_RANGE;

    const int64_t groups = k / kGroup;
    const int64_t blocks = (rows + kFrRows - 1) / kFrRows;
    // the grid within the 2^32 threads of one launch
    if (blocks * kWavesPerWg * 64 >= ((int64_t)1 << 32)) return BS_E_SHAPE;
    static_assert(kFlnsMaxK / kGroup <= kFrMaxChunks * kFrChunkTiles, "chunk roots");
    const uint8_t *tb = static_cast<const uint8_t *>(table);
    auto kern = small ? flns_rows_kernel<true> : flns_rows_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kWavesPerWg * 64), 0, (hipStream_t)stream,
                       planes, x_lns8, (int)rows, (int)groups, (int)frac_bits, tb, (int)sz.stride,
                       (int)ld, out);
    BS_LAUNCH_CHECK();
    return BS_OK;
}
