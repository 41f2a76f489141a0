// bs_lmhead_planes_topk: BITNET_PLANES lm_head with two-stage exact top-k
// ("[bitnet] T2: lm_head via BITNET_PLANES weight format (WeightForm) +
// two-stage top-k decode": eight ternary planes weighted 3^-p, a stage-1
// scan over planes 0-3 of the whole vocabulary, the per-row truncation bound
// rowScale * (sum_{p=4..7} 3^-p) * sum|h|, rescoring of every row whose
// upper bound reaches the k-th best lower bound, and the maxCandidates cap).
//
// Scores are exact int64 in units of 3^-7.  The planes are stored as digit
// sums (D03 = sum_{p<4} 3^(3-p) T_p and D47 = sum_{p>=4} 3^(7-p) T_p, one
// int8 each per position), so E1 = D03 . h and E2 = D47 . h are int8 dot
// products: four products per v_dot4 instruction instead of bit-plane
// popcounts.  Four kernels on one stream, no host synchronisation, no global
// atomics:
//   stage1  -- 16 wavefronts per workgroup over 4 tiles of 64 rows (lane =
//              row), four wavefronts per tile splitting the groups; D03 is
//              streamed with 16-byte non-temporal loads (one 8 KiB group of a
//              tile per wavefront step) against h read through the scalar
//              path.  Writes E1 and the lower bound L per row, the largest L
//              of every tile and of every workgroup, and the largest S1' of
//              every tile;
//   select  -- one workgroup: L_k = the top_k-th largest L.  Histograms of
//              the tiles' maxima give T, a lower bound on L_k (at least
//              top_k tiles, so top_k distinct rows, reach it), so only the
//              rows >= T of the tiles whose maximum reaches T take part,
//              usually a few dozen (above 2048 tiles T comes from the block
//              maxima instead); and T1, a lower bound on the
//              max_candidates-th largest S1': when T1 >= L_k every row with
//              S1' >= T1 is a candidate and the cap lies among them;
//   filter  -- every row with U >= L_k becomes a candidate; those with
//              S1' >= T1 (all of them when select found no T1) are rescored
//              at once (E2 from D47, the wavefront's lanes over its
//              candidates' 16-byte runs) and stored in the workgroup's region
//              of the candidate arrays, sorted by (S1' desc, row asc);
//   finish  -- one workgroup: the cap (the max_candidates candidates with the
//              largest S1', lowest row first) among the stored rows (when
//              there are more than fit one LDS list, the max_candidates-th
//              largest region head bounds it from below, so only region
//              prefixes are read), then the top_k of the kept rows by
//              (S' desc, row asc): first among the rows a histogram bound on
//              S' names, which is the answer when the cap keeps them all,
//              else by ranking every gathered row in both orders.  Last,
//              the exactness certificate: the largest upper bound U among
//              the dropped candidates (the filter's per-region maxima of the
//              rows it did not rescore, and the stored rows past the cap)
//              against the k-th output score.
#include <mutex>

#include "kcommon.h"
#include "dpp.h"

namespace bs {
namespace {

constexpr int kTilesPerBlock = 4;
constexpr int kWavesPerTile = 4;
constexpr int kStage1Rows = kTilesPerBlock * 64;                       // 256
constexpr int kStage1Threads = kTilesPerBlock * kWavesPerTile * 64;    // 1024
constexpr int kFilterRows = 256;                                       // 4 tiles
constexpr int kBlockThreads = 1024;     // select and finish
constexpr int kSelTiles = 1024;         // select: tiles gathered
constexpr int kSelList = 4096;          // select: pruned bounds kept in LDS
constexpr int kSelPre = 2;              // select: tile maxima per thread loaded up front
constexpr int kFinList = 512;           // finish: pruned candidates kept in LDS
constexpr int kFinKpt = 4;              // finish fallback: candidates per thread in registers
constexpr int kFinSpec = 2;             // finish: entries per region loaded up front
constexpr int kMaxCap = 4096;
static_assert(kMaxCap >= kBlockThreads + kFinList, "finish: ranks and the dropped list share ti");
constexpr int kMaxGroups = 79;          // 10112 / 128
constexpr int kResU = 4;                // rescoring: 16-byte runs in flight per lane
constexpr long long kNoRow = (long long)0x8000000000000000ull;

// Order-preserving map of int64 onto uint64.
__device__ __forceinline__ unsigned long long okey(long long v) {
    return (unsigned long long)v ^ 0x8000000000000000ull;
}

// Tie-break key: larger for a lower row index.
__device__ __forceinline__ unsigned long long tie_key(int row) {
    return 0xFFFFFFFFull - (unsigned)row;
}

// (key desc, row asc)
__device__ __forceinline__ bool better(long long ka, int ia, long long kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
    const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)v, m);
    const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(v >> 32), m);
    return ((unsigned long long)hi << 32) | lo;
}

// 16 int8 weights against 16 int8 activations, added to acc.
__device__ __forceinline__ int dot16(const uint4 &w, int h0, int h1, int h2, int h3, int acc) {
    acc = __builtin_amdgcn_sdot4((int)w.x, h0, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, h1, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, h2, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, h3, acc, false);
    return acc;
}

__device__ __forceinline__ int abs_bytes(int v) {
    return abs((int)(int8_t)v) + abs((int)(int8_t)(v >> 8)) + abs((int)(int8_t)(v >> 16)) +
           abs(v >> 24);
}

struct LmhWs {
    long long *scalars;     // [0] = L_k, [1] = sum|h|, [2] = T1: candidates with S1' < T1
                            // are not rescored (kNoRow: every candidate is)
    int *e1;                // [V] E1
    long long *lower;       // [V] L
    long long *tile_max;    // [tiles] largest L of each 64-row tile
    long long *wg_max;      // [nwg] largest L of each stage-1 workgroup
    long long *tile_max_s1; // [tiles] largest S1' of each 64-row tile
    int *region_count;      // [nwf] candidates per filter workgroup
    int *region_kept;       // [nwf] candidates rescored and stored per filter workgroup
    int *cand;              // [nwf * 256] candidate rows, per-workgroup regions
    long long *cand_s1;     // [nwf * 256] their S1'
    long long *cand_s;      // [nwf * 256] their S'
    long long *cand_u;      // [nwf * 256] their upper bound U = S1' + B'
    long long *region_umax; // [nwf] largest U of the workgroup's candidates not rescored
    int *cc;                // [V] compacted candidates (more regions than one pass scans)
    long long *cc_s1;       // [V]
    long long *cc_s;        // [V]
    long long *cc_u;        // [V]
};

// ---------------------------------------------------------------- stage 1
__global__ __launch_bounds__(kStage1Threads) void lmh_stage1(
    const uint8_t *__restrict__ planes03, const int32_t *__restrict__ row_scale,
    const int32_t *__restrict__ hw, int vocab, int groups, LmhWs ws) {
    __shared__ int e1_part[kTilesPerBlock * kWavesPerTile][64];
    __shared__ int habs_part[kTilesPerBlock * kWavesPerTile];
    __shared__ long long tmax[kTilesPerBlock];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int tloc = wave / kWavesPerTile, half = wave % kWavesPerTile;
    const int tiles = (vocab + 63) / 64;
    const int tile = blockIdx.x * kTilesPerBlock + tloc;
    int e1 = 0;
    if (tile < tiles) {
        const uint8_t *tbase = planes03 + (size_t)tile * groups * 8192 + 16 * lane;
        // this wavefront takes groups half, half + kWavesPerTile, ...
        for (int g = half; g < groups; g += kWavesPerTile) {
            uint4 a[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) a[c] = load_stream16(tbase + (size_t)g * 8192 + 1024 * c);
            const int32_t *hg = hw + g * 32;      // uniform: scalar loads
#pragma unroll
            for (int c = 0; c < 8; ++c)
                e1 = dot16(a[c], hg[4 * c], hg[4 * c + 1], hg[4 * c + 2], hg[4 * c + 3], e1);
        }
    }
    // sum|h| (h is in the caches by now)
    int ha = 0;
    for (int w = threadIdx.x; w < groups * 32; w += kStage1Threads) ha += abs_bytes(hw[w]);
    ha = wave_sum(ha);
    if (lane == 0) habs_part[wave] = ha;
    e1_part[wave][lane] = e1;
    __syncthreads();
    long long habs = 0;
#pragma unroll
    for (int w = 0; w < kTilesPerBlock * kWavesPerTile; ++w) habs += habs_part[w];
    if (blockIdx.x == 0 && threadIdx.x == 0) ws.scalars[1] = habs;
    if (threadIdx.x < kStage1Rows) {
        // wavefront tl holds the rows of tile tl
        const int tl = threadIdx.x >> 6;
        const int trow = blockIdx.x * kTilesPerBlock + tl;
        const int row = trow * 64 + lane;
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerTile; ++w) tot += e1_part[tl * kWavesPerTile + w][lane];
        long long lower = kNoRow, s1 = kNoRow;
        if (row < vocab) {
            const long long rs = row_scale[row];
            s1 = 81LL * rs * (long long)tot;
            lower = s1 - 40LL * (rs < 0 ? -rs : rs) * habs;
            ws.e1[row] = tot;
            ws.lower[row] = lower;
        }
        long long mx = lower, mx1 = s1;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const long long o = (long long)shfl_xor_u64((unsigned long long)mx, off);
            const long long o1 = (long long)shfl_xor_u64((unsigned long long)mx1, off);
            mx = o > mx ? o : mx;
            mx1 = o1 > mx1 ? o1 : mx1;
        }
        if (lane == 0) {
            tmax[tl] = mx;
            if (trow < tiles) {
                ws.tile_max[trow] = mx;
                ws.tile_max_s1[trow] = mx1;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        long long mx = tmax[0];
#pragma unroll
        for (int t = 1; t < kTilesPerBlock; ++t) mx = tmax[t] > mx ? tmax[t] : mx;
        ws.wg_max[blockIdx.x] = mx;
    }
}

// ------------------------------------------ block-wide selection helpers
// Keys are visited as key_at(i, j) for i = c0 + j * blockDim.x + threadIdx.x
// (j = 0 .. KPT-1, unrolled, so a caller may map j to a register) over
// chunks c0 of KPT * blockDim.x keys; valid(i, j) says whether key i takes
// part.  Every thread of the workgroup calls.
struct SelShared {
    unsigned int hist[256];
    unsigned long long bc[2];
    unsigned long long mm[2];
    unsigned int cnt[2];
};

// The `want`-th largest (1-based) of the valid keys.  The keys are first
// offset by their minimum, so only the bytes in which they differ are
// visited, most significant first, with a 256-bin histogram per byte.
// Histogram increments are combined per wavefront when all its matching
// lanes share a digit.
template <int KPT, typename KeyAt, typename Valid>
__device__ __forceinline__ unsigned long long radix_select_desc(int n, unsigned long long want,
                                                                KeyAt key_at, Valid valid,
                                                                SelShared &sh) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) {
        sh.mm[0] = ~0ull;
        sh.mm[1] = 0;
    }
    unsigned long long lo = ~0ull, hi = 0;
    for (int c0 = 0; c0 < n; c0 += KPT * (int)blockDim.x) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = c0 + j * (int)blockDim.x + (int)threadIdx.x;
            if (i < n && valid(i, j)) {
                const unsigned long long k = key_at(i, j);
                lo = k < lo ? k : lo;
                hi = k > hi ? k : hi;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long l2 = shfl_xor_u64(lo, off), h2 = shfl_xor_u64(hi, off);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    __syncthreads();
    if (lane == 0) {
        atomicMin(&sh.mm[0], lo);
        atomicMax(&sh.mm[1], hi);
    }
    __syncthreads();
    const unsigned long long kmin = sh.mm[0], kmax = sh.mm[1];
    __syncthreads();   // mm is re-initialised by the next call
    if (kmin >= kmax) return kmin;   // a single distinct value
    const unsigned long long span = kmax - kmin;
    unsigned long long prefix = 0, mask = 0;
    for (int shift = ((63 - __clzll(span)) / 8) * 8; shift >= 0; shift -= 8) {
        for (int d = threadIdx.x; d < 256; d += blockDim.x) sh.hist[d] = 0;
        __syncthreads();
        for (int c0 = 0; c0 < n; c0 += KPT * (int)blockDim.x) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const int i = c0 + j * (int)blockDim.x + (int)threadIdx.x;
                const bool v = i < n && valid(i, j);
                const unsigned long long k = v ? key_at(i, j) - kmin : 0ull;
                const bool m = v && (k & mask) == prefix;
                const int d = (int)((k >> shift) & 255u);
                const uint64_t bm = __ballot(m);
                if (bm) {
                    const int first = __builtin_ctzll(bm);
                    const int d0 = __builtin_amdgcn_readlane(d, first);
                    if (__ballot(m && d == d0) == bm) {
                        if (lane == first) atomicAdd(&sh.hist[d0], (unsigned)__popcll(bm));
                    } else if (m) {
                        atomicAdd(&sh.hist[d], 1u);
                    }
                }
            }
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            // lane l holds digits 255-4l .. 252-4l (descending)
            unsigned c[4];
            unsigned s = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = sh.hist[255 - 4 * lane - j];
                s += c[j];
            }
            unsigned incl = s;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            unsigned long long pre = incl - s;   // matching keys in higher digits
            if (lane == 0) {
                sh.bc[0] = prefix;
                sh.bc[1] = want;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (pre < want && want <= pre + c[j]) {
                    sh.bc[0] = prefix | ((unsigned long long)(255 - 4 * lane - j) << shift);
                    sh.bc[1] = want - pre;
                }
                pre += c[j];
            }
        }
        __syncthreads();
        prefix = sh.bc[0];
        want = sh.bc[1];
        mask |= 255ull << shift;
    }
    return kmin + prefix;
}

// Counts of the keys for which cls(i, j) is 1 and 2.
template <int KPT, typename Cls>
__device__ __forceinline__ void block_count2(int n, Cls cls, SelShared &sh, unsigned &c1,
                                             unsigned &c2) {
    if (threadIdx.x == 0) {
        sh.cnt[0] = 0;
        sh.cnt[1] = 0;
    }
    __syncthreads();
    unsigned a = 0, b = 0;
    for (int c0 = 0; c0 < n; c0 += KPT * (int)blockDim.x) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = c0 + j * (int)blockDim.x + (int)threadIdx.x;
            const int c = i < n ? cls(i, j) : 0;
            a += (unsigned)__popcll(__ballot(c == 1));
            b += (unsigned)__popcll(__ballot(c == 2));
        }
    }
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&sh.cnt[0], a);
        atomicAdd(&sh.cnt[1], b);
    }
    __syncthreads();
    c1 = sh.cnt[0];
    c2 = sh.cnt[1];
    __syncthreads();
}

// Ranks of n <= 1024 entries: beats(j, e) says whether entry j comes before
// entry e in a strict total order; use(e, rank) runs once per entry with its
// rank.  The pairwise comparisons are shared out over the whole workgroup:
// entries are padded to a multiple of 64 (npad), P = blockDim / npad threads
// per entry each take a 1/P share of j (a wavefront's share is uniform), and
// the partial ranks meet in rk (int[blockDim] in LDS).
template <typename Beats, typename Use>
__device__ __forceinline__ void block_rank(int n, Beats beats, Use use, int *rk) {
    const int npad = (n + 63) & ~63;
    const int P = (int)blockDim.x / npad;
    const int t = (int)threadIdx.x, e = t % npad;
    const int part = __builtin_amdgcn_readfirstlane(t / npad);   // uniform: npad % 64 == 0
    const int chunk = (n + P - 1) / P;
    int r = 0;
    if (part < P) {
        const int j0 = part * chunk, j1 = min(n, j0 + chunk);
        if (e < n) {
#pragma unroll 8
            for (int j = j0; j < j1; ++j) r += beats(j, e) ? 1 : 0;
        }
    }
    if (t < npad * P) rk[t] = r;
    __syncthreads();
    if (t < n) {
        int tot = 0;
        for (int q = 0; q < P; ++q) tot += rk[q * npad + t];
        use(t, tot);
    }
    __syncthreads();
}

// The workgroup maxima of four 64-bit values, in every thread (a minimum is
// the complement of the maximum of complements), over the first `nactive`
// wavefronts' values.  Each of those reduces by DPP moves and its lane 63
// writes a slot; wavefront 0 folds the slots (lane = 16 * value + slot, row
// shifts), since a fold in every thread would repeat the same VALU work in
// all of the workgroup's wavefronts; every thread then reads the results.
// Every thread calls; NW (<= 16) wavefronts; red, fin in LDS, reusable after
// the next barrier.
template <int NW>
__device__ __forceinline__ void block_max4(unsigned long long v[4], int nactive,
                                           unsigned long long (*red)[4],
                                           unsigned long long *fin) {
    static_assert(NW <= 16, "one slot per lane of a 16-lane row");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wave < nactive) {   // uniform per wavefront
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = wave_max_u64_lane63(v[k]);
        if (lane == 63) {
#pragma unroll
            for (int k = 0; k < 4; ++k) red[wave][k] = v[k];
        }
    }
    __syncthreads();
    if (wave == 0) {
        const int w = lane & 15;
        unsigned long long x = w < nactive ? red[w][lane >> 4] : 0ull;
        x = dpp_max_u64<0x111, 0xF>(x);   // row_shr:1
        x = dpp_max_u64<0x112, 0xF>(x);   // row_shr:2
        x = dpp_max_u64<0x114, 0xF>(x);   // row_shr:4
        x = dpp_max_u64<0x118, 0xF>(x);   // row_shr:8
        if (w == 15) fin[lane >> 4] = x;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = fin[k];
}

// r + (a > b) for unsigned 64-bit a, b: the compare into VCC and an add of
// the carry (the compiler otherwise turns each compare into a 0/1 value,
// packs eight of them and counts the bits: about four instructions more).
__device__ __forceinline__ int add_gt_u64(int r, unsigned long long a, unsigned long long b) {
    asm("v_cmp_gt_u64_e32 vcc, %1, %2\n\tv_addc_co_u32_e32 %0, vcc, 0, %0, vcc"
        : "+v"(r)
        : "v"(a), "v"(b)
        : "vcc");
    return r;
}

// block_rank under two orders at once: step1(j, e, r) and step2(j, e, r)
// return r plus whether entry j precedes entry e in each order; use(e,
// rank1, rank2) runs on thread e (e < n).  rk1, rk2: int[blockDim] in LDS.
template <typename Step1, typename Step2, typename Use>
__device__ __forceinline__ void block_rank2(int n, Step1 step1, Step2 step2, Use use, int *rk1,
                                            int *rk2) {
    const int npad = (n + 63) & ~63;
    const int P = (int)blockDim.x / npad;
    const int t = (int)threadIdx.x, e = t % npad;
    const int part = __builtin_amdgcn_readfirstlane(t / npad);   // uniform: npad % 64 == 0
    const int chunk = (n + P - 1) / P;
    int r1 = 0, r2 = 0;
    if (part < P) {
        const int j0 = part * chunk, j1 = min(n, j0 + chunk);
        if (e < n) {
            // eight at a time, written out: the compiler will not unroll
            // loops holding inline assembly by a count that needs a remainder
            int j = j0;
            for (; j + 8 <= j1; j += 8) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    r1 = step1(j + k, e, r1);
                    r2 = step2(j + k, e, r2);
                }
            }
            for (; j < j1; ++j) {
                r1 = step1(j, e, r1);
                r2 = step2(j, e, r2);
            }
        }
    }
    if (t < npad * P) {
        rk1[t] = r1;
        rk2[t] = r2;
    }
    __syncthreads();
    if (t < n) {
        int a = 0, b = 0;
        for (int q = 0; q < P; ++q) {
            a += rk1[q * npad + t];
            b += rk2[q * npad + t];
        }
        use(t, a, b);
    }
    __syncthreads();
}

// The `want`-th largest (1-based) of n <= blockDim.x keys, thread t holding
// key t (t < n).
__device__ __forceinline__ unsigned long long rank_select_desc(int n, int want,
                                                               unsigned long long mykey,
                                                               unsigned long long *lds, int *rk,
                                                               unsigned long long *result) {
    const int t = (int)threadIdx.x;
    if (t < n) lds[t] = mykey;
    __syncthreads();
    block_rank(
        n,
        [&](int j, int e) {
            const unsigned long long o = lds[j], m = lds[e];
            return o > m || (o == m && j < e);
        },
        [&](int e, int r) {
            if (r == want - 1) *result = lds[e];
        },
        rk);
    const unsigned long long v = *result;
    __syncthreads();   // lds and result reusable
    return v;
}

// The lower edge of the bin, in a 256-bin histogram of keys (bin b holds
// kmin + [b << shift, (b + 1) << shift)), in which the count from the top
// reaches want: at least `want` keys reach it.  One wavefront calls; the
// histogram must hold at least `want` keys.  Lane l takes bins 255-4l ..
// 252-4l.
__device__ __forceinline__ void hist_edge(const unsigned *hist, unsigned want,
                                          unsigned long long kmin, int shift, int lane,
                                          unsigned long long *out) {
    unsigned c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        sum += c[j];
    }
    unsigned incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = (unsigned)__shfl_up((int)incl, off);
        if (lane >= off) incl += o;
    }
    unsigned run = incl - sum;   // keys in the bins above this lane's
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (run < want && run + c[j] >= want)
            *out = kmin + ((unsigned long long)(255 - 4 * lane - j) << shift);
        run += c[j];
    }
}

// ----------------------------------------------------------------- select
// The tail kernels take the workspace arrays (and sizes) they read first as
// leading arguments: the first 14 argument dwords are preloaded into scalar
// registers at wave launch, where the fields of the struct argument are
// loaded from memory.
__global__ __launch_bounds__(kBlockThreads) void lmh_select(
    const long long *__restrict__ tile_max, const long long *__restrict__ tile_max_s1,
    const long long *__restrict__ wg_max, long long *__restrict__ scalars,
    const long long *__restrict__ lower, int vocab, int tiles, int nwg, int top_k, int cap,
    LmhWs wsk) {
    LmhWs ws = wsk;
    ws.tile_max = const_cast<long long *>(tile_max);
    ws.tile_max_s1 = const_cast<long long *>(tile_max_s1);
    ws.wg_max = const_cast<long long *>(wg_max);
    ws.scalars = scalars;
    ws.lower = const_cast<long long *>(lower);
    __shared__ SelShared sh;
    __shared__ unsigned long long list[kSelList];
    __shared__ int tlist[kSelTiles];
    __shared__ int rk[kBlockThreads];
    __shared__ unsigned long long res;
    __shared__ unsigned int n_t, n_l;
    __shared__ unsigned int hist1[256];
    __shared__ unsigned long long red4[kBlockThreads / 64][4], fin4[4], edge[2];
    const int t = (int)threadIdx.x;
    if (t == 0) {
        n_t = 0;
        n_l = 0;
    }
    // the first kSelPre * blockDim tile maxima, loaded now so their latency
    // overlaps the workgroup maxima's and the threshold selection
    unsigned long long tpre[kSelPre], tpre1[kSelPre];   // L and S1' tile maxima
#pragma unroll
    for (int u = 0; u < kSelPre; ++u) {
        const int tt = u * (int)blockDim.x + t;
        tpre[u] = tt < tiles ? okey(ws.tile_max[tt]) : 0ull;
        tpre1[u] = tt < tiles ? okey(ws.tile_max_s1[tt]) : 0ull;
    }
    // Two bounds from histograms of the tile maxima (all of them in
    // registers when tiles <= kSelPre * blockDim; 256 bins over the span of
    // each set): T, the lower edge of the bin in which the count of the
    // tiles' largest L from the top reaches top_k, is a lower bound on L_k
    // (top_k distinct rows reach it); T1 likewise over the tiles' largest S1'
    // with cap (used below).  With more tiles, T is the top_k-th largest
    // maximum over blocks of two stage-1 workgroups.  T = 0, which keeps
    // every row, when there are fewer tiles (blocks) than top_k.
    const bool in_regs = tiles <= kSelPre * (int)blockDim.x;
    const bool want_t1 = in_regs && cap < vocab && tiles >= cap;
    unsigned long long thr = 0, t1key = 0;
    const int nblk = (nwg + 1) / 2;
    if (in_regs) {
        if (t < 256) {
            sh.hist[t] = 0;
            hist1[t] = 0;
        }
        unsigned long long lo = ~0ull, hi = 0, lo1 = ~0ull, hi1 = 0;
#pragma unroll
        for (int u = 0; u < kSelPre; ++u) {
            if (u * (int)blockDim.x + t < tiles) {
                lo = tpre[u] < lo ? tpre[u] : lo;
                hi = tpre[u] > hi ? tpre[u] : hi;
                lo1 = tpre1[u] < lo1 ? tpre1[u] : lo1;
                hi1 = tpre1[u] > hi1 ? tpre1[u] : hi1;
            }
        }
        unsigned long long mx[4] = {hi, ~lo, hi1, ~lo1};
        // (also orders the histograms' clearing)
        block_max4<kBlockThreads / 64>(mx, min(kBlockThreads / 64, (tiles + 63) / 64), red4, fin4);
        const unsigned long long kmin = ~mx[1], span = mx[0] - kmin;
        const unsigned long long kmin1 = ~mx[3], span1 = mx[2] - kmin1;
        const int shift = span >> 8 ? 64 - __clzll(span) - 8 : 0;   // bins of 2^shift keys
        const int shift1 = span1 >> 8 ? 64 - __clzll(span1) - 8 : 0;
#pragma unroll
        for (int u = 0; u < kSelPre; ++u) {
            if (u * (int)blockDim.x + t < tiles) {
                atomicAdd(&sh.hist[(int)((tpre[u] - kmin) >> shift)], 1u);
                atomicAdd(&hist1[(int)((tpre1[u] - kmin1) >> shift1)], 1u);
            }
        }
        __syncthreads();
        const int wave = t >> 6;
        if (wave == 0 && tiles >= top_k)
            hist_edge(sh.hist, (unsigned)top_k, kmin, shift, t & 63, &edge[0]);
        if (wave == 1 && want_t1) hist_edge(hist1, (unsigned)cap, kmin1, shift1, t & 63, &edge[1]);
        __syncthreads();
        if (tiles >= top_k) thr = edge[0];
        if (want_t1) t1key = edge[1];
    } else if (nblk >= top_k) {
        auto blk_key = [&](int i) {
            const unsigned long long a = okey(ws.wg_max[2 * i]);
            const unsigned long long b = 2 * i + 1 < nwg ? okey(ws.wg_max[2 * i + 1]) : 0ull;
            return a > b ? a : b;
        };
        if (nblk <= (int)blockDim.x)
            thr = rank_select_desc(nblk, top_k, t < nblk ? blk_key(t) : 0ull, list, rk, &res);
        else
            thr = radix_select_desc<4>(
                nblk, (unsigned long long)top_k, [&](int i, int) { return blk_key(i); },
                [](int, int) { return true; }, sh);
    }
    __syncthreads();
    // the tiles whose maximum reaches T
    auto take_tile = [&](int tt, unsigned long long key) {
        if (tt < tiles && key >= thr) {
            const unsigned slot = atomicAdd(&n_t, 1u);
            if (slot < (unsigned)kSelTiles) tlist[slot] = tt;
        }
    };
#pragma unroll
    for (int u = 0; u < kSelPre; ++u) take_tile(u * (int)blockDim.x + t, tpre[u]);
    for (int c0 = kSelPre * (int)blockDim.x; c0 < tiles; c0 += (int)blockDim.x) {
        const int tt = c0 + t;
        take_tile(tt, tt < tiles ? okey(ws.tile_max[tt]) : 0ull);
    }
    __syncthreads();
    const int nt = (int)n_t;
    unsigned long long kk = 0;
    bool done = false;
    if (nt <= kSelTiles) {
        // their rows that reach T, four loads in flight per thread
        for (int c0 = 0; c0 < nt * 64; c0 += 4 * (int)blockDim.x) {
            unsigned long long k[4];
            bool v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = c0 + u * (int)blockDim.x + t;
                const int row = i < nt * 64 ? tlist[i >> 6] * 64 + (i & 63) : vocab;
                v[u] = row < vocab;
                k[u] = v[u] ? okey(ws.lower[row]) : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (v[u] && k[u] >= thr) {
                    const unsigned slot = atomicAdd(&n_l, 1u);
                    if (slot < (unsigned)kSelList) list[slot] = k[u];
                }
            }
        }
        __syncthreads();
        const int ln = (int)n_l;
        if (ln <= (int)blockDim.x) {
            // pairwise ranks shared out over the workgroup (faster, measured,
            // than one wavefront walking the list with lane broadcasts even
            // for a few dozen entries)
            kk = rank_select_desc(ln, top_k, t < ln ? list[t] : 0ull, list, rk, &res);
            done = true;
        } else if (ln <= kSelList) {
            kk = radix_select_desc<4>(
                ln, (unsigned long long)top_k, [&](int i, int) { return list[i]; },
                [](int, int) { return true; }, sh);
            done = true;
        }
    }
    if (!done)
        kk = radix_select_desc<4>(
            vocab, (unsigned long long)top_k, [&](int i, int) { return okey(ws.lower[i]); },
            [&](int i, int) { return okey(ws.lower[i]) >= thr; }, sh);
    const long long lk = (long long)(kk ^ 0x8000000000000000ull);
    if (t == 0) ws.scalars[0] = lk;

    // T1 (from the histogram above) is a lower bound on the cap-th largest
    // S1' over all rows: at least cap rows (one per tile) reach it.  If
    // T1 >= L_k, every row with S1' >= T1 is a candidate (U >= S1' >= L_k), so
    // the capped set (the cap candidates with the largest S1') lies among
    // those rows, and the filter rescores only them.  Otherwise T1 = kNoRow:
    // every candidate is.
    long long t1 = kNoRow;
    if (want_t1) {
        const long long b1 = (long long)(t1key ^ 0x8000000000000000ull);
        if (b1 >= lk) t1 = b1;
    }
    if (t == 0) ws.scalars[2] = t1;
}

// --------------------------------------------------- filter + rescoring
// One workgroup per 256 rows (four wavefronts, lane = row).  Its candidates
// with S1' >= T1 are rescored and go to slots [256 * blockIdx.x,
// 256 * blockIdx.x + kept), sorted by (S1' desc, row asc); the number of
// candidates goes to region_count[blockIdx.x], kept to region_kept.
__global__ __launch_bounds__(kFilterRows) void lmh_filter(
    const long long *__restrict__ scalars, const int *__restrict__ e1p,
    const uint8_t *__restrict__ planes47, const int32_t *__restrict__ row_scale,
    const int8_t *__restrict__ h, int vocab, int groups, LmhWs wsk) {
    LmhWs ws = wsk;
    ws.scalars = const_cast<long long *>(scalars);
    ws.e1 = const_cast<int *>(e1p);
    __shared__ uint4 hs[kMaxGroups * 8];   // h, 16 positions per entry
    __shared__ int rowtab[4][64];
    __shared__ int e2l[4][64];
    __shared__ long long cs1[kFilterRows];
    __shared__ int crow[kFilterRows];
    __shared__ int wcount[4];
    __shared__ unsigned long long wumax[kFilterRows / 64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kFilterRows + (int)threadIdx.x;
    const uint2 *h2 = reinterpret_cast<const uint2 *>(h);
    uint2 *hs2 = reinterpret_cast<uint2 *>(hs);
    for (int t = threadIdx.x; t < groups * 16; t += kFilterRows) hs2[t] = h2[t];
    const long long lk = ws.scalars[0], habs = ws.scalars[1], t1 = ws.scalars[2];
    bool cand = false;
    long long s1 = 0, u = 0;
    int e1 = 0, rs = 0;
    if (row < vocab) {
        rs = row_scale[row];
        e1 = ws.e1[row];
        s1 = 81LL * (long long)rs * (long long)e1;
        const long long ars = rs < 0 ? -(long long)rs : (long long)rs;
        u = s1 + 40LL * ars * habs;
        cand = u >= lk;
    }
    const bool keep = cand && s1 >= t1;
    // the largest U among this wavefront's candidates that are not rescored
    // (for the exactness certificate)
    unsigned long long wu = cand && !keep ? okey(u) : 0ull;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = shfl_xor_u64(wu, off);
        wu = o > wu ? o : wu;
    }
    // this wavefront's rows to rescore, and the first pass of their planes
    // 4-7 loads, issued before the workgroup-wide steps below so that their
    // latency overlaps them
    const uint64_t m = __ballot(keep);
    const int nc = __popcll(m);
    const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (keep) rowtab[wave][pos] = row;
    e2l[wave][lane] = 0;
    wave_lds_fence();
    const int nrun = groups * 8;            // 16-byte runs per row
    const int total = nc * nrun;
    const size_t dim = (size_t)groups * 128;
    uint4 w0[kResU];
    int cix0[kResU], run0[kResU];
#pragma unroll
    for (int u = 0; u < kResU; ++u) {
        const int f = 64 * u + lane;
        cix0[u] = -1;
        if (f < total) {
            const int c = f / nrun;
            const int p = f - c * nrun;
            w0[u] = *reinterpret_cast<const uint4 *>(planes47 + (size_t)rowtab[wave][c] * dim +
                                                     16 * (size_t)p);
            cix0[u] = c;
            run0[u] = p;
        }
    }
    if (lane == 0) wumax[wave] = wu;
    const int ncand = __syncthreads_count(cand);
    const int nct = __syncthreads_count(keep);
    if (threadIdx.x == 0) {
        ws.region_count[blockIdx.x] = ncand;
        ws.region_kept[blockIdx.x] = nct;
        unsigned long long m = wumax[0];
        for (int w = 1; w < kFilterRows / 64; ++w) m = wumax[w] > m ? wumax[w] : m;
        ws.region_umax[blockIdx.x] = m ? (long long)(m ^ 0x8000000000000000ull) : kNoRow;
    }
    if (nct == 0) return;   // whole workgroup (no loads were issued)
    if (lane == 0) wcount[wave] = nc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcount[w];
    if (keep) {
        cs1[before + pos] = s1;
        crow[before + pos] = row;
    }
    __syncthreads();
    int rank = 0;   // position in the region: (S1' desc, row asc)
    if (keep) {
        for (int j = 0; j < nct; ++j) rank += better(cs1[j], crow[j], s1, row);
    }
    if (nc == 0) return;

#pragma unroll
    for (int u = 0; u < kResU; ++u) {
        if (cix0[u] >= 0) {
            const uint4 hv = hs[run0[u]];
            atomicAdd(&e2l[wave][cix0[u]],
                      dot16(w0[u], (int)hv.x, (int)hv.y, (int)hv.z, (int)hv.w, 0));
        }
    }
    for (int f0 = 64 * kResU; f0 < total; f0 += 64 * kResU) {
        uint4 w[kResU];
        int cix[kResU], run[kResU];
#pragma unroll
        for (int u = 0; u < kResU; ++u) {
            const int f = f0 + 64 * u + lane;
            cix[u] = -1;
            if (f < total) {
                const int c = f / nrun;
                const int p = f - c * nrun;
                w[u] = *reinterpret_cast<const uint4 *>(planes47 + (size_t)rowtab[wave][c] * dim +
                                                        16 * (size_t)p);
                cix[u] = c;
                run[u] = p;
            }
        }
#pragma unroll
        for (int u = 0; u < kResU; ++u) {
            if (cix[u] >= 0) {
                const uint4 hv = hs[run[u]];
                atomicAdd(&e2l[wave][cix[u]],
                          dot16(w[u], (int)hv.x, (int)hv.y, (int)hv.z, (int)hv.w, 0));
            }
        }
    }
    wave_lds_fence();
    if (keep) {
        const size_t slot = (size_t)blockIdx.x * kFilterRows + rank;
        ws.cand[slot] = row;
        ws.cand_s1[slot] = s1;
        ws.cand_s[slot] = (long long)rs * (81LL * (long long)e1 + (long long)e2l[wave][pos]);
        ws.cand_u[slot] = u;
    }
}

// ----------------------------------------------------------------- finish
// Where candidate i (in row order) is stored: in the filter workgroups'
// regions, found by binary search over the regions' exclusive prefix sums in
// LDS, or (when there are too many regions for that) in compacted arrays.
struct CandSrc {
    const int *ro;          // LDS prefix sums, or nullptr for compacted arrays
    int nreg;
    const int *rows;
    const long long *s1;
    const long long *s;
    const long long *u;
};

__device__ __forceinline__ size_t cand_slot(const CandSrc &c, int i) {
    if (!c.ro) return (size_t)i;
    int lo = 0, hi = c.nreg - 1;   // the last region whose prefix is <= i
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (c.ro[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return (size_t)lo * kFilterRows + (size_t)(i - c.ro[lo]);
}

template <bool REG>
__device__ __forceinline__ void finish_body(int n, int top_k, int cap, int32_t *__restrict__ top_idx,
                                            int64_t *__restrict__ top_score, const CandSrc &src,
                                            SelShared &sh, long long *tk, int *ti,
                                            unsigned int *nkept, long long *sk) {
    constexpr int KPT = kFinKpt;
    long long r_s1[KPT], r_s[KPT];
    int r_id[KPT];
    if constexpr (REG) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = j * (int)blockDim.x + (int)threadIdx.x;
            r_s1[j] = 0;
            r_s[j] = 0;
            r_id[j] = 0;
            if (i < n) {
                const size_t sl = cand_slot(src, i);
                r_s1[j] = src.s1[sl];
                r_s[j] = src.s[sl];
                r_id[j] = src.rows[sl];
            }
        }
    }
    auto S1 = [&](int i, int j) -> long long {
        if constexpr (REG) return r_s1[j]; else return src.s1[cand_slot(src, i)];
    };
    auto S = [&](int i, int j) -> long long {
        if constexpr (REG) return r_s[j]; else return src.s[cand_slot(src, i)];
    };
    auto ID = [&](int i, int j) -> int {
        if constexpr (REG) return r_id[j]; else return src.rows[cand_slot(src, i)];
    };
    auto all = [](int, int) { return true; };

    // the rows that are rescored: all of C, or its top `cap` by (S1', index)
    const bool capped = n > cap;
    unsigned long long tau = 0, theta = 0;
    if (capped) {
        tau = radix_select_desc<KPT>(
            n, (unsigned long long)cap, [&](int i, int j) { return okey(S1(i, j)); }, all, sh);
        unsigned gt, eq;
        block_count2<KPT>(
            n,
            [&](int i, int j) {
                const unsigned long long k = okey(S1(i, j));
                return k > tau ? 1 : (k == tau ? 2 : 0);
            },
            sh, gt, eq);
        const unsigned need = (unsigned)cap - gt;   // rows tying at tau that are kept
        if (need < eq)
            theta = radix_select_desc<KPT>(
                n, (unsigned long long)need, [&](int i, int j) { return tie_key(ID(i, j)); },
                [&](int i, int j) { return okey(S1(i, j)) == tau; }, sh);
    }
    // the kept rows into LDS
    if (threadIdx.x == 0) *nkept = 0;
    __syncthreads();
    for (int c0 = 0; c0 < n; c0 += KPT * (int)blockDim.x) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = c0 + j * (int)blockDim.x + (int)threadIdx.x;
            if (i < n) {
                bool keep = true;
                if (capped) {
                    const unsigned long long k = okey(S1(i, j));
                    keep = k > tau || (k == tau && tie_key(ID(i, j)) >= theta);
                }
                if (keep) {
                    const unsigned slot = atomicAdd(nkept, 1u);
                    if (slot < (unsigned)kMaxCap) {
                        tk[slot] = S(i, j);
                        ti[slot] = ID(i, j);
                    }
                }
            }
        }
    }
    __syncthreads();
    // order them by (S' desc, index asc): bitonic sort over a power of two
    const int m = (int)min(*nkept, (unsigned)kMaxCap);
    int mp = 1;
    while (mp < m) mp <<= 1;
    for (int i = m + threadIdx.x; i < mp; i += blockDim.x) {
        tk[i] = kNoRow;
        ti[i] = 0x7FFFFFFF;
    }
    __syncthreads();
    for (int size = 2; size <= mp; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < mp; i += blockDim.x) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;   // this run puts the best first
                    if (better(tk[i], ti[i], tk[j], ti[j]) != up) {
                        const long long a = tk[i];
                        tk[i] = tk[j];
                        tk[j] = a;
                        const int b = ti[i];
                        ti[i] = ti[j];
                        ti[j] = b;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < top_k; i += blockDim.x) {
        top_idx[i] = ti[i];
        top_score[i] = tk[i];
        if (i == top_k - 1) *sk = tk[i];
    }
}

// The top_k of the m rows (tk, ti) by (S' desc, row asc): each row's rank
// among them, those below top_k written at their rank.  rk: int[blockDim].
__device__ __forceinline__ void output_by_rank(int m, int top_k, const long long *tk,
                                               const int *ti, int32_t *__restrict__ top_idx,
                                               int64_t *__restrict__ top_score, int *rk,
                                               long long *sk) {
    auto put = [&](int e, int r) {
        if (r < top_k) {
            top_idx[r] = ti[e];
            top_score[r] = tk[e];
            if (r == top_k - 1) *sk = tk[e];
        }
    };
    if (m <= (int)blockDim.x) {
        block_rank(m, [&](int j, int e) { return better(tk[j], ti[j], tk[e], ti[e]); }, put, rk);
        return;
    }
    for (int e = threadIdx.x; e < m; e += blockDim.x) {
        int r = 0;
        for (int j = 0; j < m; ++j) r += better(tk[j], ti[j], tk[e], ti[e]);
        put(e, r);
    }
}

__global__ __launch_bounds__(kBlockThreads) void lmh_finish(
    const long long *__restrict__ region_umax, const int *__restrict__ region_kept,
    const int *__restrict__ region_count, int nwf, int vocab,
    const long long *__restrict__ cand_s1, const long long *__restrict__ cand_s,
    const long long *__restrict__ cand_u, const int *__restrict__ cand, int top_k, int cap,
    int32_t *__restrict__ top_idx, int64_t *__restrict__ top_score, int32_t *__restrict__ info,
    LmhWs wsk) {
    LmhWs ws = wsk;
    ws.region_umax = const_cast<long long *>(region_umax);
    ws.region_kept = const_cast<int *>(region_kept);
    ws.region_count = const_cast<int *>(region_count);
    ws.cand_s1 = const_cast<long long *>(cand_s1);
    ws.cand_s = const_cast<long long *>(cand_s);
    ws.cand_u = const_cast<long long *>(cand_u);
    ws.cand = const_cast<int *>(cand);
    __shared__ SelShared sh;
    __shared__ long long tk[kMaxCap];
    __shared__ int ti[kMaxCap];
    __shared__ int ro[kBlockThreads];
    __shared__ long long l1s1[kFinList], l1s[kFinList], l1u[kFinList];
    __shared__ int l1id[kFinList];
    __shared__ int list_all;                   // the l1 list holds every stored candidate
    __shared__ unsigned long long cert_base1;  // least S1' key of the l1 list
    __shared__ int cert_packed1;               // (S1', row) fits one 64-bit key
    __shared__ unsigned long long pk1[kFinList], pk2[kFinList];
    __shared__ unsigned long long red4[kBlockThreads / 64][4], fin4[4];
    __shared__ int l2[kFinList];
    __shared__ int fast_fail;
    __shared__ int wtot[kBlockThreads / 64], wcand[kBlockThreads / 64];
    __shared__ int wpre[kBlockThreads / 64 + 1];
    __shared__ unsigned int nkept, nl1;
    __shared__ int ncand_sh;
    __shared__ long long sk_sh;               // the k-th output score
    const int t = (int)threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int nwaves = kBlockThreads / 64;
    int n = 0;                                // rescored (stored) candidates
    CandSrc src;
    // the filter's per-region maxima of U, for the certificate at the end
    const long long umax0 = t < nwf ? ws.region_umax[t] : kNoRow;

    auto body = [&]() {

    // region t's counts, then its first kFinSpec stored entries (its head,
    // the largest S1', first), loaded while the prefix sums below run, so the
    // cap bound and the gather wait on no further load for regions that hold
    // no more; entries past a region's count are not loaded
    const int kept0 = t < nwf ? ws.region_kept[t] : 0;
    const int count0 = t < nwf ? ws.region_count[t] : 0;
    long long sp_s1[kFinSpec], sp_s[kFinSpec], sp_u[kFinSpec];
    int sp_id[kFinSpec];
#pragma unroll
    for (int u = 0; u < kFinSpec; ++u) {
        const size_t sl = (size_t)t * kFilterRows + u;
        sp_s1[u] = u < kept0 ? ws.cand_s1[sl] : 0;
        sp_s[u] = u < kept0 ? ws.cand_s[sl] : 0;
        sp_u[u] = u < kept0 ? ws.cand_u[sl] : 0;
        sp_id[u] = u < kept0 ? ws.cand[sl] : 0;
    }
    if (t == 0) list_all = 0;
    const long long head_pre = sp_s1[0];
    // exclusive prefix sums of the regions' stored counts, 1024 regions at a
    // time, and the number of candidates (wavefront 0 scans the wavefronts'
    // totals once for all)
    if (t == 0) ncand_sh = 0;
    for (int r0 = 0; r0 < nwf; r0 += kBlockThreads) {
        const int r = r0 + t;
        const int c = r0 == 0 ? kept0 : (r < nwf ? ws.region_kept[r] : 0);
        const int ca = wave_sum(r0 == 0 ? count0 : (r < nwf ? ws.region_count[r] : 0));
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wtot[wave] = incl;
        if (lane == 0) wcand[wave] = ca;
        __syncthreads();
        if (wave == 0) {
            const int x = lane < nwaves ? wtot[lane] : 0;
            const int y = wave_sum(lane < nwaves ? wcand[lane] : 0);
            int inc = x;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(inc, off);
                if (lane >= off) inc += o;
            }
            if (lane < nwaves) wpre[lane] = inc - x;
            if (lane == 63) {
                wpre[nwaves] = inc;
                ncand_sh += y;
            }
        }
        __syncthreads();
        ro[t] = n + wpre[wave] + incl - c;
        n += wpre[nwaves];
        __syncthreads();
        if (nwf <= kBlockThreads) break;   // one pass: the candidates stay in their regions
        // more regions than one pass: copy them into the compacted arrays,
        // one wavefront per region
        const int nr = min(kBlockThreads, nwf - r0);
        for (int k = wave; k < nr; k += nwaves) {
            const int cnt = ws.region_kept[r0 + k], dst = ro[k];
            const size_t from = (size_t)(r0 + k) * kFilterRows;
            for (int l = lane; l < cnt; l += 64) {
                if (dst + l < vocab) {
                    ws.cc[dst + l] = ws.cand[from + l];
                    ws.cc_s1[dst + l] = ws.cand_s1[from + l];
                    ws.cc_s[dst + l] = ws.cand_s[from + l];
                    ws.cc_u[dst + l] = ws.cand_u[from + l];
                }
            }
        }
        __syncthreads();   // copies visible to the workgroup, ro and wtot reusable
    }
    const bool regions = nwf <= kBlockThreads;
    src.ro = regions ? ro : nullptr;
    src.nreg = regions ? nwf : 0;
    src.rows = regions ? ws.cand : ws.cc;
    src.s1 = regions ? ws.cand_s1 : ws.cc_s1;
    src.s = regions ? ws.cand_s : ws.cc_s;
    src.u = regions ? ws.cand_u : ws.cc_u;
    // n rows were rescored: every candidate, or (T1 above kNoRow) those with
    // S1' >= T1, at least cap rows among which the capped set lies
    n = min(n, vocab);
    const int ncand = min(ncand_sh, vocab);
    if (t == 0) {
        info[0] = ncand;
        info[1] = ncand > cap ? 1 : 0;
    }

    if (n <= cap) {
        // every rescored row is kept: gather them, then rank
        for (int i = t; i < n; i += blockDim.x) {
            const size_t sl = cand_slot(src, i);
            tk[i] = src.s[sl];
            ti[i] = src.rows[sl];
        }
        __syncthreads();
        output_by_rank(n, top_k, tk, ti, top_idx, top_score, ro, &sk_sh);   // ro no longer needed
        return;
    }
    if (regions) {
        // T: the cap-th largest region head (cap distinct rows reach it; 0
        // when fewer than cap regions are non-empty, or when every row fits
        // the list below)
        const bool nonempty = t < nwf && (t + 1 < nwf ? ro[t + 1] : n) > ro[t];
        const int nne = n > kFinList ? __syncthreads_count(nonempty) : 0;   // n is uniform
        unsigned long long thr = 0;
        if (nne >= cap && n > kFinList) {
            const unsigned long long head = nonempty ? okey(head_pre) : 0ull;
            thr = radix_select_desc<1>(
                nwf, (unsigned long long)cap, [&](int, int) { return head; },
                [&](int, int) { return nonempty; }, sh);
        }
        if (t == 0) nl1 = 0;
        __syncthreads();
        // the sorted prefix >= T of every region
        if (t < nwf) {
            const int cnt = (t + 1 < nwf ? ro[t + 1] : n) - ro[t];
            const size_t base = (size_t)t * kFilterRows;
            bool more = true;
#pragma unroll
            for (int u = 0; u < kFinSpec; ++u) {
                if (more && u < cnt && okey(sp_s1[u]) >= thr) {
                    const unsigned slot = atomicAdd(&nl1, 1u);
                    if (slot < (unsigned)kFinList) {
                        l1s1[slot] = sp_s1[u];
                        l1s[slot] = sp_s[u];
                        l1u[slot] = sp_u[u];
                        l1id[slot] = sp_id[u];
                    }
                } else {
                    more = false;
                }
            }
            for (int e0 = kFinSpec; more && e0 < cnt; e0 += 4) {
                long long v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = e0 + u < cnt ? ws.cand_s1[base + e0 + u] : kNoRow;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (e0 + u < cnt && okey(v[u]) >= thr) {
                        const unsigned slot = atomicAdd(&nl1, 1u);
                        if (slot < (unsigned)kFinList) {
                            l1s1[slot] = v[u];
                            l1s[slot] = ws.cand_s[base + e0 + u];
                            l1u[slot] = ws.cand_u[base + e0 + u];
                            l1id[slot] = ws.cand[base + e0 + u];
                        }
                    } else {
                        more = false;   // the region is sorted: the rest are below T
                    }
                }
            }
        }
        __syncthreads();
        const int nl = (int)nl1;
        if (t == 0) list_all = nl == n && nl <= kFinList;
        if (nl <= kFinList) {
            // the ranks by (S1' desc, row asc) and by (S' desc, row asc) in
            // one pass: the cap keeps the entries whose first rank is below
            // cap, and a kept entry's output rank is its second rank less the
            // dropped entries that precede it by (S', row)
            int *dropped = ti + kBlockThreads;   // ti's first kBlockThreads: ranks
            int r1 = cap, r2 = 0;
            auto use = [&](int e, int a, int b) {
                r1 = a;
                r2 = b;
                if (a >= cap) dropped[atomicAdd(&nkept, 1u)] = e;
            };
            if (t == 0) nkept = 0;               // here: the number dropped
            if (t < 256) sh.hist[t] = 0;         // for the S' bound below
            // Each order as one 64-bit key when the list allows it:
            // ((okey(score) - least) << 17) | (2^17 - 1 - row) orders by
            // (score desc, row asc) when the scores span less than 2^47 and
            // rows are below 2^17, and a comparison is then one compare.
            unsigned long long mx[4] = {0, 0, 0, 0};
            if (t < nl) {
                const unsigned long long a1 = okey(l1s1[t]), a2 = okey(l1s[t]);
                mx[0] = a1;
                mx[1] = ~a1;
                mx[2] = a2;
                mx[3] = ~a2;
            }
            block_max4<kBlockThreads / 64>(mx, (nl + 63) / 64, red4, fin4);
            const unsigned long long base1 = ~mx[1], base2 = ~mx[3];
            const bool packed = vocab <= (1 << 17) && mx[0] - base1 < (1ull << 47) &&
                                mx[2] - base2 < (1ull << 47);
            if (t == 0) {
                cert_base1 = base1;
                cert_packed1 = vocab <= (1 << 17) && mx[0] - base1 < (1ull << 47);
            }
            // The top_k by S' first: T2, the lower edge of the histogram bin
            // (256 bins over the gathered rows' S' span) in which the count
            // from the top reaches top_k; the m rows >= T2 are ranked among
            // themselves by (S', row) and each by (S1', row) among all nl
            // gathered rows.  When every one of them ranked below top_k by S'
            // is within the cap, those are the output (the cap keeps them, and
            // every other gathered row, kept or not, is below them by S');
            // otherwise both orders are ranked over all nl rows below.
            {
                const unsigned long long span2 = mx[2] - base2;
                const int shift2 = span2 >> 8 ? 64 - __clzll(span2) - 8 : 0;
                if (t < nl) atomicAdd(&sh.hist[(int)((okey(l1s[t]) - base2) >> shift2)], 1u);
                if (t == 0) {
                    nl1 = 0;   // here: the rows >= T2
                    fast_fail = 0;
                }
                __syncthreads();
                if (t < 64) hist_edge(sh.hist, (unsigned)top_k, base2, shift2, t, &sh.bc[0]);
                __syncthreads();
                const unsigned long long t2 = sh.bc[0];
                if (t < nl && okey(l1s[t]) >= t2) l2[atomicAdd(&nl1, 1u)] = t;
                __syncthreads();
                const int m = (int)nl1;   // >= top_k
                if (m <= 256) {
                    const int npad = (m + 63) & ~63;
                    const int P = (int)blockDim.x / npad;
                    const int e = t % npad;
                    const int part = __builtin_amdgcn_readfirstlane(t / npad);
                    int a = 0, b = 0;
                    if (part < P && e < m) {
                        const int q = l2[e];
                        const long long q1 = l1s1[q], q2 = l1s[q];
                        const int qid = l1id[q];
                        const int c1 = (nl + P - 1) / P, c2 = (m + P - 1) / P;
                        for (int j = part * c1; j < min(nl, (part + 1) * c1); ++j)
                            a += better(l1s1[j], l1id[j], q1, qid) ? 1 : 0;
                        for (int p2 = part * c2; p2 < min(m, (part + 1) * c2); ++p2) {
                            const int j = l2[p2];
                            b += better(l1s[j], l1id[j], q2, qid) ? 1 : 0;
                        }
                    }
                    if (t < npad * P) {
                        ro[t] = a;
                        ti[t] = b;
                    }
                    __syncthreads();
                    int ra = 0, rb = 0;
                    if (t < m) {
                        for (int q = 0; q < P; ++q) {
                            ra += ro[q * npad + t];
                            rb += ti[q * npad + t];
                        }
                        if (rb < top_k && ra >= cap) fast_fail = 1;
                    }
                    __syncthreads();
                    if (!fast_fail) {
                        if (t < m && rb < top_k) {
                            const int q = l2[t];
                            top_idx[rb] = l1id[q];
                            top_score[rb] = l1s[q];
                            if (rb == top_k - 1) sk_sh = l1s[q];
                        }
                        return;
                    }
                }
            }
            if (packed) {
                if (t < nl) {
                    const unsigned long long tie = (unsigned long long)((1 << 17) - 1 - l1id[t]);
                    pk1[t] = ((okey(l1s1[t]) - base1) << 17) | tie;
                    pk2[t] = ((okey(l1s[t]) - base2) << 17) | tie;
                }
                __syncthreads();
                block_rank2(
                    nl, [&](int j, int e, int r) { return add_gt_u64(r, pk1[j], pk1[e]); },
                    [&](int j, int e, int r) { return add_gt_u64(r, pk2[j], pk2[e]); }, use, ro,
                    ti);   // the region prefix sums are no longer needed
            } else {
                block_rank2(
                    nl,
                    [&](int j, int e, int r) {
                        return r + (better(l1s1[j], l1id[j], l1s1[e], l1id[e]) ? 1 : 0);
                    },
                    [&](int j, int e, int r) {
                        return r + (better(l1s[j], l1id[j], l1s[e], l1id[e]) ? 1 : 0);
                    },
                    use, ro, ti);
            }
            if (r1 < cap) {   // thread t < nl holds entry t
                const int nd = (int)nkept;
                const long long me = l1s[t];
                const int my_id = l1id[t];
                int r = r2;
                for (int d = 0; d < nd; ++d) {
                    const int j = dropped[d];
                    r -= better(l1s[j], l1id[j], me, my_id) ? 1 : 0;
                }
                if (r < top_k) {
                    top_idx[r] = my_id;
                    top_score[r] = me;
                    if (r == top_k - 1) sk_sh = me;
                }
            }
            return;
        }
    }
    // fallback: block-wide radix selections over every candidate
    if (n <= kFinKpt * kBlockThreads)
        finish_body<true>(n, top_k, cap, top_idx, top_score, src, sh, tk, ti, &nkept, &sk_sh);
    else
        finish_body<false>(n, top_k, cap, top_idx, top_score, src, sh, tk, ti, &nkept, &sk_sh);
    };   // body
    body();

    // Exactness certificate (info[2]): 1 when nothing was dropped, or when
    // the largest upper bound U among the candidates the cap dropped lies
    // strictly below the k-th output score S'_k; a dropped row's S' <= U,
    // so it can neither pass nor tie the output.  The dropped rows: every
    // candidate that was not rescored (the filter's per-region maxima) and
    // the rescored rows past the top `cap` by (S1' desc, row asc).
    __syncthreads();
    const int ncand = min(ncand_sh, vocab);
    if (ncand <= cap) {
        if (t == 0) info[2] = 1;
        return;
    }
    unsigned long long m = umax0 != kNoRow ? okey(umax0) : 0ull;
    for (int r = t + kBlockThreads; r < nwf; r += kBlockThreads) {
        const long long v = ws.region_umax[r];
        if (v != kNoRow) m = okey(v) > m ? okey(v) : m;
    }
    if (n > cap && list_all) {
        // every stored row is in the LDS list (n <= 512): a row is dropped
        // when at least cap rows precede it by (S1' desc, row asc); its rank
        // counts are shared out over P = blockDim / npad parts of the list
        const int npad = (n + 63) & ~63;
        const int P = kBlockThreads / npad;
        const int e = t % npad, part = t / npad;
        const int c1 = (n + P - 1) / P;
        const int j0 = part * c1, j1 = min(n, (part + 1) * c1);
        int c = 0;
        if (cert_packed1) {
            // one 64-bit key per row: ((S1' key - least) << 17) | (2^17 - 1 - row)
            // orders by (S1' desc, row asc); pk1 is free once the output is written
            if (t < n)
                pk1[t] = ((okey(l1s1[t]) - cert_base1) << 17) |
                         (unsigned long long)((1 << 17) - 1 - l1id[t]);
            __syncthreads();
            if (part < P && e < n) {
                const unsigned long long q = pk1[e];
#pragma unroll 8
                for (int j = j0; j < j1; ++j) c += pk1[j] > q ? 1 : 0;
            }
        } else if (part < P && e < n) {
            const long long q1 = l1s1[e];
            const int qid = l1id[e];
#pragma unroll 8
            for (int j = j0; j < j1; ++j) c += better(l1s1[j], l1id[j], q1, qid) ? 1 : 0;
        }
        ti[t] = c;   // ti is free once the output is written
        __syncthreads();
        if (t < n) {
            int r1 = 0;
            for (int q = 0; q < P; ++q) r1 += ti[q * npad + t];
            if (r1 >= cap) m = okey(l1u[t]) > m ? okey(l1u[t]) : m;
        }
    } else if (n > cap) {
        if (src.ro) {
            // the output phase reused ro: the regions' exclusive prefix sums
            const int c = t < nwf ? ws.region_kept[t] : 0;
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            if (lane == 63) wtot[wave] = incl;
            __syncthreads();
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += wtot[w];
            ro[t] = pre + incl - c;
            __syncthreads();
        }
        // the cap over the stored rows by (S1' desc, row asc), as the finish
        // fallback selects it: tau the cap-th largest S1' key, theta the tie
        // bound among rows at tau
        auto key1 = [&](int i, int) { return okey(src.s1[cand_slot(src, i)]); };
        auto all = [](int, int) { return true; };
        const unsigned long long tau =
            radix_select_desc<1>(n, (unsigned long long)cap, key1, all, sh);
        unsigned gt, eq;
        block_count2<1>(
            n,
            [&](int i, int j) {
                const unsigned long long k = key1(i, j);
                return k > tau ? 1 : (k == tau ? 2 : 0);
            },
            sh, gt, eq);
        const unsigned need = (unsigned)cap - gt;   // rows tying at tau that are kept
        unsigned long long theta = 0;
        if (need < eq)
            theta = radix_select_desc<1>(
                n, (unsigned long long)need,
                [&](int i, int) { return tie_key(src.rows[cand_slot(src, i)]); },
                [&](int i, int j) { return key1(i, j) == tau; }, sh);
        for (int i = t; i < n; i += kBlockThreads) {
            const size_t sl = cand_slot(src, i);
            const unsigned long long k = okey(src.s1[sl]);
            if (k < tau || (k == tau && tie_key(src.rows[sl]) < theta))
                m = okey(src.u[sl]) > m ? okey(src.u[sl]) : m;
        }
    }
    m = wave_max_u64_lane63(m);   // DPP moves, no LDS round trip per step
    if (lane == 63) red4[wave][0] = m;
    __syncthreads();
    if (t == 0) {
        unsigned long long mm = 0;
        for (int w = 0; w < nwaves; ++w) mm = red4[w][0] > mm ? red4[w][0] : mm;
        info[2] = (mm == 0 || okey(sk_sh) > mm) ? 1 : 0;
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

struct LmhLayout {
    size_t scalars, e1, lower, tile_max, wg_max, tile_max_s1, region_count,
        region_kept, region_umax, cand, cand_s1, cand_s, cand_u, cc, cc_s1, cc_s, cc_u, total;
    int tiles, nwg, nwf;
};

static constexpr size_t align_ws(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Every region of the workspace is written before it is read, so it needs no
// initialisation and calls of any shapes may share one workspace.  The total
// grows with vocab.
static constexpr LmhLayout lmh_layout(int64_t vocab) {
    LmhLayout L{};
    L.tiles = (int)((vocab + 63) / 64);
    L.nwg = (L.tiles + kTilesPerBlock - 1) / kTilesPerBlock;
    L.nwf = (int)((vocab + kFilterRows - 1) / kFilterRows);
    const size_t slots = (size_t)L.nwf * kFilterRows;
    size_t off = 0;
    L.scalars = off;      off += kWsAlign;
    L.e1 = off;           off += align_ws((size_t)vocab * 4);
    L.lower = off;        off += align_ws((size_t)vocab * 8);
    L.tile_max = off;     off += align_ws((size_t)L.tiles * 8);
    L.wg_max = off;       off += align_ws((size_t)L.nwg * 8);
    L.tile_max_s1 = off;  off += align_ws((size_t)L.tiles * 8);
    L.region_count = off; off += align_ws((size_t)L.nwf * 4);
    L.region_kept = off;  off += align_ws((size_t)L.nwf * 4);
    L.region_umax = off;  off += align_ws((size_t)L.nwf * 8);
    L.cand = off;         off += align_ws(slots * 4);
    L.cand_s1 = off;      off += align_ws(slots * 8);
    L.cand_s = off;       off += align_ws(slots * 8);
    L.cand_u = off;       off += align_ws(slots * 8);
    L.cc = off;           off += align_ws((size_t)vocab * 4);
    L.cc_s1 = off;        off += align_ws((size_t)vocab * 8);
    L.cc_s = off;         off += align_ws((size_t)vocab * 8);
    L.cc_u = off;         off += align_ws((size_t)vocab * 8);
    L.total = off;
    return L;
}

// |S'| <= 2^31 * (81*40 + 40) * 128 * dim must fit int64: dim <= 10230; the
// largest multiple of 128 below that is 10112 (79 groups).
static constexpr int64_t kLmhMaxDim = 10112;
static_assert(kLmhMaxDim / 128 == kMaxGroups, "LDS copy of h sized for the largest dim");

static int32_t lmh_check(int64_t vocab, int64_t dim, int32_t top_k, int32_t cap) {
    if (int32_t st = check_rows_k(vocab, dim, kLmhMaxDim)) return st;
    if (vocab > ((int64_t)1 << 31) - 1024) return BS_E_SHAPE;
    if (top_k < 1 || cap < top_k || (int64_t)top_k > vocab || cap > kMaxCap) return BS_E_RANGE;
    return BS_OK;
}

extern "C" size_t bs_lmhead_workspace_bytes(int64_t vocab, int64_t dim, int32_t top_k,
                                            int32_t max_candidates) {
    if (lmh_check(vocab, dim, top_k, max_candidates) != BS_OK) return 0;
    return lmh_layout(vocab).total;
}

static int32_t lmh_args(const uint8_t *planes03, const uint8_t *planes47,
                        const int32_t *row_scale, const int8_t *h, int64_t vocab, int64_t dim,
                        int32_t top_k, int32_t max_candidates, const int32_t *top_idx,
                        const int64_t *top_score, const int32_t *info) {
    if (!planes03 || !planes47 || !row_scale || !h || !top_idx || !top_score || !info)
        return BS_E_NULL;
    if (int32_t st = lmh_check(vocab, dim, top_k, max_candidates)) return st;
    if (((uintptr_t)planes03 & 15) || ((uintptr_t)planes47 & 15) || ((uintptr_t)row_scale & 3) ||
        ((uintptr_t)h & 7) || ((uintptr_t)top_idx & 3) || ((uintptr_t)top_score & 7) ||
        ((uintptr_t)info & 3))
        return BS_E_ALIGN;
    return BS_OK;
}

// The four kernels on `stream`, with the scratch regions of lmh_layout(vocab)
// at `base` (256-byte aligned, device memory of at least L.total bytes).
static int32_t lmh_launch(const uint8_t *planes03, const uint8_t *planes47,
                          const int32_t *row_scale, const int8_t *h, int64_t vocab, int64_t dim,
                          int32_t top_k, int32_t max_candidates, int32_t *top_idx,
                          int64_t *top_score, int32_t *info, unsigned char *base,
                          const LmhLayout &L, hipStream_t st) {
    LmhWs ws;
    ws.scalars = reinterpret_cast<long long *>(base + L.scalars);
    ws.e1 = reinterpret_cast<int *>(base + L.e1);
    ws.lower = reinterpret_cast<long long *>(base + L.lower);
    ws.tile_max = reinterpret_cast<long long *>(base + L.tile_max);
    ws.wg_max = reinterpret_cast<long long *>(base + L.wg_max);
    ws.tile_max_s1 = reinterpret_cast<long long *>(base + L.tile_max_s1);
    ws.region_count = reinterpret_cast<int *>(base + L.region_count);
    ws.region_kept = reinterpret_cast<int *>(base + L.region_kept);
    ws.region_umax = reinterpret_cast<long long *>(base + L.region_umax);
    ws.cand = reinterpret_cast<int *>(base + L.cand);
    ws.cand_s1 = reinterpret_cast<long long *>(base + L.cand_s1);
    ws.cand_s = reinterpret_cast<long long *>(base + L.cand_s);
    ws.cand_u = reinterpret_cast<long long *>(base + L.cand_u);
    ws.cc = reinterpret_cast<int *>(base + L.cc);
    ws.cc_s1 = reinterpret_cast<long long *>(base + L.cc_s1);
    ws.cc_s = reinterpret_cast<long long *>(base + L.cc_s);
    ws.cc_u = reinterpret_cast<long long *>(base + L.cc_u);

    const int groups = (int)(dim / 128);
    hipLaunchKernelGGL(lmh_stage1, dim3(L.nwg), dim3(kStage1Threads), 0, st, planes03, row_scale,
                       reinterpret_cast<const int32_t *>(h), (int)vocab, groups, ws);
    BS_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmh_select, dim3(1), dim3(kBlockThreads), 0, st, ws.tile_max,
                       ws.tile_max_s1, ws.wg_max, ws.scalars, ws.lower, (int)vocab, L.tiles, L.nwg,
                       top_k, max_candidates, ws);
    BS_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmh_filter, dim3((unsigned)L.nwf), dim3(kFilterRows), 0, st, ws.scalars,
                       ws.e1, planes47, row_scale, h, (int)vocab, groups, ws);
    BS_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmh_finish, dim3(1), dim3(kBlockThreads), 0, st, ws.region_umax,
                       ws.region_kept, ws.region_count, L.nwf, (int)vocab, ws.cand_s1, ws.cand_s,
                       ws.cand_u, ws.cand, top_k, max_candidates, top_idx, top_score, info, ws);
    BS_LAUNCH_CHECK();
    return BS_OK;
}

extern "C" int32_t bs_lmhead_planes_topk(const uint8_t *planes03, const uint8_t *planes47,
                                         const int32_t *row_scale, const int8_t *h,
                                         int64_t vocab, int64_t dim, int32_t top_k,
                                         int32_t max_candidates, int32_t *top_idx,
                                         int64_t *top_score, int32_t *info, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    if (int32_t st = lmh_args(planes03, planes47, row_scale, h, vocab, dim, top_k,
                              max_candidates, top_idx, top_score, info))
        return st;
    const LmhLayout L = lmh_layout(vocab);
    if (!ws_ok(workspace, workspace_bytes, L.total)) return BS_E_WORKSPACE;
    return lmh_launch(planes03, planes47, row_scale, h, vocab, dim, top_k, max_candidates,
                      top_idx, top_score, info, static_cast<unsigned char *>(workspace), L,
                      (hipStream_t)stream);
}

// ------------------------------------------------ allocation-free variant
//
// The scratch of bs_lmhead_planes_topk_noalloc lives in this file-scope
// device array, sized for the largest vocabulary the variant accepts; every
// GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: host
// code only ever passes the address that hipGetSymbolAddress returned for
// the device, looked up once per device (with that device current) on the
// variant's first call there.
constexpr int64_t kLmhNoAllocMaxVocab = BS_LMHEAD_NOALLOC_MAX_VOCAB;
constexpr size_t kLmhScratchBytes = lmh_layout(kLmhNoAllocMaxVocab).total;
static_assert(kLmhScratchBytes % kWsAlign == 0, "scratch is a whole number of regions");

static __device__ __align__(256) unsigned char scratch[kLmhScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // per device; written once under the mutex

// The device address of `scratch` on device `dev`, looked up on first use.
int32_t scratch_for(int dev, unsigned char **out) {
    if (dev < 0 || dev >= kMaxDevices) return BS_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return BS_E_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return BS_E_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return BS_E_HIP;
        if (e != hipSuccess || p == nullptr || ((uintptr_t)p % kWsAlign) != 0) return BS_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<unsigned char *>(g_scratch_ptr[dev]);
    return BS_OK;
}
}  // namespace

extern "C" int32_t bs_lmhead_planes_topk_noalloc(const uint8_t *planes03,
                                                 const uint8_t *planes47,
                                                 const int32_t *row_scale, const int8_t *h,
                                                 int64_t vocab, int64_t dim, int32_t top_k,
                                                 int32_t max_candidates, int32_t *top_idx,
                                                 int64_t *top_score, int32_t *info,
                                                 void *stream) {
    if (int32_t st = lmh_args(planes03, planes47, row_scale, h, vocab, dim, top_k,
                              max_candidates, top_idx, top_score, info))
        return st;
    if (vocab > kLmhNoAllocMaxVocab) return BS_E_WORKSPACE;
    const LmhLayout L = lmh_layout(vocab);
    if (L.total > kLmhScratchBytes) return BS_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int dev = -1;
    if (st != nullptr) {
        if (hipStreamGetDevice(st, &dev) != hipSuccess) return BS_E_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return BS_E_HIP;
    }
    unsigned char *base = nullptr;
    if (int32_t rc = scratch_for(dev, &base)) return rc;
    return lmh_launch(planes03, planes47, row_scale, h, vocab, dim, top_k, max_candidates,
                      top_idx, top_score, info, base, L, st);
}
