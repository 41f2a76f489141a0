// bs_lmhead_planes_topk: BITNET_PLANES lm_head with two-stage exact top-k
// ("[bitnet] T2: lm_head via BITNET_PLANES weight format (WeightForm) +
// two-stage top-k decode": eight ternary planes weighted 3^-p, a stage-1
// scan over planes 0-3 of the whole vocabulary, the per-row truncation bound
// rowScale * (sum_{p=4..7} 3^-p) * sum|h|, rescoring of every row whose
// upper bound reaches the k-th best lower bound, and the maxCandidates cap).
//
// Scores are exact int64 in units of 3^-7.  Four kernels on one stream, no
// host synchronisation:
//   1. stage1  -- 8 wavefronts per workgroup, one 64-row tile each (lane =
//                 row), streaming planes 0-3 (8 KB per tile and group) with
//                 AND+POPCOUNT against ballot-built bit planes of h; writes
//                 S1' and E1 per row and the workgroup's top_k lower bounds;
//   2. select  -- one workgroup: L_k = top_k-th largest of those lists
//                 (MSB-first radix select on the order-preserving key);
//   3. filter  -- every row: U >= L_k appends the row to the candidate list;
//   4. finish  -- one workgroup: apply the cap (radix select of the top cap
//                 rows by S1' then index), rescore with planes 4-7, bitonic
//                 sort by (S' desc, index asc), write top-k and info, and
//                 re-zero the workspace counter.
#include "kcommon.h"

namespace bs {
namespace {

constexpr int kStage1Waves = 8;
constexpr int kStage1Threads = kStage1Waves * 64;
constexpr int kFinishThreads = 1024;
constexpr int kMaxCap = 4096;

// Order-preserving map of int64 onto uint64.
__device__ __forceinline__ unsigned long long okey(long long v) {
    return (unsigned long long)v ^ 0x8000000000000000ull;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

struct LmhWs {
    long long *s1;          // [V]   stage-1 score S1'
    int *e1;                // [V]   E1
    long long *lower;       // [nwg * top_k] per-workgroup best lower bounds
    long long *scalars;     // [0] = L_k, [1] = sum|h|
    unsigned int *count;    // [1]   candidate count (zero between calls)
    int *cand;              // [V]   candidate rows
};

// ---------------------------------------------------------------- stage 1
__global__ __launch_bounds__(kStage1Threads) void lmh_stage1(
    const uint8_t *__restrict__ planes03, const int32_t *__restrict__ row_scale,
    const int8_t *__restrict__ h, int vocab, int groups, int dim, int top_k, LmhWs ws) {
    __shared__ long long lds_l[kStage1Threads];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tiles = (vocab + 63) / 64;
    const int tile = blockIdx.x * kStage1Waves + wave;
    const int row = tile * 64 + lane;

    // sum |h| (each wavefront computes it; all agree)
    int habs_part = 0;
    for (int i = lane; i < dim; i += 64) habs_part += abs((int)h[i]);
    const long long habs = wave_sum(habs_part);

    long long lower = (long long)0x8000000000000000ull;   // "no row"
    if (tile < tiles) {
        int e1 = 0;
        for (int g = 0; g < groups; ++g) {
            XPlanes xp;
            ballot_planes(h + (size_t)g * 128, xp);
            const uint8_t *blk = planes03 + ((size_t)tile * groups + g) * 8192 + 16 * lane;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 nzv = *reinterpret_cast<const uint4 *>(blk + 2048 * q);
                const uint4 ngv = *reinterpret_cast<const uint4 *>(blk + 2048 * q + 1024);
                const uint32_t nz[4] = {nzv.x, nzv.y, nzv.z, nzv.w};
                const uint32_t ng[4] = {ngv.x, ngv.y, ngv.z, ngv.w};
                const int pw = q == 0 ? 27 : q == 1 ? 9 : q == 2 ? 3 : 1;   // 3^(3-q)
                e1 += pw * group_dot(nz, ng, xp);
            }
        }
        if (row < vocab) {
            const long long rs = row_scale[row];
            const long long s1 = 81LL * rs * (long long)e1;
            const long long bnd = 40LL * (rs < 0 ? -rs : rs) * habs;
            ws.s1[row] = s1;
            ws.e1[row] = e1;
            lower = s1 - bnd;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) ws.scalars[1] = habs;

    // this workgroup's top_k lower bounds (values only; ties need no order)
    lds_l[threadIdx.x] = lower;
    __syncthreads();
    int rank = 0;
    for (int j = 0; j < kStage1Threads; ++j) {
        const long long o = lds_l[j];
        rank += (o > lower) || (o == lower && j < (int)threadIdx.x);
    }
    long long *out = ws.lower + (size_t)blockIdx.x * top_k;
    if (rank < top_k) out[rank] = lower;
    for (int slot = kStage1Threads + threadIdx.x; slot < top_k; slot += kStage1Threads)
        out[slot] = (long long)0x8000000000000000ull;
}

// --------------------------------------------- radix select (one workgroup)
// Finds the `want`-th largest (1-based) of n keys given by key_of(i), with
// MSB-first 8-bit digits.  Returns the key.  All threads participate.
template <typename KeyOf>
__device__ unsigned long long radix_select_desc(int n, unsigned long long want, KeyOf key_of,
                                                unsigned int *hist, unsigned long long *bc) {
    unsigned long long prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int d = threadIdx.x; d < 256; d += blockDim.x) hist[d] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const unsigned long long k = key_of(i);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long cum = 0;
            int d = 255;
            for (; d > 0; --d) {
                if (cum + hist[d] >= want) break;
                cum += hist[d];
            }
            bc[0] = prefix | ((unsigned long long)d << shift);
            bc[1] = want - cum;
        }
        __syncthreads();
        prefix = bc[0];
        want = bc[1];
        mask |= 255ull << shift;
        __syncthreads();
    }
    return prefix;
}

__global__ __launch_bounds__(kFinishThreads) void lmh_select(int n, int top_k, LmhWs ws) {
    __shared__ unsigned int hist[256];
    __shared__ unsigned long long bc[2];
    const unsigned long long k = radix_select_desc(
        n, (unsigned long long)top_k,
        [&](int i) { return okey(ws.lower[i]); }, hist, bc);
    if (threadIdx.x == 0) ws.scalars[0] = (long long)(k ^ 0x8000000000000000ull);
}

// ----------------------------------------------------------------- filter
__global__ __launch_bounds__(256) void lmh_filter(const int32_t *__restrict__ row_scale,
                                                  int vocab, LmhWs ws) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= vocab) return;
    const long long lk = ws.scalars[0], habs = ws.scalars[1];
    const long long rs = row_scale[row];
    const long long upper = ws.s1[row] + 40LL * (rs < 0 ? -rs : rs) * habs;
    if (upper >= lk) {
        const unsigned int slot = atomicAdd(ws.count, 1u);
        if (slot < (unsigned int)vocab) ws.cand[slot] = row;
    }
}

// ----------------------------------------------------------------- finish
__global__ __launch_bounds__(kFinishThreads) void lmh_finish(
    const uint8_t *__restrict__ planes47, const int32_t *__restrict__ row_scale,
    const int8_t *__restrict__ h, int vocab, int groups, int dim, int top_k, int cap,
    int32_t *__restrict__ top_idx, int64_t *__restrict__ top_score, int32_t *__restrict__ info,
    LmhWs ws) {
    __shared__ unsigned int hist[256];
    __shared__ unsigned long long bc[2];
    __shared__ long long key[kMaxCap];
    __shared__ int idx[kMaxCap];
    __shared__ unsigned int nsel;
    extern __shared__ uint32_t hplanes[];     // [groups][8 planes][4 dwords]

    const unsigned int n = min(*ws.count, (unsigned int)vocab);
    const bool capped = n > (unsigned int)cap;

    // bit planes of h for every group
    for (int w = threadIdx.x; w < groups * 32; w += blockDim.x) {
        const int g = w >> 5, b = (w >> 2) & 7, d = w & 3;
        uint32_t m = 0;
        for (int i = 0; i < 32; ++i) m |= (uint32_t)((h[g * 128 + 32 * d + i] >> b) & 1) << i;
        hplanes[w] = m;
    }
    if (threadIdx.x == 0) nsel = 0;
    __syncthreads();

    if (!capped) {
        for (unsigned int i = threadIdx.x; i < n; i += blockDim.x) idx[i] = ws.cand[i];
        __syncthreads();
        if (threadIdx.x == 0) nsel = n;
    } else {
        // cap-th largest S1' among the candidates, then the lowest indices
        // among the rows that tie with it
        const unsigned long long tau = radix_select_desc(
            (int)n, (unsigned long long)cap, [&](int i) { return okey(ws.s1[ws.cand[i]]); },
            hist, bc);
        __shared__ unsigned int n_gt;
        if (threadIdx.x == 0) n_gt = 0;
        __syncthreads();
        for (unsigned int i = threadIdx.x; i < n; i += blockDim.x)
            if (okey(ws.s1[ws.cand[i]]) > tau) atomicAdd(&n_gt, 1u);
        __syncthreads();
        const unsigned int need_ties = (unsigned int)cap - n_gt;
        // largest of ~index among ties = smallest index; want the need_ties-th
        const unsigned long long theta = radix_select_desc(
            (int)n, (unsigned long long)need_ties,
            [&](int i) {
                const int r = ws.cand[i];
                return okey(ws.s1[r]) == tau ? (unsigned long long)(0xFFFFFFFFu - (unsigned)r) : 0ull;
            },
            hist, bc);
        for (unsigned int i = threadIdx.x; i < n; i += blockDim.x) {
            const int r = ws.cand[i];
            const unsigned long long kk = okey(ws.s1[r]);
            if (kk > tau || (kk == tau && (unsigned long long)(0xFFFFFFFFu - (unsigned)r) >= theta)) {
                const unsigned int slot = atomicAdd(&nsel, 1u);
                if (slot < (unsigned int)kMaxCap) idx[slot] = r;
            }
        }
    }
    __syncthreads();
    const int m = (int)min(nsel, (unsigned int)cap);

    // rescore with planes 4..7: one wavefront per row, lanes over (group, plane)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
    for (int c = wave; c < m; c += nwaves) {
        const int r = idx[c];
        int part = 0;
        for (int pair = lane; pair < groups * 4; pair += 64) {
            const int g = pair >> 2, q = pair & 3;
            const uint8_t *f = planes47 + (size_t)r * dim + 128 * g + 32 * q;
            const uint4 nzv = *reinterpret_cast<const uint4 *>(f);
            const uint4 ngv = *reinterpret_cast<const uint4 *>(f + 16);
            const uint32_t nz[4] = {nzv.x, nzv.y, nzv.z, nzv.w};
            const uint32_t ng[4] = {ngv.x, ngv.y, ngv.z, ngv.w};
            const uint32_t *hp = hplanes + g * 32;
            int s = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                int cn = 0, cg = 0;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    cn += __builtin_popcount(nz[d] & hp[b * 4 + d]);
                    cg += __builtin_popcount(ng[d] & hp[b * 4 + d]);
                }
                const int t = cn - 2 * cg;
                s += (b == 7) ? -t * 128 : t * (1 << b);
            }
            const int pw = q == 0 ? 27 : q == 1 ? 9 : q == 2 ? 3 : 1;    // 3^(7-(q+4))
            part += pw * s;
        }
        const int e2 = wave_sum(part);
        if (lane == 0) key[c] = (long long)row_scale[r] * (81LL * (long long)ws.e1[r] + e2);
    }
    // pad to a power of two with entries that sort last
    int mp = 1;
    while (mp < m) mp <<= 1;
    for (int i = m + threadIdx.x; i < mp; i += blockDim.x) {
        key[i] = (long long)0x8000000000000000ull;
        idx[i] = 0x7FFFFFFF;
    }
    __syncthreads();

    // bitonic sort: (key descending, index ascending)
    for (int size = 2; size <= mp; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < mp; i += blockDim.x) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;    // this run sorts "first = best"
                    const bool i_first = key[i] > key[j] || (key[i] == key[j] && idx[i] < idx[j]);
                    if (i_first != up) {
                        const long long tk = key[i];
                        key[i] = key[j];
                        key[j] = tk;
                        const int ti = idx[i];
                        idx[i] = idx[j];
                        idx[j] = ti;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < top_k; i += blockDim.x) {
        top_idx[i] = idx[i];
        top_score[i] = key[i];
    }
    if (threadIdx.x == 0) {
        info[0] = (int32_t)n;
        info[1] = capped ? 1 : 0;
        *ws.count = 0;
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

struct LmhLayout {
    size_t s1, e1, lower, scalars, count, cand, total;
    int nwg;
};

// The candidate counter is the only word that must be zero on entry.  It sits
// at offset 0 whatever the shapes, so calls of different shapes can share one
// workspace: every other region is written before it is read.
static LmhLayout lmh_layout(int64_t vocab, int32_t top_k) {
    LmhLayout L;
    const int64_t tiles = pad64(vocab) / 64;
    L.nwg = (int)((tiles + kStage1Waves - 1) / kStage1Waves);
    size_t off = 0;
    L.count = off;   off += kWsAlign;
    L.scalars = off; off += kWsAlign;
    L.s1 = off;      off += align_up((size_t)vocab * 8, kWsAlign);
    L.e1 = off;      off += align_up((size_t)vocab * 4, kWsAlign);
    L.lower = off;   off += align_up((size_t)L.nwg * (size_t)top_k * 8, kWsAlign);
    L.cand = off;    off += align_up((size_t)vocab * 4, kWsAlign);
    L.total = off;
    return L;
}

// |S'| <= 2^31 * (81*40 + 40) * 128 * dim must fit int64: dim <= 10230; the
// largest multiple of 128 below that is 10112.
static constexpr int64_t kLmhMaxDim = 10112;

static int32_t lmh_check(int64_t vocab, int64_t dim, int32_t top_k, int32_t cap) {
    if (int32_t st = check_rows_k(vocab, dim, kLmhMaxDim)) return st;
    if (top_k < 1 || cap < top_k || (int64_t)top_k > vocab || cap > kMaxCap) return BS_E_RANGE;
    return BS_OK;
}

extern "C" size_t bs_lmhead_workspace_bytes(int64_t vocab, int64_t dim, int32_t top_k,
                                            int32_t max_candidates) {
    if (lmh_check(vocab, dim, top_k, max_candidates) != BS_OK) return 0;
    return lmh_layout(vocab, top_k).total;
}

extern "C" int32_t bs_lmhead_planes_topk(const uint8_t *planes03, const uint8_t *planes47,
                                         const int32_t *row_scale, const int8_t *h,
                                         int64_t vocab, int64_t dim, int32_t top_k,
                                         int32_t max_candidates, int32_t *top_idx,
                                         int64_t *top_score, int32_t *info, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    if (!planes03 || !planes47 || !row_scale || !h || !top_idx || !top_score || !info)
        return BS_E_NULL;
    if (int32_t st = lmh_check(vocab, dim, top_k, max_candidates)) return st;
    const LmhLayout L = lmh_layout(vocab, top_k);
    if (!ws_ok(workspace, workspace_bytes, L.total)) return BS_E_WORKSPACE;

    unsigned char *base = static_cast<unsigned char *>(workspace);
    LmhWs ws;
    ws.s1 = reinterpret_cast<long long *>(base + L.s1);
    ws.e1 = reinterpret_cast<int *>(base + L.e1);
    ws.lower = reinterpret_cast<long long *>(base + L.lower);
    ws.scalars = reinterpret_cast<long long *>(base + L.scalars);
    ws.count = reinterpret_cast<unsigned int *>(base + L.count);
    ws.cand = reinterpret_cast<int *>(base + L.cand);

    hipStream_t st = (hipStream_t)stream;
    const int groups = (int)(dim / 128);
    hipLaunchKernelGGL(lmh_stage1, dim3(L.nwg), dim3(kStage1Threads), 0, st, planes03,
                       row_scale, h, (int)vocab, groups, (int)dim, top_k, ws);
    BS_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmh_select, dim3(1), dim3(kFinishThreads), 0, st, L.nwg * top_k, top_k,
                       ws);
    BS_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmh_filter, dim3((unsigned)((vocab + 255) / 256)), dim3(256), 0, st,
                       row_scale, (int)vocab, ws);
    BS_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmh_finish, dim3(1), dim3(kFinishThreads), (size_t)groups * 32 * 4, st,
                       planes47, row_scale, h, (int)vocab, groups, (int)dim, top_k,
                       max_candidates,
                       top_idx, top_score, info, ws);
    BS_LAUNCH_CHECK();
    return BS_OK;
}
