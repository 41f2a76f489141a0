// bs_lns8_phase_gemv: the BitState LNS8 eight-phase GEMV on gfx950
// ("BitState / HSDR PoC Technical Brief - v0.5", sections 3, 3.1 and 4).
//
// Weights are ternary bitplanes (the tiled layout of bs_ternary_gemv), the
// activations LNS8 bytes S1|E4|L3.  A ternary weight has log offset 0, so a
// product keeps the activation code and takes the sign S1 XOR [t < 0].  Each
// product adds +-(1 << E4) to one of eight int32 accumulators A[L3]; the row
// result S = 2^-9 * sum_p A[p] * F[p] is materialised once per row.
//
// Mapping: a workgroup owns one 64-row tile (lane j of every wavefront =
// row 64*tile + j, so the activation codes are uniform across a wavefront)
// and a run of 128-weight groups, one or more per wavefront.  Two
// reductions, identical in result:
//   DIRECT   -- per product position (uniform), route +-(1 << E4) to A[L3];
//   POPCOUNT -- per 64-lane tile, enumerate the active states s with a
//               ballot loop (AMD has no match-any: find the first remaining
//               lane, broadcast its code, ballot the lanes holding the same
//               code), then C_s = popcount(A_s & W_nz) - 2 popcount(A_s & W_nz
//               & (sign ^ W_neg)) and A[s & 7] += C_s << (s >> 3): the
//               histogram H[phase][band] folded into A as it is produced.
// The wavefronts' A[8] meet in LDS (integer addition is associative, so the
// order is free).  When K is split over several workgroups per tile (64
// tiles alone would leave most of the GPU idle), each workgroup writes its
// partial A to the workspace with agent-scope stores (coherent across the
// XCDs' L2s: written through, as the compiler implements agent-scope atomic
// stores), waits for them to complete, and counts itself done on the tile's
// counter with an agent-scope atomic add; the workgroup that finds itself
// last reads the partials with agent-scope loads, sums them, writes A and S
// and returns the counter and the partials to zero for the next call.  One launch, no spin,
// and no L2 write-back or invalidate: a release/acquire pair on the counter
// (buffer_wbl2 + buffer_inv) measured 19.5 us per call instead of 10-11.
#include "kcommon.h"

namespace bs {
namespace {

// F[p] = 2^((p-2)/8), p = 0..7, correctly rounded to binary64.
__device__ constexpr double kF[8] = {
    0x1.ae89f995ad3adp-1, 0x1.d5818dcfba487p-1, 0x1.0000000000000p+0, 0x1.172b83c7d517bp+0,
    0x1.306fe0a31b715p+0, 0x1.4bfdad5362a27p+0, 0x1.6a09e667f3bcdp+0, 0x1.8ace5422aa0dbp+0};

// S = 2^-9 * sum_p A[p] F[p], evaluated exactly and rounded once: every F[p]
// is an integer multiple of 2^-53 (F[p] < 2), so the sum is the integer
// sum_p A[p] * (F[p] * 2^53) (below 2^88, int128) times 2^-62.  The int128 to
// binary64 conversion rounds to nearest even; the power-of-two scaling is
// exact.
__device__ __forceinline__ double materialize(const int A[8]) {
    __int128 t = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p)
        t += (__int128)A[p] * (__int128)(int64_t)(kF[p] * 9007199254740992.0);
    return ldexp((double)t, -62);
}

// One unit of work: 64 positions (half h of group g) for the wavefront's 64
// rows.  Lane j holds row j's W_nonzero / W_negative bits of those positions
// (bit i = position 64h + i) and, for the ballots, the activation byte of
// position 64h + j.
template <int PATH>
__device__ __forceinline__ void lns8_unit(const uint8_t *__restrict__ planes,
                                          const uint8_t *__restrict__ x, int tile, int groups,
                                          int u, int lane, int A[8]) {
    const int g = u >> 1, h = u & 1;
    const size_t blk = (size_t)tile * groups + g;
    const uint2 nzv = *reinterpret_cast<const uint2 *>(planes + blk * 2048 + 16 * lane + 8 * h);
    const uint2 ngv = *reinterpret_cast<const uint2 *>(planes + blk * 2048 + 1024 + 16 * lane + 8 * h);
    const uint64_t wnz = (uint64_t)nzv.x | ((uint64_t)nzv.y << 32);
    const uint64_t wng = (uint64_t)ngv.x | ((uint64_t)ngv.y << 32);
    const int b = x[(size_t)g * 128 + 64 * h + lane];
    const int code = b & 0x7F;
    if (PATH == BS_LNS8_DIRECT) {
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
    } else {
        // pneg: the lanes' positions whose product sign is negative, S1 xor
        // [t < 0] where t != 0.  With t' = nz - 2 pneg (the product signs) and
        // any position mask M, sum_{i in M} t'_i = popcount(nz & (M ^ pneg)) -
        // popcount(pneg) (per position t'm = nz (m ^ pneg) - pneg, as in the
        // ternary GEMV), so a state costs one bitop3 and one count per 32
        // positions; the -popcount(pneg) terms of a phase's states add up to
        // -popcount(pneg) * sum_s 2^band(s), whose sum the scalar unit keeps.
        const uint64_t sign = __ballot(b >> 7);
        const uint64_t pneg = wnz & (sign ^ wng);
        const uint32_t nz0 = (uint32_t)wnz, nz1 = (uint32_t)(wnz >> 32);
        uint32_t pn0 = (uint32_t)pneg, pn1 = (uint32_t)(pneg >> 32);
        // opaque to the compiler, which would otherwise fold the nz & of
        // pneg into nz & (M ^ sign ^ neg) and spend an xor and an and per
        // word instead of one bitop3
        asm volatile("" : "+v"(pn0));
        asm volatile("" : "+v"(pn1));
        const int npn = bcnt_add(pn1, bcnt_add(pn0, 0));
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint64_t rem = __ballot(code != 0 && (code & 7) == p);
            int sum = 0;
            uint32_t bands = 0;   // uniform: sum of 2^band over the phase's states
            while (rem) {
                const int first = __builtin_ctzll(rem);
                const int st = lane_value(code, first);
                const uint64_t as = __ballot(code == st);
                rem &= ~as;
                const int band = st >> 3;
                const int c = bcnt_add(nz1 & ((uint32_t)(as >> 32) ^ pn1),
                                       bcnt_add(nz0 & ((uint32_t)as ^ pn0), 0));
                sum += c << band;
                bands += 1u << band;
            }
            // |sum|, npn * bands <= 64 * 64 * 2^15 = 2^27
            A[p] += sum - __mul24(npn, (int)bands);
        }
    }
}

// One workgroup per (64-row tile, split): wavefront w takes the units (64
// positions each, two per group) [(split * W + w) * upw, ... + upw).
template <int PATH>
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
    for (int u = u0; u < u1; ++u) lns8_unit<PATH>(planes, x, tile, groups, u, lane, A);
#pragma unroll
    for (int p = 0; p < 8; ++p) red[wave][p][lane] = A[p];
    __syncthreads();
    // pair (p, j) sums phase p of row j over the wavefronts; the 512 pairs
    // are shared out over however many threads the workgroup has
    for (int idx = threadIdx.x; idx < 512; idx += blockDim.x) {
        const int p = idx >> 6, j = idx & 63;
        int t = 0;
        for (int w = 0; w < nw; ++w) t += red[w][p][j];
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
    if (path != BS_LNS8_DIRECT && path != BS_LNS8_POPCOUNT) return BS_E_RANGE;
    if (((uintptr_t)planes & 15) || ((uintptr_t)x_lns8 & 3) || ((uintptr_t)acc & 3) ||
        ((uintptr_t)s & 7))
        return BS_E_ALIGN;
    if (!ws_ok(workspace, workspace_bytes, lns8_ws_bytes(rows, k))) return BS_E_WORKSPACE;

    const Lns8Plan pl = lns8_plan(rows, k);
    const Lns8Ws w = lns8_ws(rows, k);
    hipStream_t st = (hipStream_t)stream;
    unsigned char *base = static_cast<unsigned char *>(workspace);
    int *counters = reinterpret_cast<int *>(base + w.counters);
    int *partial = reinterpret_cast<int *>(base + w.partial);
    auto kern = path == BS_LNS8_DIRECT ? lns8_kernel<BS_LNS8_DIRECT> : lns8_kernel<BS_LNS8_POPCOUNT>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(pl.tiles * pl.nsplit)), dim3(pl.waves * 64), 0, st,
                       planes, x_lns8, (int)rows, (int)pl.groups, pl.upw, pl.nsplit, acc, s,
                       counters, partial);
    BS_LAUNCH_CHECK();
    return BS_OK;
}
