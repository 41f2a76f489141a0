// bs_lns8_phase_gemv: the BitState LNS8 eight-phase GEMV on gfx950
// ("BitState / HSDR PoC Technical Brief - v0.5", sections 3, 3.1 and 4).
//
// Weights are ternary bitplanes (the tiled layout of bs_ternary_gemv), the
// activations LNS8 bytes S1|E4|L3.  A ternary weight has log offset 0, so a
// product keeps the activation code and takes the sign S1 XOR [t < 0].  Each
// product adds +-(1 << E4) to one of eight int32 accumulators A[L3]; the row
// result S = 2^-9 * sum_p A[p] * F[p] is materialised once per row.
//
// Mapping: as for the ternary GEMV, one wavefront per (64-row tile, run of
// groups), lane j = row 64*tile + j, the activation codes uniform across the
// wave.  Two reductions, identical in result:
//   DIRECT   -- per product position (uniform), route +-(1 << E4) to A[L3];
//   POPCOUNT -- per 64-lane tile, enumerate the active states s with a
//               ballot loop (AMD has no match-any: find the first remaining
//               lane, broadcast its code, ballot the lanes holding the same
//               code), then C_s = popcount(A_s & W_nz) - 2 popcount(A_s & W_nz
//               & (sign ^ W_neg)) and A[s & 7] += C_s << (s >> 3): the
//               histogram H[phase][band] folded into A as it is produced.
// Split partials meet in a workspace through int32 atomic adds (order-free:
// integer addition is associative); the last workgroup of a tile, told by an
// atomic counter, reads them back with atomic exchanges (which re-zero the
// workspace), writes A and materialises S.
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

__device__ __forceinline__ void add_phase(int A[8], int p, int v) {
    switch (p) {
    case 0: A[0] += v; break;
    case 1: A[1] += v; break;
    case 2: A[2] += v; break;
    case 3: A[3] += v; break;
    case 4: A[4] += v; break;
    case 5: A[5] += v; break;
    case 6: A[6] += v; break;
    default: A[7] += v; break;
    }
}

template <int PATH>
__global__ __launch_bounds__(64) void lns8_kernel(
    const uint8_t *__restrict__ planes, const uint8_t *__restrict__ x, int rows, int groups,
    int gpb, int nsplit, int32_t *__restrict__ acc_out, double *__restrict__ s_out,
    int *__restrict__ ws_acc, unsigned int *__restrict__ ws_cnt) {
    const int tile = blockIdx.x / nsplit;
    const int split = blockIdx.x - tile * nsplit;
    const int lane = threadIdx.x;
    const int row = tile * 64 + lane;
    const int g0 = split * gpb;
    const int g1 = min(groups, g0 + gpb);

    int A[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int g = g0; g < g1; ++g) {
        const size_t blk = (size_t)tile * groups + g;
        const uint4 nzv = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 16 * lane);
        const uint4 ngv = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 1024 + 16 * lane);
        const uint32_t nz[4] = {nzv.x, nzv.y, nzv.z, nzv.w};
        const uint32_t ng[4] = {ngv.x, ngv.y, ngv.z, ngv.w};
        const uint8_t *xg = x + (size_t)g * 128;
        if (PATH == BS_LNS8_DIRECT) {
#pragma unroll 1
            for (int d = 0; d < 4; ++d) {
#pragma unroll 4
                for (int i = 0; i < 32; ++i) {
                    const int b = xg[32 * d + i];        // uniform activation byte
                    const int code = b & 0x7F;
                    if (code == 0) continue;
                    const int nzb = (nz[d] >> i) & 1;
                    const int ngb = (ng[d] >> i) & 1;
                    // +1, -1 or 0: the product sign is S1 xor [t < 0]
                    const int c = nzb - 2 * (nzb & (ngb ^ (b >> 7)));
                    add_phase(A, code & 7, c * (1 << (code >> 3)));
                }
            }
        } else {
#pragma unroll 1
            for (int h = 0; h < 2; ++h) {
                const uint64_t wnz = (uint64_t)nz[2 * h] | ((uint64_t)nz[2 * h + 1] << 32);
                const uint64_t wng = (uint64_t)ng[2 * h] | ((uint64_t)ng[2 * h + 1] << 32);
                const int b = xg[64 * h + lane];         // lane = position in the tile
                const int code = b & 0x7F;
                const uint64_t sign = __ballot(b >> 7);
                const uint64_t pneg = wnz & (sign ^ wng);
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    uint64_t rem = __ballot(code != 0 && (code & 7) == p);
                    while (rem) {
                        const int first = __builtin_ctzll(rem);
                        const int s = lane_value(code, first);
                        const uint64_t as = __ballot(code == s);
                        rem &= ~as;
                        const int cs = __popcll(as & wnz) - 2 * __popcll(as & pneg);
                        A[p] += cs * (1 << (s >> 3));
                    }
                }
            }
        }
    }

    if (nsplit == 1) {
        if (row < rows) {
#pragma unroll
            for (int p = 0; p < 8; ++p) acc_out[(size_t)row * 8 + p] = A[p];
            if (s_out) s_out[row] = materialize(A);
        }
        return;
    }
    if (row < rows) {
#pragma unroll
        for (int p = 0; p < 8; ++p) atomicAdd(&ws_acc[(size_t)row * 8 + p], A[p]);
    }
    // every atomic of this wavefront is performed before the tile counter
    // moves; the counter and the accumulators are only touched by atomic
    // read-modify-writes, so no cache write-back or invalidate is needed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    unsigned int prev = 0;
    if (lane == 0) prev = atomicAdd(&ws_cnt[tile], 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev == (unsigned int)(nsplit - 1)) {
        if (row < rows) {
            int T[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                T[p] = atomicExch(&ws_acc[(size_t)row * 8 + p], 0);
                acc_out[(size_t)row * 8 + p] = T[p];
            }
            if (s_out) s_out[row] = materialize(T);
        }
        if (lane == 0) atomicExch(&ws_cnt[tile], 0u);
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

// |A[p]| <= k * 2^15 must fit int32: k <= 65535, the largest multiple of 128
// below that is 65408.
static constexpr int64_t kLns8MaxK = 65408;

static size_t lns8_ws_layout(int64_t rows, size_t *cnt_off) {
    const int64_t R = pad64(rows);
    const size_t acc_bytes = align_up((size_t)R * 8 * 4, kWsAlign);
    if (cnt_off) *cnt_off = acc_bytes;
    return acc_bytes + align_up((size_t)(R / 64) * 4, kWsAlign);
}

extern "C" size_t bs_lns8_workspace_bytes(int64_t rows, int64_t k) {
    if (check_rows_k(rows, k, kLns8MaxK) != BS_OK) return 0;
    return lns8_ws_layout(rows, nullptr);
}

extern "C" int32_t bs_lns8_phase_gemv(const uint8_t *planes, const uint8_t *x_lns8,
                                      int64_t rows, int64_t k, int32_t path, int32_t *acc,
                                      double *s, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    if (!planes || !x_lns8 || !acc) return BS_E_NULL;
    if (int32_t st = check_rows_k(rows, k, kLns8MaxK)) return st;
    if (path != BS_LNS8_DIRECT && path != BS_LNS8_POPCOUNT) return BS_E_RANGE;
    size_t cnt_off = 0;
    const size_t need = lns8_ws_layout(rows, &cnt_off);
    if (!ws_ok(workspace, workspace_bytes, need)) return BS_E_WORKSPACE;

    const SplitK sk = plan_splitk(rows, k, 2048);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    auto kern = path == BS_LNS8_DIRECT ? lns8_kernel<BS_LNS8_DIRECT> : lns8_kernel<BS_LNS8_POPCOUNT>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(sk.tiles * sk.nsplit)), dim3(64), 0,
                       (hipStream_t)stream, planes, x_lns8, (int)rows, (int)sk.groups,
                       (int)sk.gpb, (int)sk.nsplit, acc, s, reinterpret_cast<int *>(ws),
                       reinterpret_cast<unsigned int *>(ws + cnt_off));
    BS_LAUNCH_CHECK();
    return BS_OK;
}
