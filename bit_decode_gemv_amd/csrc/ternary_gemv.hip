// bs_ternary_gemv: exact batch-1 ternary GEMV on gfx950.
//
// Computes, per row r, y[r] = sum_g floor(scale[r][g] * s[r][g] / 2^frac)
// with s the masked signed sum of the ternary row against int8 activations
// ("A standalone deterministic integer inference engine for BitNet-style
// LLMs", section 4.2; the W_nonzero / W_negative planes of "BitState / HSDR
// PoC Technical Brief - v0.5", section 4).
//
// Mapping: one wavefront per (64-row tile, run of `gpb` groups); lane j owns
// row 64*tile + j and streams its 16-byte W_nonzero and W_negative fields of
// each group (1 KB contiguous per plane per wavefront).  The activations of a
// group become eight bit-planes through wavefront ballots and stay in scalar
// registers, so the inner loop is AND + POPCOUNT against uniform operands:
// the signed population C = N - 2*Nneg of the brief, per activation bit.
// Tiles are split along K so that small row counts still fill the 256 CUs;
// the split partials meet in a workspace accumulator through int64 atomics
// (order-free because integer addition is associative, integer-engine page
// section 3.2) and the last workgroup of a tile writes y and re-zeroes the
// workspace.
#include "kcommon.h"

namespace bs {
namespace {

__global__ __launch_bounds__(64) void ternary_gemv_kernel(
    const uint8_t *__restrict__ planes, const int16_t *__restrict__ pscales,
    const int8_t *__restrict__ x, int rows, int groups, int gpb, int nsplit, int shift,
    int64_t *__restrict__ y, unsigned long long *__restrict__ ws_acc,
    unsigned int *__restrict__ ws_cnt) {
    const int tile = blockIdx.x / nsplit;
    const int split = blockIdx.x - tile * nsplit;
    const int lane = threadIdx.x;
    const int row = tile * 64 + lane;
    const int g0 = split * gpb;
    const int g1 = min(groups, g0 + gpb);

    int64_t acc = 0;
    for (int g = g0; g < g1; ++g) {
        const size_t blk = (size_t)tile * groups + g;
        const uint4 nzv = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 16 * lane);
        const uint4 ngv = *reinterpret_cast<const uint4 *>(planes + blk * 2048 + 1024 + 16 * lane);
        const int sc = pscales[blk * 64 + lane];
        XPlanes xp;
        ballot_planes(x + (size_t)g * 128, xp);
        const uint32_t nz[4] = {nzv.x, nzv.y, nzv.z, nzv.w};
        const uint32_t ng[4] = {ngv.x, ngv.y, ngv.z, ngv.w};
        const int s = group_dot(nz, ng, xp);
        acc += (int64_t)((s * sc) >> shift);   // arithmetic shift = floor
    }

    if (nsplit == 1) {
        if (row < rows) y[row] = acc;
        return;
    }
    if (row < rows) atomicAdd(&ws_acc[row], (unsigned long long)acc);
    __threadfence();
    unsigned int prev = 0;
    if (lane == 0) prev = atomicAdd(&ws_cnt[tile], 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev == (unsigned int)(nsplit - 1)) {
        __threadfence();
        if (row < rows) y[row] = (int64_t)atomicExch(&ws_acc[row], 0ull);
        if (lane == 0) atomicExch(&ws_cnt[tile], 0u);
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

static size_t ternary_ws_layout(int64_t rows, size_t *cnt_off) {
    const int64_t R = pad64(rows);
    const size_t acc_bytes = align_up((size_t)R * 8, kWsAlign);
    if (cnt_off) *cnt_off = acc_bytes;
    return acc_bytes + align_up((size_t)(R / 64) * 4, kWsAlign);
}

extern "C" size_t bs_ternary_gemv_workspace_bytes(int64_t rows, int64_t k) {
    if (check_rows_k(rows, k, (int64_t)1 << 24) != BS_OK) return 0;
    return ternary_ws_layout(rows, nullptr);
}

extern "C" int32_t bs_ternary_gemv(const uint8_t *planes, const int16_t *scales,
                                   const int8_t *x, int64_t rows, int64_t k, int32_t frac,
                                   int64_t *y, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (!planes || !scales || !x || !y) return BS_E_NULL;
    if (int32_t st = check_rows_k(rows, k, (int64_t)1 << 24)) return st;
    if (frac < 0 || frac > 62) return BS_E_RANGE;
    size_t cnt_off = 0;
    const size_t need = ternary_ws_layout(rows, &cnt_off);
    if (!ws_ok(workspace, workspace_bytes, need)) return BS_E_WORKSPACE;

    const SplitK sk = plan_splitk(rows, k, 2048);
    // |scale * s| < 2^30, so a shift of 31 already gives floor for any frac >= 31
    const int shift = frac > 31 ? 31 : frac;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    hipLaunchKernelGGL(ternary_gemv_kernel, dim3((unsigned)(sk.tiles * sk.nsplit)), dim3(64), 0,
                       (hipStream_t)stream, planes, scales, x, (int)rows, (int)sk.groups,
                       (int)sk.gpb, (int)sk.nsplit, shift, y,
                       reinterpret_cast<unsigned long long *>(ws),
                       reinterpret_cast<unsigned int *>(ws + cnt_off));
    BS_LAUNCH_CHECK();
    return BS_OK;
}
