// Activation encoders upstream of the GEMVs, on gfx950.
//
// bs_act_quant_i8: per-token absmax quantisation of int64 fixed-point
// activations to the int8 vector the ternary GEMV consumes ("A standalone
// deterministic integer inference engine for BitNet-style LLMs", section 4.4:
// absmax -> int8 per token; section 3.1: int64 fixed-point activations):
//   A = max_i |x_i|,  q_i = sgn(x_i) * floor((254 |x_i| + A) / (2A))
// (127 x / A rounded half away from zero; all zero when A = 0).
//
// bs_lns8_encode: int64 fixed-point activations (frac fractional bits) to LNS8
// bytes S1|E4|L3 ("BitState / HSDR PoC Technical Brief - v0.5", section 3:
// code k stands for 2^((k-74)/8), code 0 is exact zero; section 9 lists
// saturation and underflow among the checks).  The code of v = X / 2^frac is
// the nearest integer to 74 + 8 log2|v| (the midpoints 2^((c - 74.5)/8) are
// irrational, so there is no tie), 127 above the top code, the zero byte
// below code 1; bit 7 carries the sign of a non-zero code.  The host turns
// the code edges into exact integers once per call: t[c] = the least
// magnitude |X| whose code is at least c, i.e. ceil(2^(frac + (2c - 149)/16)),
// found by a long double estimate and settled by exact big-integer
// comparisons n^16 <=> 2^e; the kernel then binary-searches |X| among them.
//
// Both are one-workgroup kernels (a decode step quantises one vector of a
// few thousand values): the launch, not the arithmetic, is their cost.
#include <math.h>
#include <string.h>

#include "kcommon.h"
#include "dpp.h"

namespace bs {
namespace {

constexpr int kEncThreads = 1024;
constexpr uint64_t kActAbsMax = (uint64_t)1 << 55;

__device__ __forceinline__ uint64_t abs_u64(int64_t v) {
    return v < 0 ? (uint64_t)0 - (uint64_t)v : (uint64_t)v;
}

// Each thread holds up to kPerThread values in registers between the two
// passes (max, then quantise), loaded together so their latencies overlap;
// longer vectors stream through a loop.
constexpr int kPerThread = 16;

// q = floor((254 m + a) / (2a)) = floor(127 m / a + 1/2) for 0 <= m <= a <=
// 2^55, a > 0 (so q is in [0, 127]).  Estimate: binary32 m (the high word is
// below 2^24, so only the low word's conversion and the sum round, relative
// error < 2^-23) times s127 = 127 / a (relative error < 2^-22) plus 1/2; the
// product is below 128 with an error below 2^-14, so the estimate is within
// one of q, and one exact integer check each way settles it (254 m + a and
// 2a (q + 1) stay below 2^63).
__device__ __forceinline__ int8_t quant_one(int64_t v, uint64_t a, float s127) {
    if (a == 0) return 0;
    const uint64_t m = abs_u64(v);
    const float fm = (float)(uint32_t)(m >> 32) * 4294967296.0f + (float)(uint32_t)m;
    int q = (int)(fm * s127 + 0.5f);
    q = q < 0 ? 0 : (q > 127 ? 127 : q);
    const uint64_t num = 254 * m + a, den = 2 * a;
    const uint64_t t = den * (uint64_t)q;
    q = t > num ? q - 1 : (t + den <= num ? q + 1 : q);
    return (int8_t)(v < 0 ? -q : q);
}

__global__ void act_quant_kernel(const int64_t *__restrict__ x, int64_t k,
                                 int8_t *__restrict__ q, int64_t *__restrict__ absmax,
                                 int32_t *__restrict__ status) {
    __shared__ uint64_t red[16], fin;
    const bool held = k <= (int64_t)kPerThread * blockDim.x;
    int64_t v[kPerThread];
    uint64_t m = 0;
    if (held) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t i = threadIdx.x + (int64_t)j * blockDim.x;
            v[j] = i < k ? x[i] : 0;
        }
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            // slots past k are skipped, by whole wavefronts where none holds a
            // value, rather than folded in as zeros
            if (threadIdx.x + (int64_t)j * blockDim.x < k) {
                const uint64_t a = abs_u64(v[j]);
                m = a > m ? a : m;
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < k; i += blockDim.x) {
            const uint64_t a = abs_u64(x[i]);
            m = a > m ? a : m;
        }
    }
    const uint64_t a = block_max_u64(m, red, &fin);
    if (a > kActAbsMax) {   // fail loud: no quantised values, the status says why
        for (int64_t i = threadIdx.x; i < k; i += blockDim.x) q[i] = 0;
        if (threadIdx.x == 0) {
            *absmax = -1;
            *status = BS_E_OVERFLOW;
        }
        return;
    }
    const float s127 = a != 0 ? 127.0f / (float)a : 0.0f;
    if (held) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t i = threadIdx.x + (int64_t)j * blockDim.x;
            if (i < k) q[i] = quant_one(v[j], a, s127);
        }
    } else {
        for (int64_t i = threadIdx.x; i < k; i += blockDim.x) q[i] = quant_one(x[i], a, s127);
    }
    if (threadIdx.x == 0) {
        *absmax = (int64_t)a;
        *status = BS_OK;
    }
}

struct EncodeEdges {
    uint64_t t[128];   // t[c], c = 1..127: least |X| with code >= c; t[0] unused
};

__global__ void lns8_encode_kernel(const int64_t *__restrict__ x, int64_t k, EncodeEdges edges,
                                   uint8_t *__restrict__ out) {
    __shared__ uint64_t t[128];
    if (threadIdx.x < 128) t[threadIdx.x] = edges.t[threadIdx.x];
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < k;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t v = x[i];
        const uint64_t m = abs_u64(v);
        // code = number of c in 1..127 with t[c] <= m (the edges increase)
        int lo = 0, hi = 127;   // answer in [lo, hi]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (t[mid] <= m) lo = mid;
            else hi = mid - 1;
        }
        out[i] = (uint8_t)(lo == 0 ? 0 : (lo | (v < 0 ? 0x80 : 0)));
    }
}

// ---- host: exact code edges ------------------------------------------------

// Little-endian base-2^32 natural numbers large enough for n^16, n < 2^64.
struct Big {
    uint32_t d[34];
    int n;
};

static void big_from_u64(Big &b, uint64_t v) {
    memset(&b, 0, sizeof b);
    b.d[0] = (uint32_t)v;
    b.d[1] = (uint32_t)(v >> 32);
    b.n = 2;
}

static void big_square(const Big &a, Big &r) {
    Big t;
    memset(&t, 0, sizeof t);
    for (int i = 0; i < a.n; ++i) {
        uint64_t carry = 0;
        for (int j = 0; j < a.n; ++j) {
            const uint64_t cur = (uint64_t)a.d[i] * a.d[j] + t.d[i + j] + carry;
            t.d[i + j] = (uint32_t)cur;
            carry = cur >> 32;
        }
        t.d[i + a.n] = (uint32_t)carry;
    }
    t.n = 2 * a.n;
    while (t.n > 1 && t.d[t.n - 1] == 0) --t.n;
    r = t;
}

// Is n^16 >= 2^e (e >= 0)?
static bool pow16_at_least(uint64_t n, int e) {
    Big b;
    big_from_u64(b, n);
    for (int s = 0; s < 4; ++s) big_square(b, b);
    int top = b.n - 1;
    while (top > 0 && b.d[top] == 0) --top;
    const int bits = 32 * top + (b.d[top] ? 32 - __builtin_clz(b.d[top]) : 0);
    return bits - 1 >= e;   // the top set bit is 2^(bits-1) <= n^16 < 2^bits
}

// t = ceil(2^(e/16)) for odd e (an irrational power, so ceil = floor + 1);
// UINT64_MAX when it exceeds 2^63 (no int64 magnitude reaches it).
static uint64_t edge_for(int e) {
    if (e < 0) return 1;
    if (e >= 16 * 63) return UINT64_MAX;
    const long double est = powl(2.0L, (long double)e / 16.0L);
    uint64_t n = (uint64_t)floorl(est);
    n = n > 2 ? n - 2 : 1;
    // the least n with n^16 >= 2^e, from at most a few steps above the estimate
    while (!pow16_at_least(n, e)) ++n;
    return n;
}

static void encode_edges(int frac, EncodeEdges &ed) {
    ed.t[0] = 0;
    for (int c = 1; c < 128; ++c) ed.t[c] = edge_for(16 * frac + 2 * c - 149);
}

}  // namespace
}  // namespace bs

using namespace bs;

extern "C" int32_t bs_act_quant_i8(const int64_t *x, int64_t k, int8_t *q, int64_t *absmax,
                                   int32_t *status, void *stream) {
    if (!x || !q || !absmax || !status) return BS_E_NULL;
    if (k < 1 || k > ((int64_t)1 << 31)) return BS_E_SHAPE;
    if (((uintptr_t)x & 7) || ((uintptr_t)absmax & 7) || ((uintptr_t)status & 3))
        return BS_E_ALIGN;
    hipLaunchKernelGGL(act_quant_kernel, dim3(1), dim3(kEncThreads), 0, (hipStream_t)stream, x,
                       k, q, absmax, status);
    BS_LAUNCH_CHECK();
    return BS_OK;
}

extern "C" int32_t bs_lns8_encode_edges(int32_t frac, uint64_t *edges) {
    if (!edges) return BS_E_NULL;
    if (frac < 0 || frac > 62) return BS_E_RANGE;
    EncodeEdges ed;
    encode_edges(frac, ed);
    memcpy(edges, ed.t, sizeof ed.t);
    return BS_OK;
}

extern "C" int32_t bs_lns8_encode(const int64_t *x, int64_t k, int32_t frac, uint8_t *out,
                                  void *stream) {
    if (!x || !out) return BS_E_NULL;
    if (k < 1 || k > ((int64_t)1 << 31)) return BS_E_SHAPE;
    if (frac < 0 || frac > 62) return BS_E_RANGE;
    if ((uintptr_t)x & 7) return BS_E_ALIGN;
    EncodeEdges ed;
    encode_edges(frac, ed);
    const int64_t blocks = (k + 255) / 256;
    hipLaunchKernelGGL(lns8_encode_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)),
                       dim3(256), 0, (hipStream_t)stream, x, k, ed, out);
    BS_LAUNCH_CHECK();
    return BS_OK;
}
