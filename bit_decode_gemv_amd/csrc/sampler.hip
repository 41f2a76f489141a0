// bs_sample_candidates: one token from the scored candidates of the lm_head,
// on gfx950 (the candidate-shaped sampler of "[bitnet] T2: lm_head via
// BITNET_PLANES ..." (ScoredToken / sampleFromCandidates); the integer
// samplers of "A standalone deterministic integer inference engine for
// BitNet-style LLMs", section 3.3: greedy / temperature / top-p / min-p,
// lowest-index tie-break, a counter-based SHA-256 + Lemire draw keyed by
// (seed, position)).
//
// Order: candidates rank by (score desc, index asc, input position asc).
// Greedy returns rank 0.  Otherwise each rank gets the Q31 weight
//   w = P(t mod 2^16) >> (t >> 16),  t = (s_0 - s) * beta  (0 once t >> 16
//   reaches 32),
// P(u) ~ 2^31 * 2^(-u/2^16) the integer cubic (Horner with floor shifts,
// coefficients 1484817034, 495114803, 84039593 in Q31: a minimax fit with
// P(0) = 1 and P(1) = 1/2 exactly), beta the base-2 inverse temperature in
// Q16.  Top-p keeps the ranks whose preceding cumulative weight is below
// p * W (W the sum of all weights), min-p those whose weight is at least
// p * w_0 (p in Q16 both); both predicates hold on a prefix of the ranks.  The
// draw is Lemire's nearly-divisionless bounded integer in [0, total of the kept
// weights): each attempt a takes the first 8 bytes (big endian) of
// SHA-256(seed_le64 || position_le64 || a_le32) as the 64-bit source, up to
// 16 attempts; the token is the first rank whose cumulative weight exceeds
// the draw.  SHA-256 is written here from FIPS 180-4 (the round constants and
// initial value are derived from the cube and square roots of the first
// primes, as the standard defines them).
//
// One workgroup of up to 1024 threads, thread i holding candidate i (with
// at most 64 candidates, four wavefronts share their ranking), plus one
// wavefront that hashes the draw sources while the candidates are ranked
// (when 960 or fewer candidates leave room for it); every step is integer,
// so the result is the oracle's bit for bit.
#include "kcommon.h"

namespace bs {
namespace {

constexpr int kMaxCand = 1024;
constexpr int kRankWaves = 4;   // wavefronts sharing the ranking of at most 64 candidates
constexpr int kMaxDraws = 16;
constexpr int64_t kA1 = 1484817034, kA2 = 495114803, kA3 = 84039593;

__constant__ uint32_t kSha256K[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4,
    0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe,
    0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f,
    0x4a7484aa, 0x5cb0a9dc, 0x76f988da, 0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7,
    0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc,
    0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
    0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070, 0x19a4c116,
    0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7,
    0xc67178f2};
__constant__ uint32_t kSha256H0[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                                      0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};

// Rotate right (one v_alignbit_b32 on vector registers).
__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) {
    return (x >> n) | (x << (32 - n));
}

// a ^ b ^ c as one v_bitop3_b32 (truth table 0x96); the compiler would emit
// two xors.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// First 8 digest bytes (as a big-endian integer) of SHA-256 over the 20-byte
// message seed_le64 || position_le64 || attempt_le32: one padded block
// (FIPS 180-4 sections 5.1.1 and 6.2), message words built directly, the
// schedule kept in a rolling 16-word window so everything stays in
// registers.
__device__ uint64_t sha256_draw(uint64_t seed, uint64_t position, uint32_t attempt) {
    auto bswap = [](uint32_t v) {
        return (v >> 24) | ((v >> 8) & 0xFF00u) | ((v << 8) & 0xFF0000u) | (v << 24);
    };
    uint32_t w[16];
    w[0] = bswap((uint32_t)seed);
    w[1] = bswap((uint32_t)(seed >> 32));
    w[2] = bswap((uint32_t)position);
    w[3] = bswap((uint32_t)(position >> 32));
    w[4] = bswap(attempt);
    w[5] = 0x80000000u;   // the padding bit after 20 bytes
#pragma unroll
    for (int i = 6; i < 15; ++i) w[i] = 0;
    w[15] = 20 * 8;       // message length in bits
    uint32_t a = kSha256H0[0], b = kSha256H0[1], c = kSha256H0[2], d = kSha256H0[3];
    uint32_t e = kSha256H0[4], f = kSha256H0[5], g = kSha256H0[6], h = kSha256H0[7];
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        uint32_t wi;
        if (i < 16) {
            wi = w[i];
        } else {
            const uint32_t w15 = w[(i - 15) & 15], w2 = w[(i - 2) & 15];
            const uint32_t s0 = xor3(rotr(w15, 7), rotr(w15, 18), w15 >> 3);
            const uint32_t s1 = xor3(rotr(w2, 17), rotr(w2, 19), w2 >> 10);
            wi = w[i & 15] + s0 + w[(i - 7) & 15] + s1;
            w[i & 15] = wi;
        }
        const uint32_t S1 = xor3(rotr(e, 6), rotr(e, 11), rotr(e, 25));
        const uint32_t ch = (e & f) ^ (~e & g);
        const uint32_t t1 = h + S1 + ch + kSha256K[i] + wi;
        const uint32_t S0 = xor3(rotr(a, 2), rotr(a, 13), rotr(a, 22));
        const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
        const uint32_t t2 = S0 + mj;
        h = g; g = f; f = e; e = d + t1;
        d = c; c = b; b = a; a = t1 + t2;
    }
    return ((uint64_t)(kSha256H0[0] + a) << 32) | (uint64_t)(kSha256H0[1] + b);
}

__device__ __forceinline__ uint64_t pow2_neg_q31(uint64_t u) {
    int64_t h = kA3;
    h = kA2 - ((h * (int64_t)u) >> 16);
    h = kA1 - ((h * (int64_t)u) >> 16);
    return (uint64_t)(((int64_t)1 << 31) - ((h * (int64_t)u) >> 16));
}

__device__ __forceinline__ uint64_t weight_q31(uint64_t d, uint32_t beta) {
    if (beta == 0) return (uint64_t)1 << 31;
    if (d >= ((uint64_t)1 << 32)) return 0;   // then t >> 16 >= 2^16
    const uint64_t t = d * beta;
    const uint64_t n = t >> 16;
    if (n >= 32) return 0;
    return pow2_neg_q31(t & 0xFFFF) >> n;
}

__global__ void sample_kernel(const int32_t *__restrict__ idx, const int64_t *__restrict__ score,
                              int n, int mode, uint32_t beta, uint32_t top_p, uint32_t min_p,
                              uint64_t seed, uint64_t position, int64_t *__restrict__ result) {
    __shared__ int64_t s_in[kMaxCand];
    __shared__ int32_t i_in[kMaxCand];
    __shared__ int64_t s_rk[kMaxCand];
    __shared__ int32_t i_rk[kMaxCand];
    __shared__ uint64_t cum[kMaxCand];
    __shared__ int rk_part[kRankWaves][64];
    __shared__ uint64_t draw_sh;
    __shared__ int kept_sh, pick_sh, used_sh;
    const int t = threadIdx.x;
    // Candidates take threads [0, nc), thread i holding candidate i; with at
    // most 64 (one wavefront) kRankWaves wavefronts each hold all of them
    // (lane i: candidate i) and share the ranking.  The draw sources take the
    // wavefront from thread hw: its own, after those (its hashing then runs
    // on another SIMD while the candidates are ranked), when the workgroup
    // has room for it, else the first.
    const bool one_wave = n <= 64;
    const int nc = (n + 63) & ~63;
    const int hw = one_wave ? 64 * kRankWaves : ((int)blockDim.x > nc ? nc : 0);
    const int cand = one_wave ? (t < 64 * kRankWaves ? (t & 63) : n) : t;
    int64_t my_s = 0;
    int32_t my_i = 0;
    if (cand < n) {
        my_s = score[cand];
        my_i = idx[cand];
    }
    // The draw sources do not depend on the candidates: lane a of the hashing
    // wavefront hashes attempt a (SHA-256 of seed, position, a) while the
    // candidates are ranked.  With at most 64 candidates the ranking reads
    // them from lane registers, so no barrier comes before it and the two
    // meet only at the barrier after the ranking; otherwise the candidates go
    // to LDS first.
    if (!one_wave) {
        if (t < n) {
            s_in[t] = my_s;
            i_in[t] = my_i;
        }
        __syncthreads();
    }
    uint64_t u = 0;
    if (mode != 0 && t >= hw && t < hw + 64) u = sha256_draw(seed, position, (uint32_t)(t - hw));
    // rank: the candidates before this one by (score desc, index asc,
    // input position asc)
    const int64_t s = my_s;
    const int32_t id = my_i;
    auto beats = [&](int64_t sj, int32_t ij, int j) {
        return (sj > s) || (sj == s && (ij < id || (ij == id && j < cand)));
    };
    if (one_wave) {
        // wavefront w compares against candidates [w * chunk, (w + 1) * chunk),
        // each straight from lane j's registers
        if (t < 64 * kRankWaves) {
            const int w = t >> 6, chunk = (n + kRankWaves - 1) / kRankWaves;
            const int j0 = w * chunk, j1 = min(n, j0 + chunk);
            int r = 0;
            if (cand < n) {
                for (int j = j0; j < j1; ++j) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_s, j);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(
                        (int)(uint32_t)((uint64_t)my_s >> 32), j);
                    r += beats((int64_t)(((uint64_t)hi << 32) | lo),
                               __builtin_amdgcn_readlane(my_i, j), j);
                }
            }
            rk_part[w][t & 63] = r;
        }
        __syncthreads();
        if (t < n) {
            int r = 0;
#pragma unroll
            for (int w = 0; w < kRankWaves; ++w) r += rk_part[w][t];
            s_rk[r] = s;
            i_rk[r] = id;
        }
    } else if (t < n) {
        int r = 0;
        for (int j = 0; j < n; ++j) r += beats(s_in[j], i_in[j], j);
        s_rk[r] = s;
        i_rk[r] = id;
    }
    __syncthreads();
    if (mode == 0) {   // greedy
        if (t == 0) {
            result[0] = i_rk[0];
            result[1] = 0;
            result[2] = 1;
            result[3] = 0;
            result[4] = 0;
            result[5] = 0;
        }
        return;
    }
    // weights in rank order and their inclusive prefix sums
    uint64_t w = 0;
    if (t < n) w = weight_q31((uint64_t)s_rk[0] - (uint64_t)s_rk[t], beta);
    if (nc == 64) {
        // one wavefront of candidates: an inclusive scan by lane shuffles
        if (t < 64) {
            uint64_t incl = w;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)incl, off);
                const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(incl >> 32), off);
                if (t >= off) incl += ((uint64_t)hi << 32) | lo;
            }
            cum[t] = incl;
        }
        __syncthreads();
    } else {
        cum[t] = w;
        __syncthreads();
        for (int off = 1; off < nc; off <<= 1) {
            const uint64_t add = t >= off ? cum[t - off] : 0;
            __syncthreads();
            cum[t] += add;
            __syncthreads();
        }
    }
    const uint64_t wall = cum[n - 1];
    const uint64_t w0 = (uint64_t)1 << 31;   // rank 0: d = 0
    if (t == 0) kept_sh = 0;
    __syncthreads();
    if (t < n) {
        const uint64_t before = cum[t] - w;
        const bool keep = ((before << 16) < (uint64_t)top_p * wall) &&
                          ((w << 16) >= (uint64_t)min_p * w0);
        if (keep) atomicAdd(&kept_sh, 1);   // the kept ranks form a prefix
    }
    __syncthreads();
    const int kept = kept_sh;
    const uint64_t total = cum[kept - 1];
    if (t >= hw && t < hw + 64) {
        // lane a holds attempt a's source (its digest's rounds ran on the
        // vector unit: rotates, three-input xors and the choose/majority
        // functions are one instruction each there); the first attempt that
        // Lemire's method accepts is the draw, and the attempts it used are
        // its index + 1, as if taken one by one
        const uint64_t tot = total;
        const uint64_t lo = u * tot;
        bool reject = lo < tot;
        if (__ballot(reject)) {
            const uint64_t thr = ((uint64_t)0 - tot) % tot;   // uniform; needed rarely
            reject = reject && lo < thr;
        }
        const uint64_t ok = __ballot(!reject && t - hw < kMaxDraws);
        // every lane computes its bounded value, so the accepted lane's can be
        // read from the whole wavefront
        const uint64_t hi = __umul64hi(u, tot);
        const int first = ok ? __builtin_ctzll(ok) : 0;
        const uint32_t vlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)hi, first);
        const uint32_t vhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(hi >> 32), first);
        if (t == hw) {
            draw_sh = ok ? ((uint64_t)vhi << 32) | vlo : UINT64_MAX;
            used_sh = ok ? first + 1 : kMaxDraws;
            pick_sh = -1;
        }
    }
    __syncthreads();
    const uint64_t v = draw_sh;
    if (t < kept && v != UINT64_MAX && cum[t] - w <= v && v < cum[t]) pick_sh = t;
    __syncthreads();
    if (t == 0) {
        const int r = pick_sh;   // -1 only when no draw was accepted
        result[0] = r < 0 ? -1 : i_rk[r];
        result[1] = r;
        result[2] = kept;
        result[3] = (int64_t)total;
        result[4] = r < 0 ? -1 : (int64_t)v;
        result[5] = used_sh;
    }
}

}  // namespace
}  // namespace bs

using namespace bs;

extern "C" int32_t bs_sample_candidates(const int32_t *idx, const int64_t *score, int32_t n,
                                        int32_t mode, uint32_t beta_q16, uint32_t top_p_q16,
                                        uint32_t min_p_q16, uint64_t seed, uint64_t position,
                                        int64_t *result, void *stream) {
    if (!idx || !score || !result) return BS_E_NULL;
    if (n < 1 || n > kMaxCand) return BS_E_SHAPE;
    if (mode != BS_SAMPLE_GREEDY && mode != BS_SAMPLE_DRAW) return BS_E_RANGE;
    if (top_p_q16 < 1 || top_p_q16 > 65536 || min_p_q16 > 65536) return BS_E_RANGE;
    if (((uintptr_t)idx & 3) || ((uintptr_t)score & 7) || ((uintptr_t)result & 7))
        return BS_E_ALIGN;
    // the candidates' wavefronts (kRankWaves for at most 64 candidates) and,
    // when there is room, one more for the draw sources
    const int nc = (n + 63) / 64 * 64;
    const int threads = n <= 64 ? 64 * kRankWaves + 64 : nc + (nc < kMaxCand ? 64 : 0);
    hipLaunchKernelGGL(sample_kernel, dim3(1), dim3(threads), 0, (hipStream_t)stream, idx, score,
                       n, mode, beta_q16, top_p_q16, min_p_q16, seed, position, result);
    BS_LAUNCH_CHECK();
    return BS_OK;
}
