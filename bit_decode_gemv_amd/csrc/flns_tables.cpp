// Host-side tables of the pure fractional-LNS reduction ("BitState / HSDR
// PoC Technical Brief - v0.5", section 5.2: count-to-log folding and the
// kappa+/kappa- pair-add corrections).
//
// With N = 8*2^f units per octave, every entry is a real value rounded to
// the nearest integer:
//   fold[n] = N*log2 n                    n = 1..128
//   kp[D]   = N*log2(1 + 2^(-D/N))        same-sign add, kp[0] = N
//   km[D]   = N*log2(1 - 2^(-D/N))        opposite-sign add, D >= 1
// each table ending at the first D whose value rounds to 0 (both decrease in
// magnitude with D).  The values are evaluated in x87 extended precision
// (64-bit significand): the largest magnitude at f = 12 is about 5.1e5, so
// the evaluation error is below 1e-12 units, and an entry is accepted only
// if it lies more than 1e-9 units away from a rounding tie.
#include <math.h>
#include <string.h>

#include "bs_internal.h"
#include "flns_layout.h"

namespace bs {
namespace {

constexpr long double kTieGuard = 1e-9L;

long double ln2() { return logl(2.0L); }

long double kp_real(int64_t D, int64_t N) {
    return (long double)N * log1pl(exp2l(-(long double)D / (long double)N)) / ln2();
}

// 1 - 2^-a taken as -expm1(-a ln 2), so a small D keeps its digits.
long double km_real(int64_t D, int64_t N) {
    return (long double)N * log2l(-expm1l(-((long double)D / (long double)N) * ln2()));
}

bool round_checked(long double v, int64_t *out) {
    const long double r = roundl(v);
    if (fabsl(fabsl(v - r) - 0.5L) < kTieGuard) return false;
    *out = (int64_t)r;
    return true;
}

// First D >= d_min at which round(f(D)) == 0, starting from an estimate of
// the crossing: |f(D)| < 1/2 from D ~ -N*log2(c) on.
template <typename F>
int64_t first_zero(F f, int64_t d_min, long double estimate) {
    int64_t d = (int64_t)floorl(estimate) - 3;
    if (d < d_min) d = d_min;
    int64_t v = 0;
    while (round_checked(f(d), &v) && v == 0 && d > d_min) --d;   // estimate too high
    for (;; ++d) {
        if (!round_checked(f(d), &v)) return -1;
        if (v == 0) return d;
    }
}

}  // namespace

bool flns_sizes(int f, FlnsSizes *s) {
    if (f < 0 || f > BS_FLNS_MAX_FRAC) return false;
    const int64_t N = (int64_t)8 << f;
    const long double h = ln2() / (2.0L * (long double)N);
    // kp(D) < 1/2  <=>  2^(-D/N) < 2^(1/2N) - 1;  |km(D)| < 1/2  <=>  2^(-D/N) < 1 - 2^(-1/2N)
    const int64_t n_kp = first_zero([N](int64_t D) { return kp_real(D, N); }, 0,
                                    -(long double)N * log2l(expm1l(h)));
    const int64_t n_km = first_zero([N](int64_t D) { return km_real(D, N); }, 1,
                                    -(long double)N * log2l(-expm1l(-h)));
    if (n_kp < 0 || n_km < 0) return false;
    s->n_kp = n_kp;
    s->n_km = n_km;
    s->stride = (n_kp > n_km ? n_kp : n_km) + 1;
    s->elem = f <= kFlnsSmallMaxFrac ? 2 : 4;
    s->bytes = (int64_t)align_up((size_t)(kFlnsCorrOff + 2 * s->stride * s->elem), 16);
    return true;
}

bool flns_log_scale(int f, uint32_t d, int64_t *out) {
    if (f < 0 || f > BS_FLNS_MAX_FRAC || d == 0) return false;
    return round_checked((long double)((int64_t)8 << f) * log2l((long double)d), out);
}

}  // namespace bs

using namespace bs;

extern "C" int64_t bs_flns_table_bytes(int32_t frac_bits) {
    FlnsSizes s;
    return flns_sizes(frac_bits, &s) ? s.bytes : 0;
}

extern "C" int32_t bs_flns_table_build(int32_t frac_bits, void *table, int64_t table_bytes) {
    if (!table) return BS_E_NULL;
    FlnsSizes s;
    if (!flns_sizes(frac_bits, &s)) return BS_E_RANGE;
    if (table_bytes != s.bytes) return BS_E_SHAPE;
    uint8_t *base = static_cast<uint8_t *>(table);
    memset(base, 0, (size_t)s.bytes);
    int32_t hdr[16] = {kFlnsMagic, frac_bits, (int32_t)s.n_kp, (int32_t)s.n_km, (int32_t)s.elem,
                       (int32_t)s.bytes, (int32_t)s.stride};
    memcpy(base, hdr, sizeof hdr);
    const int64_t N = (int64_t)8 << frac_bits;
    int32_t fold[kFlnsFoldSlots] = {0};
    for (int n = 1; n <= 128; ++n) {
        int64_t v;
        if (!round_checked((long double)N * log2l((long double)n), &v)) return BS_E_RANGE;
        fold[n] = (int32_t)v;
    }
    memcpy(base + kFlnsHdrBytes, fold, sizeof fold);
    uint8_t *corr = base + kFlnsCorrOff;
    auto put = [&](int64_t i, int64_t v) {
        if (s.elem == 2) {
            const int16_t e = (int16_t)v;
            memcpy(corr + 2 * i, &e, 2);
        } else {
            const int32_t e = (int32_t)v;
            memcpy(corr + 4 * i, &e, 4);
        }
    };
    for (int64_t D = 0; D < s.n_kp; ++D) {
        int64_t v;
        if (!round_checked(kp_real(D, N), &v) || v == 0) return BS_E_RANGE;
        put(D, v);
    }
    for (int64_t D = 1; D < s.n_km; ++D) {
        int64_t v;
        if (!round_checked(km_real(D, N), &v) || v == 0) return BS_E_RANGE;
        put(s.stride + D, v);
    }
    return BS_OK;
}
