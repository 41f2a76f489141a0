/*
 * Oracle for the pure fractional-LNS reduction of the BitState brief: a
 * plain, slow CPU implementation that follows the algorithm's steps in the
 * page's order.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load, call or link this code.  The
 * product library never includes, links or calls it, and this file includes
 * nothing from the product.  The two share no code.
 *
 * Source: [BS] "BitState / HSDR PoC Technical Brief - v0.5", section 5.2
 * (pure fractional-LNS candidate: count-to-log folding, the kappa+/kappa-
 * pair add, exact cancellation, the balanced 8 -> 4 -> 2 -> 1 reduction, the
 * log-domain scale) and section 7, Phase A (the same steps listed for the
 * standalone correctness phase, "at several internal fractional
 * precisions").
 *
 * Coordinates.  A product state of code k (1..127) has magnitude
 * 2^((k-74)/8) (section 3: code 74 is 1.0, eight codes per octave).  The
 * internal log coordinate keeps f fractional bits of a code unit: the
 * integer L stands for the magnitude 2^((L/2^f - 74)/8), so N = 8*2^f units
 * make one octave.  A value is either zero or (sign, L).
 *
 * Tables: each entry is the real value rounded to the nearest integer.  The
 * real values are irrational except where noted, so no entry is a tie.
 *   lc[n] = round(N*log2 n),              n = 1..128: the fold of a signed
 *                                         population of n identical states
 *                                         (exact for powers of two);
 *   kp[D] = round(N*log2(1 + 2^(-D/N))),  D = 0..n_kp-1: same-sign add,
 *                                         kp[0] = N exactly (doubling);
 *   km[D] = round(N*log2(1 - 2^(-D/N))),  D = 1..n_km-1: opposite-sign add
 *                                         (km[0] is unused: D = 0 cancels).
 * n_kp and n_km are the first D at which the rounded value is 0; from there
 * on the smaller operand no longer moves the larger one.  Entries are
 * computed in binary128 (libquadmath); *min_margin reports how far the least
 * clear entry lies from a rounding tie, in table units.
 *
 * Reduction order of one row (K = 128*T):
 *   1. per Tile128 j (positions 128j..128j+127) and code c = 1..127, the
 *      signed population C_j[c] = sum of (-1)^(S1 xor [t < 0]) over the
 *      positions with code c and t != 0;
 *   2. every C_j[c] != 0 folds to (sign C, c*2^f + lc[|C|]);
 *   3. per phase p, the leaves (j, band b) with c = 8b + p, laid out at index
 *      16j + b (zero where C = 0), reduce by the balanced pairwise tree:
 *      element m of the next level is v[2m] + v[2m+1], an unpaired last
 *      element moves up unchanged (equivalently: zero padding, zero being
 *      the identity);
 *   4. the eight phase aggregates reduce by the same tree, 8 -> 4 -> 2 -> 1;
 *   5. a non-zero result adds round(N*log2 d) for the shared scale d >= 1.
 *
 * Return codes: 0 = ok, -2 = shape error, -3 = value out of range.
 */
#include <quadmath.h>
#include <stdint.h>
#include <stdlib.h>

#define OR_OK 0
#define OR_E_SHAPE (-2)
#define OR_E_RANGE (-3)

/* Round x (not a tie) to the nearest integer and track the margin to a tie. */
static int64_t round_tracked(__float128 x, __float128 *margin)
{
    __float128 v = roundq(x);
    __float128 m = 0.5Q - fabsq(x - v);
    if (m < *margin)
        *margin = m;
    return (int64_t)v;
}

/* N*log2(1 + 2^(-D/N)) and N*log2(1 - 2^(-D/N)) in binary128; 1 - 2^-a is
 * taken as -expm1(-a ln 2) so that small D keeps its digits. */
static __float128 kappa_plus(int64_t D, int64_t N)
{
    __float128 a = (__float128)D / (__float128)N;
    return (__float128)N * log1pq(exp2q(-a)) / M_LN2q;
}

static __float128 kappa_minus(int64_t D, int64_t N)
{
    __float128 a = (__float128)D / (__float128)N;
    return (__float128)N * log2q(-expm1q(-a * M_LN2q));
}

/* Build the three tables for f fractional bits.  lc has 129 entries; kp and
 * km have room for cap entries each.  Returns OR_E_RANGE if f is outside
 * 0..16 or a table does not fit. */
int or_flns_tables(int f, int32_t *lc, int32_t *kp, int64_t cap, int64_t *n_kp, int32_t *km,
                   int64_t *n_km, double *min_margin)
{
    if (f < 0 || f > 16)
        return OR_E_RANGE;
    const int64_t N = (int64_t)8 << f;
    __float128 margin = 0.5Q;
    lc[0] = 0;
    for (int n = 1; n <= 128; n++)
        lc[n] = (int32_t)round_tracked((__float128)N * log2q((__float128)n), &margin);
    int64_t d = 0;
    for (;; d++) {
        if (d >= cap)
            return OR_E_RANGE;
        int64_t v = round_tracked(kappa_plus(d, N), &margin);
        if (v == 0)
            break;
        kp[d] = (int32_t)v;
    }
    *n_kp = d;
    km[0] = 0;
    for (d = 1;; d++) {
        if (d >= cap)
            return OR_E_RANGE;
        int64_t v = round_tracked(kappa_minus(d, N), &margin);
        if (v == 0)
            break;
        km[d] = (int32_t)v;
    }
    *n_km = d;
    *min_margin = (double)margin;
    return OR_OK;
}

/* round(N*log2 d) for the shared positive scale d. */
int or_flns_log_scale(int f, uint32_t d, int64_t *out)
{
    if (f < 0 || f > 16 || d == 0)
        return OR_E_RANGE;
    __float128 margin = 0.5Q;
    *out = round_tracked((__float128)((int64_t)8 << f) * log2q((__float128)d), &margin);
    return OR_OK;
}

/* A log-domain value: zero, or (neg, lam). */
typedef struct {
    int zero;
    int neg;
    int64_t lam;
} lv;

typedef struct {
    const int32_t *kp, *km;
    int64_t n_kp, n_km;
} tabs;

static const lv LV_ZERO = {1, 0, 0};

/* The pair add of section 5.2: order the operands so that a has the larger
 * coordinate, D = a - b; same sign: a + kappa_plus(D); opposite signs:
 * exact zero when D = 0, else a + kappa_minus(D); the sign is a's. */
static lv lv_add(const tabs *tb, lv a, lv b)
{
    if (a.zero)
        return b;
    if (b.zero)
        return a;
    if (b.lam > a.lam) {
        lv t = a;
        a = b;
        b = t;
    }
    int64_t D = a.lam - b.lam;
    lv out = a;
    if (a.neg == b.neg)
        out.lam = a.lam + (D < tb->n_kp ? tb->kp[D] : 0);
    else if (D == 0)
        out = LV_ZERO;
    else
        out.lam = a.lam + (D < tb->n_km ? tb->km[D] : 0);
    return out;
}

/* Balanced pairwise reduction of v[0..n) (overwrites v). */
static lv lv_tree(const tabs *tb, lv *v, int64_t n)
{
    if (n == 0)
        return LV_ZERO;
    while (n > 1) {
        int64_t m = 0;
        for (int64_t i = 0; i + 1 < n; i += 2)
            v[m++] = lv_add(tb, v[i], v[i + 1]);
        if (n & 1)
            v[m++] = v[n - 1];
        n = m;
    }
    return v[0];
}

static int to_sign(lv v) { return v.zero ? 0 : (v.neg ? -1 : 1); }

/* One pair add on explicit operands (sign -1/0/+1, coordinate), for tests. */
int or_flns_add(const int32_t *kp, int64_t n_kp, const int32_t *km, int64_t n_km, int sa,
                int64_t la, int sb, int64_t lb, int *so, int64_t *lo)
{
    tabs tb = {kp, km, n_kp, n_km};
    lv a = {sa == 0, sa < 0, sa == 0 ? 0 : la};
    lv b = {sb == 0, sb < 0, sb == 0 ? 0 : lb};
    lv r = lv_add(&tb, a, b);
    *so = to_sign(r);
    *lo = r.zero ? 0 : r.lam;
    return OR_OK;
}

/* The balanced tree on explicit leaves (signs -1/0/+1, coordinates), for
 * tests. */
int or_flns_tree(const int32_t *kp, int64_t n_kp, const int32_t *km, int64_t n_km,
                 const int *signs, const int64_t *lams, int64_t n, int *so, int64_t *lo)
{
    tabs tb = {kp, km, n_kp, n_km};
    lv *v = malloc(sizeof(lv) * (size_t)(n > 0 ? n : 1));
    if (!v)
        return OR_E_RANGE;
    for (int64_t i = 0; i < n; i++) {
        v[i].zero = signs[i] == 0;
        v[i].neg = signs[i] < 0;
        v[i].lam = signs[i] == 0 ? 0 : lams[i];
    }
    lv r = lv_tree(&tb, v, n);
    free(v);
    *so = to_sign(r);
    *lo = r.zero ? 0 : r.lam;
    return OR_OK;
}

/* The whole row reduction (steps 1-5 above) for every row of t[rows][k]
 * against the LNS8 activation bytes x[k] (bit 7 = S1, bits 6..0 = code).
 * out[2r] = sign of the result (-1, 0, +1), out[2r+1] = its coordinate L
 * (0 for zero). */
int or_flns_gemv(const int8_t *t, const uint8_t *x, int64_t rows, int64_t k, int f,
                 uint32_t scale_d, const int32_t *lc, const int32_t *kp, int64_t n_kp,
                 const int32_t *km, int64_t n_km, int32_t *out)
{
    if (rows < 0 || k <= 0 || k % 128 != 0)
        return OR_E_SHAPE;
    if (f < 0 || f > 16 || scale_d == 0)
        return OR_E_RANGE;
    tabs tb = {kp, km, n_kp, n_km};
    int64_t ld = 0;
    or_flns_log_scale(f, scale_d, &ld);
    const int64_t T = k / 128;
    lv *leaves = malloc(sizeof(lv) * (size_t)(8 * 16 * T));
    if (!leaves)
        return OR_E_RANGE;
    int rc = OR_OK;
    for (int64_t r = 0; r < rows && rc == OR_OK; r++) {
        for (int64_t i = 0; i < 8 * 16 * T; i++)
            leaves[i] = LV_ZERO;
        for (int64_t j = 0; j < T && rc == OR_OK; j++) {
            int pop[128] = {0};
            for (int64_t i = 128 * j; i < 128 * j + 128; i++) {
                int8_t w = t[r * k + i];
                if (w < -1 || w > 1) {
                    rc = OR_E_RANGE;
                    break;
                }
                int code = x[i] & 0x7F;
                if (w == 0 || code == 0)
                    continue;
                pop[code] += ((x[i] >> 7) ^ (w < 0)) ? -1 : 1;
            }
            for (int c = 1; c < 128; c++) {
                if (pop[c] == 0)
                    continue;
                int n = pop[c] < 0 ? -pop[c] : pop[c];
                lv leaf = {0, pop[c] < 0, ((int64_t)c << f) + lc[n]};
                leaves[(c & 7) * 16 * T + 16 * j + (c >> 3)] = leaf;
            }
        }
        if (rc != OR_OK)
            break;
        lv agg[8];
        for (int p = 0; p < 8; p++)
            agg[p] = lv_tree(&tb, leaves + p * 16 * T, 16 * T);
        lv total = lv_tree(&tb, agg, 8);
        if (!total.zero)
            total.lam += ld;
        if (total.lam < INT32_MIN || total.lam > INT32_MAX) {
            rc = OR_E_RANGE;
            break;
        }
        out[2 * r] = to_sign(total);
        out[2 * r + 1] = total.zero ? 0 : (int32_t)total.lam;
    }
    free(leaves);
    return rc;
}
