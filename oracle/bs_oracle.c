/*
 * Oracle for the ternary decode-GEMV hot path: a plain, slow, obviously
 * correct CPU implementation of what the path computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load, call or link this code.  The
 * product library (bit_decode_gemv_amd) never includes, links or calls it,
 * and this file includes nothing from the product.  The two share no code.
 *
 * Sources (the pages this follows; cited by title and section):
 *   [BS]  "BitState / HSDR PoC Technical Brief - v0.5"
 *   [T2]  "[bitnet] T2: lm_head via BITNET_PLANES weight format (WeightForm)
 *          + two-stage top-k decode"
 *   [IE]  "A standalone deterministic integer inference engine for
 *          BitNet-style LLMs, with Ollama interop"
 *
 * Everything here is integer arithmetic (int64), except the fp64 sanity dot
 * of [BS] §7 Phase A.  Loops follow the definitions in the pages' order;
 * there is no blocking, fusion or reordering.  Popcount is a bit loop.
 *
 * Return codes: 0 = ok, -2 = shape error, -3 = value out of range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_E_SHAPE (-2)
#define OR_E_RANGE (-3)

/* floor(v / 2^f), written as a division with an explicit floor step, so that
 * a negative v rounds toward minus infinity ([IE] §3.3: floor division, not
 * truncation; §4.1/§4.2: the per-group arithmetic shift). */
static int64_t floor_shift(int64_t v, int f)
{
    if (f == 0)
        return v;
    int64_t d = (int64_t)1 << f;
    int64_t q = v / d;      /* C division truncates toward zero */
    int64_t r = v % d;
    if (r != 0 && v < 0)
        q -= 1;
    return q;
}

static int popcount64(uint64_t m)
{
    int n = 0;
    for (int i = 0; i < 64; i++)
        if ((m >> i) & 1u)
            n++;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Ternary GEMV: [IE] §4.2 (ternary signed sum, per-group scale and floor)   */
/* ------------------------------------------------------------------------ */

/* Definition form.  t[rows][k] in {-1,0,+1}; scale[rows][k/128] (the
 * per-group integer scale of [IE] §4.3); x[k] int8 ([IE] §4.4).
 * y[r] = sum_g floor( scale[r][g] * sum_{i in g} t[r][i]*x[i] / 2^frac ). */
int or_ternary_gemv_def(const int8_t *t, const int16_t *scale, const int8_t *x,
                        int64_t rows, int64_t k, int frac, int64_t *y)
{
    if (rows < 0 || k < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    if (frac < 0 || frac > 62)
        return OR_E_RANGE;
    int64_t groups = k / 128;
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t g = 0; g < groups; g++) {
            int64_t s = 0;
            for (int64_t i = g * 128; i < g * 128 + 128; i++) {
                int8_t w = t[r * k + i];
                if (w < -1 || w > 1)
                    return OR_E_RANGE;
                s += (int64_t)w * (int64_t)x[i];
            }
            acc += floor_shift(s * (int64_t)scale[r * groups + g], frac);
        }
        y[r] = acc;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed layout ([BS] §4: each ternary row as W_nonzero and W_negative)     */
/* ------------------------------------------------------------------------ */
/*
 * The byte layout is the one the public header of the library declares.  It
 * is implemented here a second time, from that description, so that the
 * library's packer can be checked byte for byte:
 *   rows are padded to a multiple of 64 with all-zero rows;
 *   block (tile, g) = 2048 bytes at offset (tile*G + g)*2048, G = k/128;
 *   bytes [0,1024):    W_nonzero, row 64*tile+j at bytes [16j, 16j+16);
 *   bytes [1024,2048): W_negative, same arrangement;
 *   weight i of group g is bit (i%8) of byte (i/8) of that 16-byte field.
 * Packed scales: int16 at index ((r/16)*G + g)*16 + r%16 (16-row blocks), zero
 * for padding rows.
 */
int64_t or_pad64(int64_t rows) { return (rows + 63) / 64 * 64; }

int or_ternary_pack(const int8_t *t, int64_t rows, int64_t k, uint8_t *planes)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    int64_t groups = k / 128, prow = or_pad64(rows);
    memset(planes, 0, (size_t)(prow * k / 4));
    for (int64_t r = 0; r < rows; r++) {
        int64_t tile = r / 64, j = r % 64;
        for (int64_t i = 0; i < k; i++) {
            int8_t w = t[r * k + i];
            if (w < -1 || w > 1)
                return OR_E_RANGE;
            int64_t g = i / 128, bit = i % 128;
            uint8_t *blk = planes + (tile * groups + g) * 2048;
            if (w != 0)
                blk[16 * j + bit / 8] |= (uint8_t)(1u << (bit % 8));
            if (w == -1)
                blk[1024 + 16 * j + bit / 8] |= (uint8_t)(1u << (bit % 8));
        }
    }
    return OR_OK;
}

int or_scales_pack(const int16_t *scale, int64_t rows, int64_t k, int16_t *packed)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    int64_t groups = k / 128, prow = or_pad64(rows);
    memset(packed, 0, (size_t)(prow * groups) * sizeof(int16_t));
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < groups; g++)
            packed[((r / 16) * groups + g) * 16 + r % 16] = scale[r * groups + g];
    return OR_OK;
}

/* Read one weight back from the packed planes: returns the nz and neg bits. */
static void read_bits(const uint8_t *planes, int64_t k, int64_t r, int64_t i,
                      int *nz, int *neg)
{
    int64_t groups = k / 128, tile = r / 64, j = r % 64, g = i / 128, bit = i % 128;
    const uint8_t *blk = planes + (tile * groups + g) * 2048;
    *nz = (blk[16 * j + bit / 8] >> (bit % 8)) & 1;
    *neg = (blk[1024 + 16 * j + bit / 8] >> (bit % 8)) & 1;
}

/* Unpack; a W_negative bit without its W_nonzero bit is not a ternary code
 * ([BS] §4: W_negative marks the sign of a non-zero weight). */
int or_ternary_unpack(const uint8_t *planes, int64_t rows, int64_t k, int8_t *t)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t i = 0; i < k; i++) {
            int nz, neg;
            read_bits(planes, k, r, i, &nz, &neg);
            if (neg && !nz)
                return OR_E_RANGE;
            t[r * k + i] = (int8_t)(nz ? (neg ? -1 : 1) : 0);
        }
    return OR_OK;
}

/* Masked signed-sum form over the packed planes ([IE] §4.2: the sum over the
 * +1 lanes minus the sum over the -1 lanes; zeros drop out), with the scale
 * read from the packed scales. */
int or_ternary_gemv_masked(const uint8_t *planes, const int16_t *pscale, const int8_t *x,
                           int64_t rows, int64_t k, int frac, int64_t *y)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    if (frac < 0 || frac > 62)
        return OR_E_RANGE;
    int64_t groups = k / 128;
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t g = 0; g < groups; g++) {
            int64_t pos_sum = 0, neg_sum = 0;
            for (int64_t i = g * 128; i < g * 128 + 128; i++) {
                int nz, neg;
                read_bits(planes, k, r, i, &nz, &neg);
                if (nz && !neg)
                    pos_sum += x[i];
                if (neg)
                    neg_sum += x[i];
            }
            int64_t sc = pscale[((r / 16) * groups + g) * 16 + r % 16];
            acc += floor_shift((pos_sum - neg_sum) * sc, frac);
        }
        y[r] = acc;
    }
    return OR_OK;
}

/* Packed BITNET_PLANES layout, as the public header of the library declares
 * it (implemented here a second time so the library's packer can be checked
 * byte for byte).  The four trits of planes 0-3 at one position are stored as
 * the balanced-ternary digit sum D03 = 27*T0 + 9*T1 + 3*T2 + T3 (an int8 in
 * [-40, 40], which determines the four trits), and planes 4-7 as
 * D47 = 27*T4 + 9*T5 + 3*T6 + T7: one byte per position each, the same two
 * bits per trit as two bitplanes.  D03 is tiled for the full-vocabulary scan:
 * rows padded to 64; block (tile, g) = 8192 bytes at offset (tile*G + g)*8192;
 * positions 128g + 16c .. 128g + 16c + 15 of row 64*tile + j at bytes
 * [1024c + 16j, 1024c + 16j + 16) of the block.  D47, read only for candidate
 * rows, is row major: position i of row r at byte r*K + i. */
int or_planes_pack(const int8_t *trits, int64_t V, int64_t K, uint8_t *planes03,
                   uint8_t *planes47)
{
    if (V < 0 || K % 128 != 0)
        return OR_E_SHAPE;
    int64_t groups = K / 128, pv = or_pad64(V);
    memset(planes03, 0, (size_t)(pv * K));
    memset(planes47, 0, (size_t)(V * K));
    for (int64_t r = 0; r < V; r++)
        for (int64_t i = 0; i < K; i++) {
            int d03 = 0, d47 = 0;
            for (int p = 0; p < 8; p++) {
                int8_t w = trits[(r * 8 + p) * K + i];
                if (w < -1 || w > 1)
                    return OR_E_RANGE;
                if (p < 4)
                    d03 = 3 * d03 + w;
                else
                    d47 = 3 * d47 + w;
            }
            int64_t g = i / 128, c = (i % 128) / 16, e = i % 16;
            planes03[((r / 64) * groups + g) * 8192 + 1024 * c + 16 * (r % 64) + e] =
                (uint8_t)(int8_t)d03;
            planes47[r * K + i] = (uint8_t)(int8_t)d47;
        }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Q1_0 weight apply ("A standalone deterministic integer inference engine   */
/* for BitNet-style LLMs", section 4.1): signs in {-1, +1}, one int scale   */
/* per 128-weight group, a per-group floor shift, then the sum over groups. */
/* ------------------------------------------------------------------------ */

/* Definition form: out[r] = sum_g floorshift((sum_i s_i x_i) * scale[r][g], frac). */
int or_q1_gemv_def(const int8_t *s, const int16_t *scale, const int8_t *x, int64_t rows,
                   int64_t k, int frac, int64_t *y)
{
    if (rows < 0 || k < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    if (frac < 0 || frac > 62)
        return OR_E_RANGE;
    int64_t groups = k / 128;
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t g = 0; g < groups; g++) {
            int64_t sum = 0;
            for (int64_t i = g * 128; i < g * 128 + 128; i++) {
                int8_t w = s[r * k + i];
                if (w != 1 && w != -1)
                    return OR_E_RANGE;
                sum += (int64_t)w * (int64_t)x[i];
            }
            acc += floor_shift(sum * (int64_t)scale[r * groups + g], frac);
        }
        y[r] = acc;
    }
    return OR_OK;
}

/* Packed Q1_0 signs, as the public header of the library declares them: one
 * bit per weight, 1 for +1 and 0 for -1, tiled like the ternary W_nonzero
 * plane alone: rows padded to 64; block (tile, g) = 1024 bytes at offset
 * (tile*G + g)*1024; row 64*tile+j at 16j; weight i of the group is bit
 * (i%8) of byte (i/8).  Padding rows are zero. */
int or_q1_pack(const int8_t *s, int64_t rows, int64_t k, uint8_t *bits)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    int64_t groups = k / 128;
    memset(bits, 0, (size_t)(or_pad64(rows) * k / 8));
    for (int64_t r = 0; r < rows; r++)
        for (int64_t i = 0; i < k; i++) {
            int8_t w = s[r * k + i];
            if (w != 1 && w != -1)
                return OR_E_RANGE;
            if (w == 1) {
                int64_t g = i / 128, bit = i % 128;
                bits[((r / 64) * groups + g) * 1024 + 16 * (r % 64) + bit / 8] |=
                    (uint8_t)(1u << (bit % 8));
            }
        }
    return OR_OK;
}

/* The page's masked form, read from the packed bits and packed scales:
 * block_total_g = sum_i x_i over the group (once, shared by every row),
 * pos_sum = sum of x_i over the set bits, signed_sum = 2 pos_sum -
 * block_total. */
int or_q1_gemv_masked(const uint8_t *bits, const int16_t *pscale, const int8_t *x,
                      int64_t rows, int64_t k, int frac, int64_t *y)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    if (frac < 0 || frac > 62)
        return OR_E_RANGE;
    int64_t groups = k / 128;
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t g = 0; g < groups; g++) {
            int64_t block_total = 0, pos_sum = 0;
            const uint8_t *f = bits + ((r / 64) * groups + g) * 1024 + 16 * (r % 64);
            for (int i = 0; i < 128; i++) {
                block_total += x[g * 128 + i];
                if ((f[i / 8] >> (i % 8)) & 1)
                    pos_sum += x[g * 128 + i];
            }
            int64_t sc = pscale[((r / 16) * groups + g) * 16 + r % 16];
            acc += floor_shift((2 * pos_sum - block_total) * sc, frac);
        }
        y[r] = acc;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* LNS8 eight-phase accumulation ([BS] §3, §3.1, §4, §7 Phase A)              */
/* ------------------------------------------------------------------------ */
/*
 * Activation byte: bit 7 = S1 (sign), bits 6..0 = code; code 0 is exact zero.
 * For code k != 0: phase = k & 7 (L3), band = k >> 3 (E4).  A ternary weight
 * of magnitude 1 has log offset 0, so the product state has the activation's
 * code and the sign S1 XOR [t < 0].  A product with t = 0 or code 0 adds
 * nothing.  Accumulators are int64 here; rows*8 outputs, row-major.
 */

/* (i) scalar direct routing: A[L3] += sign * (1 << E4) ([BS] §3.1). */
int or_lns8_direct(const int8_t *t, const uint8_t *x, int64_t rows, int64_t k, int64_t *acc)
{
    if (rows < 0 || k < 0)
        return OR_E_SHAPE;
    for (int64_t r = 0; r < rows; r++) {
        int64_t *A = acc + r * 8;
        for (int p = 0; p < 8; p++)
            A[p] = 0;
        for (int64_t i = 0; i < k; i++) {
            int8_t w = t[r * k + i];
            if (w < -1 || w > 1)
                return OR_E_RANGE;
            int code = x[i] & 0x7F;
            int s1 = x[i] >> 7;
            if (w == 0 || code == 0)
                continue;
            int negative = s1 ^ (w < 0);
            int phase = code & 7, band = code >> 3;
            int64_t payload = (int64_t)1 << band;
            A[phase] += negative ? -payload : payload;
        }
    }
    return OR_OK;
}

/* (ii) Tile64 x 2: each 128-input block is two 64-lane tiles; per tile the
 * L3 bits select a phase mask, E4 gives the payload, S1 the sign ([BS] §3.1,
 * the Tile64x2 procedure; lane i of tile j is position 64j+i). */
int or_lns8_tile64(const int8_t *t, const uint8_t *x, int64_t rows, int64_t k, int64_t *acc)
{
    if (rows < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    for (int64_t r = 0; r < rows; r++) {
        int64_t *A = acc + r * 8;
        for (int p = 0; p < 8; p++)
            A[p] = 0;
        for (int64_t tile = 0; tile < k / 64; tile++) {
            uint64_t phase_mask[8] = {0}, sign_mask = 0;
            for (int lane = 0; lane < 64; lane++) {
                uint8_t b = x[tile * 64 + lane];
                int code = b & 0x7F;
                if (code != 0)
                    phase_mask[code & 7] |= (uint64_t)1 << lane;
                if (b >> 7)
                    sign_mask |= (uint64_t)1 << lane;
            }
            for (int p = 0; p < 8; p++)
                for (int lane = 0; lane < 64; lane++) {
                    if (!((phase_mask[p] >> lane) & 1))
                        continue;
                    int8_t w = t[r * k + tile * 64 + lane];
                    if (w < -1 || w > 1)
                        return OR_E_RANGE;
                    if (w == 0)
                        continue;
                    int e4 = (x[tile * 64 + lane] & 0x7F) >> 3;
                    int negative = (int)((sign_mask >> lane) & 1) ^ (w < 0);
                    int64_t payload = (int64_t)1 << e4;
                    A[p] += negative ? -payload : payload;
                }
        }
    }
    return OR_OK;
}

/* (iii) signed POPCOUNT histogram over all 127 non-zero states, per 64-lane
 * tile ([BS] §4): M = A_s & W_nonzero, PNEG = sign XOR W_negative,
 * C_s = popcount(M) - 2*popcount(M & PNEG); H[phase][band] += C_s; then the
 * per-phase shift/add A[p] = sum_b H[p][b] * 2^b ([BS] §3.1, §5.1).  The
 * optional histogram is returned when hist != NULL (rows*8*16 int64). */
int or_lns8_popcount(const int8_t *t, const uint8_t *x, int64_t rows, int64_t k,
                     int64_t *acc, int64_t *hist)
{
    if (rows < 0 || k % 64 != 0)
        return OR_E_SHAPE;
    for (int64_t r = 0; r < rows; r++) {
        int64_t H[8][16];
        memset(H, 0, sizeof H);
        for (int64_t tile = 0; tile < k / 64; tile++) {
            uint64_t w_nonzero = 0, w_negative = 0, act_sign = 0;
            for (int lane = 0; lane < 64; lane++) {
                int8_t w = t[r * k + tile * 64 + lane];
                if (w < -1 || w > 1)
                    return OR_E_RANGE;
                if (w != 0)
                    w_nonzero |= (uint64_t)1 << lane;
                if (w == -1)
                    w_negative |= (uint64_t)1 << lane;
                if (x[tile * 64 + lane] >> 7)
                    act_sign |= (uint64_t)1 << lane;
            }
            for (int s = 1; s < 128; s++) {
                uint64_t a_s = 0;
                for (int lane = 0; lane < 64; lane++)
                    if ((x[tile * 64 + lane] & 0x7F) == s)
                        a_s |= (uint64_t)1 << lane;
                uint64_t m = a_s & w_nonzero;
                uint64_t pneg = act_sign ^ w_negative;
                int n = popcount64(m);
                int nneg = popcount64(m & pneg);
                H[s & 7][s >> 3] += n - 2 * nneg;
            }
        }
        for (int p = 0; p < 8; p++) {
            int64_t a = 0;
            for (int b = 0; b < 16; b++)
                a += H[p][b] * ((int64_t)1 << b);
            acc[r * 8 + p] = a;
            if (hist)
                for (int b = 0; b < 16; b++)
                    hist[(r * 8 + p) * 16 + b] = H[p][b];
        }
    }
    return OR_OK;
}

/* FP64 direct ternary dot ([BS] §7 Phase A, first item): sum_i t_i * value_i
 * with value = +-2^((code-74)/8) from libm, code 0 = 0.  A sanity reference
 * only; the exact result is the dyadic one. */
int or_lns8_fp64_dot(const int8_t *t, const uint8_t *x, int64_t rows, int64_t k, double *out)
{
    for (int64_t r = 0; r < rows; r++) {
        double s = 0.0;
        for (int64_t i = 0; i < k; i++) {
            int code = x[i] & 0x7F;
            if (code == 0 || t[r * k + i] == 0)
                continue;
            double v = exp2(((double)code - 74.0) / 8.0);
            if (x[i] >> 7)
                v = -v;
            s += (double)t[r * k + i] * v;
        }
        out[r] = s;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* BITNET_PLANES lm_head ([T2]: eight ternary planes weighted 3^-p, stage-1  */
/* scan over planes 0-3, bound-driven exact rescoring with planes 4-7)       */
/* ------------------------------------------------------------------------ */
/*
 * trits[V][8][K] in {-1,0,+1}; row_scale[V] int32; h[K] int8.
 * Scores are kept exact in int64 by scaling by 3^7:
 *   S'(r) = row_scale(r) * sum_{p=0..7} 3^(7-p) * (T_p[r] . h).
 * Order: S' descending, then row index ascending (the lowest-index
 * tie-break of [IE] §3.2 / §3.3).
 */
static int64_t plane_dot(const int8_t *trits, const int8_t *h, int64_t r, int p, int64_t K)
{
    const int8_t *row = trits + (r * 8 + p) * K;
    int64_t s = 0;
    for (int64_t i = 0; i < K; i++)
        s += (int64_t)row[i] * (int64_t)h[i];
    return s;
}

static const int64_t POW3[8] = {1, 3, 9, 27, 81, 243, 729, 2187};

typedef struct {
    int64_t key;
    int64_t idx;
} keyed_row;

/* key descending, then index ascending */
static int cmp_desc(const void *a, const void *b)
{
    const keyed_row *x = (const keyed_row *)a, *y = (const keyed_row *)b;
    if (x->key != y->key)
        return x->key > y->key ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

static int check_trits(const int8_t *trits, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        if (trits[i] < -1 || trits[i] > 1)
            return OR_E_RANGE;
    return OR_OK;
}

/* Brute force: the exact full-precision score of every row, then top-k. */
int or_lmhead_brute(const int8_t *trits, const int32_t *row_scale, const int8_t *h,
                    int64_t V, int64_t K, int top_k, int32_t *top_idx, int64_t *top_score,
                    int64_t *all_scores)
{
    if (V < 1 || K < 1 || top_k < 1 || top_k > V)
        return OR_E_RANGE;
    if (check_trits(trits, V * 8 * K))
        return OR_E_RANGE;
    keyed_row *rows = (keyed_row *)malloc((size_t)V * sizeof(keyed_row));
    if (!rows)
        return OR_E_RANGE;
    for (int64_t r = 0; r < V; r++) {
        int64_t e = 0;
        for (int p = 0; p < 8; p++)
            e += POW3[7 - p] * plane_dot(trits, h, r, p, K);
        rows[r].key = (int64_t)row_scale[r] * e;
        rows[r].idx = r;
        if (all_scores)
            all_scores[r] = rows[r].key;
    }
    qsort(rows, (size_t)V, sizeof(keyed_row), cmp_desc);
    for (int i = 0; i < top_k; i++) {
        top_idx[i] = (int32_t)rows[i].idx;
        top_score[i] = rows[i].key;
    }
    free(rows);
    return OR_OK;
}

/* The two-stage algorithm, step by step ([T2], the BitNetTwoStageDecode
 * comment: stage 1 over planes 0-3, per-row truncation bound
 * rowScale*(sum_{p=4..7} 3^-p)*sum|h|, rescoring of every row whose upper
 * bound reaches the k-th best lower bound, and the maxCandidates cap).
 * In units of 3^-7: stage-1 score S1' = 81*rs*E1 with
 * E1 = sum_{p=0..3} 3^(3-p) T_p.h; bound B' = 40*|rs|*sum|h|;
 * L = S1' - B', U = S1' + B'; L_k = k-th largest L;
 * C = { r : U(r) >= L_k }.  If |C| <= cap every row of C is rescored;
 * otherwise the cap rows of C with the largest S1' (index ascending on ties)
 * are rescored and capped = 1.  Rescoring adds E2 = sum_{p=4..7} 3^(7-p) T_p.h:
 * S' = rs*(81*E1 + E2).  info[0] = |C|, info[1] = capped, info[2] = 1 when
 * the result is certified exact: nothing dropped, or the largest upper bound
 * U among the dropped candidates strictly below the k-th output S'. */
int or_lmhead_two_stage(const int8_t *trits, const int32_t *row_scale, const int8_t *h,
                        int64_t V, int64_t K, int top_k, int cap, int32_t *top_idx,
                        int64_t *top_score, int64_t *info)
{
    if (V < 1 || K < 1 || top_k < 1 || top_k > V || cap < top_k)
        return OR_E_RANGE;
    if (check_trits(trits, V * 8 * K))
        return OR_E_RANGE;
    int64_t habs = 0;
    for (int64_t i = 0; i < K; i++)
        habs += h[i] < 0 ? -(int64_t)h[i] : (int64_t)h[i];

    int64_t *e1 = (int64_t *)malloc((size_t)V * sizeof(int64_t));
    int64_t *s1 = (int64_t *)malloc((size_t)V * sizeof(int64_t));
    int64_t *bnd = (int64_t *)malloc((size_t)V * sizeof(int64_t));
    keyed_row *lower = (keyed_row *)malloc((size_t)V * sizeof(keyed_row));
    keyed_row *cand = (keyed_row *)malloc((size_t)V * sizeof(keyed_row));
    if (!e1 || !s1 || !bnd || !lower || !cand)
        return OR_E_RANGE;

    /* stage 1: planes 0..3 over every row */
    for (int64_t r = 0; r < V; r++) {
        int64_t e = 0;
        for (int p = 0; p < 4; p++)
            e += POW3[3 - p] * plane_dot(trits, h, r, p, K);
        e1[r] = e;
        s1[r] = 81 * (int64_t)row_scale[r] * e;
        int64_t ars = row_scale[r] < 0 ? -(int64_t)row_scale[r] : (int64_t)row_scale[r];
        bnd[r] = 40 * ars * habs;
        lower[r].key = s1[r] - bnd[r];
        lower[r].idx = r;
    }
    /* k-th best lower bound */
    qsort(lower, (size_t)V, sizeof(keyed_row), cmp_desc);
    int64_t lk = lower[top_k - 1].key;

    /* candidates: upper bound reaches L_k */
    int64_t n = 0;
    for (int64_t r = 0; r < V; r++)
        if (s1[r] + bnd[r] >= lk) {
            cand[n].key = s1[r];
            cand[n].idx = r;
            n++;
        }
    int64_t keep = n;
    int capped = 0;
    int64_t umax_dropped = INT64_MIN;
    if (n > cap) {
        qsort(cand, (size_t)n, sizeof(keyed_row), cmp_desc);
        keep = cap;
        capped = 1;
        /* the largest upper bound among the candidates the cap drops */
        for (int64_t c = cap; c < n; c++) {
            int64_t r = cand[c].idx;
            if (s1[r] + bnd[r] > umax_dropped)
                umax_dropped = s1[r] + bnd[r];
        }
    }
    /* rescoring with planes 4..7 */
    for (int64_t c = 0; c < keep; c++) {
        int64_t r = cand[c].idx;
        int64_t e2 = 0;
        for (int p = 4; p < 8; p++)
            e2 += POW3[7 - p] * plane_dot(trits, h, r, p, K);
        cand[c].key = (int64_t)row_scale[r] * (81 * e1[r] + e2);
    }
    qsort(cand, (size_t)keep, sizeof(keyed_row), cmp_desc);
    for (int i = 0; i < top_k; i++) {
        top_idx[i] = (int32_t)cand[i].idx;
        top_score[i] = cand[i].key;
    }
    info[0] = n;
    info[1] = capped;
    /* certificate: the result is the exact top-k when nothing was dropped,
     * or when every dropped row's upper bound U >= S' lies strictly below
     * the k-th output score (then no dropped row can reach the output, ties
     * included) */
    info[2] = !capped || umax_dropped < top_score[top_k - 1];
    free(e1);
    free(s1);
    free(bnd);
    free(lower);
    free(cand);
    return OR_OK;
}

/* The stage-1 quantities of every row, for invariant checks in the tests:
 * s1[r] = S1'(r), bound[r] = B'(r). */
int or_lmhead_stage1(const int8_t *trits, const int32_t *row_scale, const int8_t *h,
                     int64_t V, int64_t K, int64_t *s1, int64_t *bound)
{
    int64_t habs = 0;
    for (int64_t i = 0; i < K; i++)
        habs += h[i] < 0 ? -(int64_t)h[i] : (int64_t)h[i];
    for (int64_t r = 0; r < V; r++) {
        int64_t e = 0;
        for (int p = 0; p < 4; p++)
            e += POW3[3 - p] * plane_dot(trits, h, r, p, K);
        s1[r] = 81 * (int64_t)row_scale[r] * e;
        int64_t ars = row_scale[r] < 0 ? -(int64_t)row_scale[r] : (int64_t)row_scale[r];
        bound[r] = 40 * ars * habs;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Row-parallel forms (the benchmark's all-core CPU baseline)                */
/* ------------------------------------------------------------------------ */
/*
 * The definition forms above with their rows shared out over OpenMP threads
 * (the library is built with -fopenmp).  Each row runs the same loop, in the
 * same order, as the single-thread form, and rows are independent, so the
 * results are identical; the input checks run first because a parallel loop
 * cannot return early.  Only the benchmark's CPU-baseline leg and the test
 * that compares them with the single-thread forms call these.
 */
#ifdef _OPENMP
#include <omp.h>
#endif

void or_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int or_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int trits_ok(const int8_t *t, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        if (t[i] < -1 || t[i] > 1)
            return 0;
    return 1;
}

int or_ternary_gemv_def_mt(const int8_t *t, const int16_t *scale, const int8_t *x,
                           int64_t rows, int64_t k, int frac, int64_t *y)
{
    if (rows < 0 || k < 0 || k % 128 != 0)
        return OR_E_SHAPE;
    if (frac < 0 || frac > 62)
        return OR_E_RANGE;
    if (!trits_ok(t, rows * k))
        return OR_E_RANGE;
    int64_t groups = k / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t g = 0; g < groups; g++) {
            int64_t s = 0;
            for (int64_t i = g * 128; i < g * 128 + 128; i++)
                s += (int64_t)t[r * k + i] * (int64_t)x[i];
            acc += floor_shift(s * (int64_t)scale[r * groups + g], frac);
        }
        y[r] = acc;
    }
    return OR_OK;
}

int or_lns8_direct_mt(const int8_t *t, const uint8_t *x, int64_t rows, int64_t k, int64_t *acc)
{
    if (rows < 0 || k < 0)
        return OR_E_SHAPE;
    if (!trits_ok(t, rows * k))
        return OR_E_RANGE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        int64_t *A = acc + r * 8;
        for (int p = 0; p < 8; p++)
            A[p] = 0;
        for (int64_t i = 0; i < k; i++) {
            int8_t w = t[r * k + i];
            int code = x[i] & 0x7F;
            int s1 = x[i] >> 7;
            if (w == 0 || code == 0)
                continue;
            int negative = s1 ^ (w < 0);
            int phase = code & 7, band = code >> 3;
            int64_t payload = (int64_t)1 << band;
            A[phase] += negative ? -payload : payload;
        }
    }
    return OR_OK;
}

/* Brute force with the per-row scores on all threads; the final sort is the
 * single-thread form's. */
int or_lmhead_brute_mt(const int8_t *trits, const int32_t *row_scale, const int8_t *h,
                       int64_t V, int64_t K, int top_k, int32_t *top_idx, int64_t *top_score)
{
    if (V < 1 || K < 1 || top_k < 1 || top_k > V)
        return OR_E_RANGE;
    if (!trits_ok(trits, V * 8 * K))
        return OR_E_RANGE;
    keyed_row *rows = (keyed_row *)malloc((size_t)V * sizeof(keyed_row));
    if (!rows)
        return OR_E_RANGE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < V; r++) {
        int64_t e = 0;
        for (int p = 0; p < 8; p++)
            e += POW3[7 - p] * plane_dot(trits, h, r, p, K);
        rows[r].key = (int64_t)row_scale[r] * e;
        rows[r].idx = r;
    }
    qsort(rows, (size_t)V, sizeof(keyed_row), cmp_desc);
    for (int i = 0; i < top_k; i++) {
        top_idx[i] = (int32_t)rows[i].idx;
        top_score[i] = rows[i].key;
    }
    free(rows);
    return OR_OK;
}
