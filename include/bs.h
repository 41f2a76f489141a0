/*
 * bs.h -- C ABI of the MI355X (gfx950) ternary decode-GEMV library.
 *
 * Pages cited (by title and section):
 *   [BS] "BitState / HSDR PoC Technical Brief - v0.5"
 *   [T2] "[bitnet] T2: lm_head via BITNET_PLANES weight format (WeightForm)
 *         + two-stage top-k decode"
 *   [IE] "A standalone deterministic integer inference engine for
 *         BitNet-style LLMs, with Ollama interop"
 *
 * Conventions
 *   - Every entry point returns int32_t status: BS_OK (0) or a negative
 *     BS_E_* code.  Nothing else crosses the ABI; no exceptions.
 *   - Arguments are validated on the host before any HIP call.  A failed
 *     validation leaves every output untouched and enqueues nothing.
 *   - Codec functions (bs_*pack*, bs_*unpack*) work on HOST memory,
 *     synchronously, and never touch the GPU.
 *   - Device entry points take DEVICE pointers owned by the caller, enqueue
 *     their kernels on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream) and return after enqueueing.  Results are valid once
 *     the stream reaches that point.  The library never allocates or frees
 *     device memory; entry points that need scratch take the caller's
 *     `workspace` (bs_lmhead_planes_topk_noalloc uses a device array of the
 *     library's own instead).
 *   - Fail-loud overflow contract ([IE] section 3.4): a call whose shapes
 *     would let an intermediate exceed its integer type returns
 *     BS_E_OVERFLOW instead of wrapping.
 *   - All sums are integer, so results are byte-identical whatever the
 *     launch geometry, split or atomic order ([IE] section 3.2).
 */
#ifndef BS_H
#define BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BS_ABI_VERSION 2   /* 2: lm_head info carries the exactness certificate */

enum {
    BS_OK = 0,
    BS_E_NULL = -1,      /* a required pointer is NULL                      */
    BS_E_SHAPE = -2,     /* a size is non-positive or not a multiple of 128 */
    BS_E_RANGE = -3,     /* a value is outside its documented range         */
    BS_E_OVERFLOW = -4,  /* the static bound of the integer types is broken */
    BS_E_HIP = -5,       /* a HIP call or kernel launch failed              */
    BS_E_WORKSPACE = -6, /* workspace NULL, too small or misaligned         */
    BS_E_ALIGN = -7      /* a device pointer lacks its documented alignment */
};

int32_t bs_abi_version(void);
/* Static string describing a status code (never NULL). */
const char *bs_status_str(int32_t status);

/* ======================================================================== */
/* Ternary weight codec ([BS] section 4: each ternary row as two bitplanes,  */
/* W_nonzero and W_negative; [IE] sections 4.2-4.3: 128-weight groups with  */
/* one integer scale each).  0.25 byte per weight + 2 bytes per group.       */
/* ======================================================================== */
/*
 * Packed planes layout ("tiled64"), for `rows` x `k` trits, k % 128 == 0:
 *   rows are padded to R = ceil(rows/64)*64 with all-zero rows;
 *   G = k/128 groups; block (tile, g) is 2048 bytes at byte offset
 *   (tile*G + g)*2048, tile in [0, R/64);
 *   block bytes [0, 1024):    W_nonzero, row 64*tile+j at bytes [16j, 16j+16)
 *   block bytes [1024, 2048): W_negative, same arrangement;
 *   weight 128*g + i of the row is bit (i % 8) of byte (i / 8) of its
 *   16-byte field.  W_negative is a subset of W_nonzero.
 * Total: R*k/4 bytes.  The 64-row tile is one wavefront: lane j streams row
 * j with 16-byte loads and the wavefront reads 1 KB contiguous per plane.
 *
 * Packed scales layout: int16 at index ((r/16)*G + g)*16 + r%16 holds the
 * scale of row r, group g: 16-row blocks, so the 128-byte line of one block
 * holds four of its groups and no two 16-row workgroups share a line.
 * Padding rows hold 0.  Total R*G int16.
 */

/* Bytes of packed planes (R*k/4) or a negative BS_E_* code. */
int64_t bs_ternary_planes_bytes(int64_t rows, int64_t k);
/* Number of int16 packed scales (R*k/128) or a negative BS_E_* code. */
int64_t bs_ternary_scales_count(int64_t rows, int64_t k);

/* t[rows][k] row-major, each in {-1,0,+1} (else BS_E_RANGE, output partly
 * written).  planes: bs_ternary_planes_bytes(rows,k) bytes, fully written. */
int32_t bs_ternary_pack(const int8_t *t, int64_t rows, int64_t k, uint8_t *planes);
/* Inverse of bs_ternary_pack.  A W_negative bit without its W_nonzero bit
 * is not a ternary code: BS_E_RANGE. */
int32_t bs_ternary_unpack(const uint8_t *planes, int64_t rows, int64_t k, int8_t *t);
/* scales[rows][k/128] row-major -> packed[R*k/128] (layout above). */
int32_t bs_ternary_pack_scales(const int16_t *scales, int64_t rows, int64_t k,
                               int16_t *packed);

/* ======================================================================== */
/* bs_ternary_gemv -- exact batch-1 ternary GEMV ([IE] section 4.2)          */
/* ======================================================================== */
/*
 *   y[r] = sum_{g} floor( scale[r][g] * s[r][g] / 2^frac ),
 *   s[r][g] = sum_{i in group g, t=+1} x[i] - sum_{i in group g, t=-1} x[i]
 * (the masked signed sum: zero weights drop out), computed exactly:
 * |s| <= 2^14, |scale*s| <= 2^29 (int32), y accumulated in int64.
 *
 *   planes  device, packed planes (layout above), all
 *           bs_ternary_planes_bytes of them (the kernels read the padding
 *           rows of the last tile), 16-byte aligned
 *   scales  device, packed int16 scales (layout above), all
 *           bs_ternary_scales_count of them, 2-byte aligned
 *   x       device, int8[k] activations (two's complement, -128 allowed),
 *           8-byte aligned
 *   rows    1 .. 2^31 - 64 (else BS_E_SHAPE);  k >= 128, k % 128 == 0
 *           (else BS_E_SHAPE), k <= 2^24 (else BS_E_OVERFLOW)
 *   frac    0..62: fractional bits of the fixed-point scale; the floor is
 *           applied per group, before the sum over groups
 *   y       device, int64[rows], overwritten, 8-byte aligned
 *   stream  hipStream_t (as void*) the kernel is enqueued on
 * No scratch memory: each workgroup owns complete rows.
 * Errors: BS_E_NULL, BS_E_SHAPE, BS_E_OVERFLOW (k), BS_E_RANGE (frac),
 *   BS_E_ALIGN, BS_E_HIP.
 */
int32_t bs_ternary_gemv(const uint8_t *planes, const int16_t *scales, const int8_t *x,
                        int64_t rows, int64_t k, int32_t frac, int64_t *y, void *stream);

/*
 * bs_ternary_gemv_acc -- y += W x with the arithmetic of bs_ternary_gemv (the
 * same planes, scales, x, frac and per-group floor): the residual-stream
 * update of a decoder layer, whose output projections add into the running
 * hidden state.  Each workgroup adds its rows' partial sums over a run of
 * groups to y with int64 atomics; integer addition is associative ([IE]
 * section 3.2), so the result is exact and independent of their order.
 *   y  device int64[rows], 8-byte aligned, read and written; the caller keeps
 *      |y + W x| below 2^63 ([IE] section 3.4: the bound is the caller's,
 *      who holds the accumulator)
 * Concurrent calls on one y are allowed (they add); other readers of y must
 * be ordered after the call.  Errors as bs_ternary_gemv.
 */
int32_t bs_ternary_gemv_acc(const uint8_t *planes, const int16_t *scales, const int8_t *x,
                            int64_t rows, int64_t k, int32_t frac, int64_t *y, void *stream);


/* ======================================================================== */
/* bs_q1_gemv -- Q1_0 weight apply ([IE] section 4.1)                        */
/* ======================================================================== */
/*
 * Weights are signs s in {-1, +1}, one bit each (1 = +1, 0 = -1), packed like
 * the ternary W_nonzero plane alone: rows padded to R = ceil(rows/64)*64;
 * block (tile, g) = 1024 bytes at offset (tile*G + g)*1024, row 64*tile+j at
 * 16j, weight i of the group bit (i%8) of byte (i/8).  R*k/8 bytes.  Scales
 * use the packed-scale layout of bs_ternary_gemv (bs_ternary_pack_scales).
 *   y[r] = sum_g floor( scale[r][g] * (2 * pos[r][g] - total[g]) / 2^frac ),
 *   pos[r][g] = sum of x over the group's positions with s = +1,
 *   total[g]  = sum of x over the group (shared by every row).
 * Arguments, alignment, limits and errors as for bs_ternary_gemv.
 */
int64_t bs_q1_planes_bytes(int64_t rows, int64_t k);
/* signs[rows][k] in {-1, +1} (host) -> bits[R*k/8]; any other value gives
 * BS_E_RANGE. */
int32_t bs_q1_pack(const int8_t *signs, int64_t rows, int64_t k, uint8_t *bits);
int32_t bs_q1_gemv(const uint8_t *bits, const int16_t *scales, const int8_t *x, int64_t rows,
                   int64_t k, int32_t frac, int64_t *y, void *stream);

/* ======================================================================== */
/* bs_lns8_phase_gemv -- BitState LNS8 eight-phase GEMV ([BS] sections 3-4)  */
/* ======================================================================== */
/*
 * Weights: ternary, packed exactly as for bs_ternary_gemv (no scales: the
 * shared scale stays outside the reduction, the factorised variant of [BS]
 * section 4).  Activations x_lns8[k]: bit 7 = S1 (sign), bits 6..3 = E4
 * (band 0..15), bits 2..0 = L3 (phase 0..7); code = bits 6..0, code 0 is an
 * exact zero ([BS] section 3).  The product of a weight t = +-1 (log offset
 * 0, code 74 = 1.0) with code c has code c and sign S1 XOR [t < 0]; t = 0 or
 * c = 0 gives no product.  Each product adds +-(1 << E4) to A[r][L3]
 * ([BS] section 3.1), so
 *   acc[r][p] = sum over products with phase p of sign * 2^band   (int32)
 *   s[r]      = 2^-9 * sum_p acc[r][p] * F[p],  F[p] = 2^((p-2)/8)
 * s is the exact value of that sum over the binary64 F[p] (each F[p]
 * correctly rounded), rounded once to binary64.
 *
 *   path    BS_LNS8_DIRECT (0): per-product routing into A[L3];
 *           BS_LNS8_POPCOUNT (1): per 64-position unit and active state s
 *           (A_s: the unit's positions holding code s),
 *           C_s = popcount(A_s & W_nonzero) - 2*popcount(A_s & W_nonzero &
 *           (sign XOR W_negative)), H[phase][band] += C_s,
 *           A[p] = sum_b H[p][b] * 2^b ([BS] sections 3.1, 4);
 *           BS_LNS8_MATRIX (2): the direct routing as a contraction on the
 *           int8 matrix instructions, A[p] = sum_k t_k X[k][(p, 0)] + 256 *
 *           sum_k t_k X[k][(p, 1)] with t_k the product sign and X[k][(p, h)]
 *           = 2^(E4 & 7) where position k has phase p, E4 >> 3 = h and a
 *           nonzero code.
 *           All three paths return identical bytes.
 *   rows    1 .. 2^31 - 64;  k >= 128, k % 128 == 0, k <= 65408 (|A| <= k*2^15 must
 *           fit int32, else BS_E_OVERFLOW)
 *   planes  device, 16-byte aligned; x_lns8 device uint8[k], 4-byte aligned
 *   acc     device int32[rows][8], overwritten, 4-byte aligned
 *   s       device double[rows], or NULL to skip the materialisation
 *   workspace  device scratch of at least bs_lns8_workspace_bytes(rows, k)
 *           bytes, 256-byte aligned, caller-owned (the same size for every
 *           path): when DIRECT splits K over several workgroups, a counter
 *           per 64-row tile and the partial accumulators; POPCOUNT and
 *           MATRIX do not touch it.  Zero it before its first use; every call leaves it
 *           zero again, so one workspace serves calls of any shape ordered
 *           on one stream.  Calls that may overlap need separate
 *           workspaces.
 * Errors: BS_E_NULL, BS_E_SHAPE, BS_E_OVERFLOW (k), BS_E_RANGE (path),
 *   BS_E_ALIGN, BS_E_WORKSPACE, BS_E_HIP.
 */
#define BS_LNS8_DIRECT 0
#define BS_LNS8_POPCOUNT 1
#define BS_LNS8_MATRIX 2
size_t bs_lns8_workspace_bytes(int64_t rows, int64_t k);
int32_t bs_lns8_phase_gemv(const uint8_t *planes, const uint8_t *x_lns8, int64_t rows,
                           int64_t k, int32_t path, int32_t *acc, double *s,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ======================================================================== */
/* bs_flns_phase_gemv -- pure fractional-LNS reduction ([BS] section 5.2)    */
/* ======================================================================== */
/*
 * The same products as bs_lns8_phase_gemv (ternary planes x LNS8 bytes),
 * reduced without a linear accumulator ([BS] section 5.2, section 7 Phase A):
 *
 * Coordinates.  Code k stands for 2^((k-74)/8).  The internal coordinate
 * keeps frac_bits = f fractional bits of a code unit: the integer L stands
 * for 2^((L/2^f - 74)/8), N = 8*2^f units per octave.  A value is zero or
 * (sign, L).
 * Steps, per row:
 *   1. per Tile128 j (positions 128j..128j+127, = group j) and code c, the
 *      signed state population C_j[c] = sum of (-1)^(S1 xor [t < 0]) over the
 *      positions with code c and t != 0 (|C| <= 128);
 *   2. fold: C != 0 becomes (sign C, c*2^f + round(N*log2|C|));
 *   3. per phase p, the leaves (j, band b), c = 8b + p, at index 16j + b
 *      (zero where C = 0) reduce by a balanced pairwise tree (element m of
 *      a level is the sum of elements 2m and 2m+1 of the level below, an
 *      unpaired last element moves up unchanged); every sum is the pair
 *      add of [BS] section 5.2: with a the operand of larger L and
 *      D = L_a - L_b, same signs give L_a + round(N*log2(1 + 2^(-D/N))),
 *      opposite signs give exact zero for D = 0, else
 *      L_a + round(N*log2(1 - 2^(-D/N))); the sign is a's; zero is the
 *      identity;
 *   4. the eight phase results reduce by the same tree (8 -> 4 -> 2 -> 1);
 *   5. a non-zero result adds round(N*log2 d) for the shared scale d.
 * Each rounding is to the nearest integer; none of the rounded real values
 * is a tie.  The corrections come from tables built on the host
 * (bs_flns_table_build) and copied to the device by the caller.
 *
 *   planes, x_lns8, rows, k  as bs_lns8_phase_gemv (k <= 65408)
 *   frac_bits  f, 0..BS_FLNS_MAX_FRAC
 *   scale_d    shared positive scale d >= 1 (1 = none)
 *   table      device copy of the blob from bs_flns_table_build(frac_bits),
 *              16-byte aligned; table_bytes = bs_flns_table_bytes(frac_bits)
 *              (the size identifies f: a table for another f is rejected)
 *   out        device int32[rows][2], 8-byte aligned: (sign, L) per row,
 *              sign -1 / 0 / +1, L = 0 when the result is zero
 *   workspace  device memory of at least bs_flns_workspace_bytes(rows, k)
 *              bytes (256), 256-byte aligned, caller-owned: reserved by the
 *              interface; the reduction runs in one launch per call with
 *              every partial result on chip, so it is never read or
 *              written.
 * Errors: BS_E_NULL, BS_E_SHAPE, BS_E_OVERFLOW (k), BS_E_RANGE (frac_bits,
 *   scale_d = 0, table_bytes not that of frac_bits), BS_E_ALIGN,
 *   BS_E_WORKSPACE, BS_E_HIP.
 */
#define BS_FLNS_MAX_FRAC 12

/* Bytes of the table blob for frac_bits, or 0 when frac_bits is outside
 * 0..BS_FLNS_MAX_FRAC.  Host only. */
int64_t bs_flns_table_bytes(int32_t frac_bits);

/* Fill the blob in host memory: the fold table round(N*log2 n), n = 1..128,
 * and the pair-add corrections round(N*log2(1 +- 2^(-D/N))) up to the first
 * D where they round to 0.  Host only, synchronous.  Errors: BS_E_NULL,
 * BS_E_RANGE (frac_bits; an entry this host cannot round unambiguously),
 * BS_E_SHAPE (table_bytes != bs_flns_table_bytes(frac_bits)). */
int32_t bs_flns_table_build(int32_t frac_bits, void *table, int64_t table_bytes);

size_t bs_flns_workspace_bytes(int64_t rows, int64_t k);
int32_t bs_flns_phase_gemv(const uint8_t *planes, const uint8_t *x_lns8, int64_t rows,
                           int64_t k, int32_t frac_bits, uint32_t scale_d, const void *table,
                           int64_t table_bytes, int32_t *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ======================================================================== */
/* BITNET_PLANES lm_head ([T2])                                              */
/* ======================================================================== */
/*
 * Each of `vocab` rows holds eight ternary planes T_0..T_7 over `dim`
 * positions, weighted 3^-p, and an int32 row scale.  Scores are exact int64
 * in units of 3^-7:
 *   S'(r) = row_scale[r] * sum_{p=0..7} 3^(7-p) * (T_p[r] . h)
 *
 * Packed layouts (dim % 128 == 0, G = dim/128).  The four trits of planes
 * 0-3 at one position are stored as one int8, the balanced-ternary digit sum
 * D03 = 27*T_0 + 9*T_1 + 3*T_2 + T_3 in [-40, 40] (which determines them),
 * and planes 4-7 likewise as D47 = 27*T_4 + 9*T_5 + 3*T_6 + T_7: one byte
 * per position for each half, as many bits as two bitplanes per plane.
 *   planes03 (D03, tiled for the full-vocabulary scan): rows padded to
 *     R = ceil(vocab/64)*64; block (tile, g) is 8192 bytes at offset
 *     (tile*G + g)*8192; positions 128g + 16c .. 128g + 16c + 15 of row
 *     64*tile + j are the 16 bytes at block offset 1024c + 16j (c = 0..7).
 *     R*dim bytes; padding rows are zero.
 *   planes47 (D47, row-major, gathered for candidate rows only): position i
 *     of row r at byte r*dim + i.  vocab*dim bytes.
 *
 * trits[vocab][8][dim] row-major, each in {-1,0,+1}.
 */
int64_t bs_planes03_bytes(int64_t vocab, int64_t dim);
int64_t bs_planes47_bytes(int64_t vocab, int64_t dim);
int32_t bs_planes_pack(const int8_t *trits, int64_t vocab, int64_t dim,
                       uint8_t *planes03, uint8_t *planes47);

/*
 * bs_lmhead_planes_topk -- two-stage exact top-k ([T2], BitNetTwoStageDecode):
 *   stage 1, every row:  E1 = sum_{p=0..3} 3^(3-p) (T_p . h),
 *                        S1' = 81 * row_scale * E1,
 *                        B'  = 40 * |row_scale| * sum|h|   (the page's
 *                        truncation bound rowScale*(sum_{p=4..7}3^-p)*sum|h|
 *                        in units of 3^-7), L = S1' - B', U = S1' + B';
 *   L_k = the top_k-th largest L;  C = { r : U(r) >= L_k };
 *   if |C| <= max_candidates every row of C is rescored (the result is then
 *   the exact top-k); otherwise the max_candidates rows of C with the largest
 *   S1' (lowest index first on ties) are rescored and info[1] = 1;
 *   rescoring: E2 = sum_{p=4..7} 3^(7-p) (T_p . h), S' = row_scale*(81*E1+E2);
 *   output: the top_k rescored rows by S' descending, lowest index first on
 *   ties ([IE] sections 3.2-3.3).
 *
 *   planes03, planes47 (16-byte aligned), row_scale (int32[vocab], 4-byte
 *     aligned), h (int8[dim], 8-byte aligned): device
 *   1 <= vocab <= 2^31 - 1024; dim >= 128, dim % 128 == 0, dim <= 10112
 *     (|S'| <= 2^31 * 3280 * 128 * dim must fit int64, else BS_E_OVERFLOW)
 *   1 <= top_k <= max_candidates, top_k <= vocab, max_candidates <= 4096
 *   top_idx int32[top_k], top_score int64[top_k]: device, overwritten
 *     (4- and 8-byte aligned)
 *   info    device int32[3]: info[0] = |C|, info[1] = 1 if the cap engaged,
 *           info[2] = 1 if the result is certified to be the exact top_k:
 *           nothing was dropped, or every candidate the cap dropped has an
 *           upper bound U strictly below the top_k-th output score (a
 *           dropped row's S' <= U, so it can neither pass nor tie the
 *           output); 0 means not certified, not wrong
 *   workspace  device scratch of bs_lmhead_workspace_bytes(...) bytes,
 *     256-byte aligned, caller-owned.  Every byte of it is written before it
 *     is read, so it needs no initialisation and one workspace serves calls
 *     of any shapes ordered on one stream.  It is not shared with other entry
 *     points or overlapping calls.
 * Errors: BS_E_NULL, BS_E_SHAPE, BS_E_OVERFLOW (dim), BS_E_RANGE (top_k,
 *   max_candidates), BS_E_ALIGN, BS_E_WORKSPACE, BS_E_HIP.
 */
size_t bs_lmhead_workspace_bytes(int64_t vocab, int64_t dim, int32_t top_k,
                                 int32_t max_candidates);
int32_t bs_lmhead_planes_topk(const uint8_t *planes03, const uint8_t *planes47,
                              const int32_t *row_scale, const int8_t *h, int64_t vocab,
                              int64_t dim, int32_t top_k, int32_t max_candidates,
                              int32_t *top_idx, int64_t *top_score, int32_t *info,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * bs_lmhead_planes_topk_noalloc -- bs_lmhead_planes_topk for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, arguments,
 * outputs and errors, without the workspace arguments.  Its scratch is a
 * file-scope device array of the library, sized for
 * vocab <= BS_LMHEAD_NOALLOC_MAX_VOCAB (17,916,160 bytes; each GPU the library
 * runs on holds its own copy until the process ends).  The call allocates
 * nothing: no hipMalloc, hipFree or allocating library routine.  Its first
 * call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress; a HIP failure there gives BS_E_HIP).  Every byte of
 * the scratch is written before it is read, so it needs no clearing and the
 * contents left by an earlier call do not matter.
 *   vocab   additionally <= BS_LMHEAD_NOALLOC_MAX_VOCAB, else BS_E_WORKSPACE
 *   stream  the device is the stream's (the current device for NULL)
 * All calls on one GPU share its one scratch array: calls that may overlap on
 * one GPU (different streams, or different host threads without ordering)
 * race and give undefined results; order them on one stream.
 */
#define BS_LMHEAD_NOALLOC_MAX_VOCAB 262144
int32_t bs_lmhead_planes_topk_noalloc(const uint8_t *planes03, const uint8_t *planes47,
                                      const int32_t *row_scale, const int8_t *h, int64_t vocab,
                                      int64_t dim, int32_t top_k, int32_t max_candidates,
                                      int32_t *top_idx, int64_t *top_score, int32_t *info,
                                      void *stream);

/* ======================================================================== */
/* Activation encoders upstream of the GEMVs                                 */
/* ======================================================================== */
/*
 * bs_act_quant_i8 -- per-token absmax quantisation to int8 ([IE] section
 * 4.4: BitNet quantises activations per token, absmax -> int8; section 3.1:
 * activations are int64 fixed point):
 *   A = max_i |x_i|,  q_i = sgn(x_i) * floor((254 |x_i| + A) / (2 A))
 * i.e. 127 x / A rounded half away from zero (q = 0 when A = 0); the
 * dequantised value is q * A / 127 in x's fixed point.
 *   x       device int64[k], 8-byte aligned; |x_i| <= 2^55
 *   q       device int8[k] (the activation vector of bs_ternary_gemv)
 *   absmax  device int64[1], 8-byte aligned: A, or -1 when the bound breaks
 *   status  device int32[1], 4-byte aligned: BS_OK, or BS_E_OVERFLOW when
 *           some |x_i| > 2^55 (fail loud, [IE] section 3.4: then every q_i
 *           is 0); read it after the stream synchronises
 * Errors (host): BS_E_NULL, BS_E_SHAPE (k < 1 or k > 2^31), BS_E_ALIGN,
 *   BS_E_HIP.
 */
int32_t bs_act_quant_i8(const int64_t *x, int64_t k, int8_t *q, int64_t *absmax,
                        int32_t *status, void *stream);

/*
 * bs_lns8_encode -- int64 fixed-point activations (frac fractional bits) to
 * LNS8 bytes S1|E4|L3 ([BS] section 3: code k stands for 2^((k-74)/8), code 0
 * is exact zero; section 9: LNS8 saturation / underflow).  For v = x/2^frac
 * the code is the nearest integer to 74 + 8 log2|v| (never a tie), 127 above
 * the top code (saturation), and the zero byte 0x00 when it is below 1
 * (underflow to zero); bit 7 is the sign of a non-zero code.  The output is
 * the x_lns8 operand of bs_lns8_phase_gemv / bs_flns_phase_gemv.
 *   x      device int64[k], 8-byte aligned
 *   frac   0..62
 *   out    device uint8[k]
 * Errors: BS_E_NULL, BS_E_SHAPE, BS_E_RANGE (frac), BS_E_ALIGN, BS_E_HIP.
 *
 * bs_lns8_encode_edges -- the integer code edges the encoder uses, on the
 * host: edges[c] (c = 1..127) = the least |x| whose code is at least c,
 * ceil(2^(frac + (2c - 149)/16)), or UINT64_MAX when above 2^63; edges[0]
 * = 0.  Host only.  Errors: BS_E_NULL, BS_E_RANGE.
 */
int32_t bs_lns8_encode(const int64_t *x, int64_t k, int32_t frac, uint8_t *out, void *stream);
int32_t bs_lns8_encode_edges(int32_t frac, uint64_t *edges /* host [128] */);

/* ======================================================================== */
/* Candidate sampler downstream of the lm_head ([T2] ScoredToken /          */
/* sampleFromCandidates; [IE] section 3.3 integer samplers)                 */
/* ======================================================================== */
/*
 * bs_sample_candidates -- one token from n scored candidates (e.g. the
 * top_idx / top_score of bs_lmhead_planes_topk).  Candidates rank by (score
 * desc, index asc, input position asc).
 *   mode BS_SAMPLE_GREEDY: rank 0 (argmax, lowest index on ties).
 *   mode BS_SAMPLE_DRAW: rank r gets the Q31 weight
 *       w_r = P(t mod 2^16) >> (t >> 16),  t = (score_0 - score_r) * beta_q16
 *     (0 once t >> 16 >= 32), P(u) ~ 2^31 * 2^(-u / 2^16) the integer cubic
 *     2^31 - ((A1 - ((A2 - ((A3 u) >> 16)) u >> 16)) u >> 16) with A1 =
 *     1484817034, A2 = 495114803, A3 = 84039593 (a minimax fit, P(0) = 1 and
 *     P(1) = 1/2 exactly, relative error < 1.1e-4): beta_q16 is the base-2
 *     inverse temperature in Q16 (0 = uniform).  Top-p keeps the ranks whose
 *     preceding cumulative weight is below top_p_q16/2^16 of the total,
 *     min-p those whose weight is at least min_p_q16/2^16 of w_0.  The draw
 *     is Lemire's bounded integer in [0, kept total) from the first 8 bytes
 *     (big endian) of SHA-256(seed_le64 || position_le64 || attempt_le32),
 *     attempt = 0, 1, ... (at most 16); the token is the first rank whose
 *     cumulative weight exceeds it.
 *   idx, score  device int32[n] (4-byte aligned), int64[n] (8-byte aligned)
 *   n           1..1024
 *   top_p_q16   1..65536 (65536 = off); min_p_q16 0..65536 (0 = off)
 *   result      device int64[6], 8-byte aligned: token, rank, kept ranks,
 *               kept weight total, draw, SHA-256 attempts (greedy: token,
 *               0, 1, 0, 0, 0); token and rank -1 when no attempt was
 *               accepted (probability below 2^-300)
 * Errors: BS_E_NULL, BS_E_SHAPE (n), BS_E_RANGE (mode, top_p, min_p),
 *   BS_E_ALIGN, BS_E_HIP.
 */
#define BS_SAMPLE_GREEDY 0
#define BS_SAMPLE_DRAW 1
int32_t bs_sample_candidates(const int32_t *idx, const int64_t *score, int32_t n, int32_t mode,
                             uint32_t beta_q16, uint32_t top_p_q16, uint32_t min_p_q16,
                             uint64_t seed, uint64_t position, int64_t *result, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BS_H */
