"""Oracle for the steps on either side of the GEMV hot path (test
infrastructure only: only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; it imports nothing from the
product).

Plain, slow Python on exact integers, one function per step:

* ``act_quant_i8`` -- per-token absmax quantisation of int64 fixed-point
  activations to int8 ("A standalone deterministic integer inference engine
  for BitNet-style LLMs", section 4.4: BitNet quantises activations per token,
  absmax -> int8; section 3.1: activations are int64 fixed point);
* ``lns8_encode`` -- int64 fixed-point activations to LNS8 bytes S1|E4|L3
  ("BitState / HSDR PoC Technical Brief - v0.5", section 3: code 0 is exact
  zero, code k stands for 2^((k-74)/8); section 9 lists LNS8 saturation and
  underflow among the correctness checks);
* ``sample_candidates`` -- one token drawn from scored candidates ("[bitnet]
  T2: lm_head via BITNET_PLANES ..." comment introducing ScoredToken and
  sampleFromCandidates; integer-engine page section 3.3: integer samplers,
  greedy / temperature / top-p / min-p, lowest-index tie-break, a
  counter-based SHA-256 + Lemire draw keyed by (seed, position)).

The pages fix the steps but not every constant; the readings taken here:

* quantisation rounds half away from zero: q = sgn(x) floor((254|x| + A) /
  (2A)), A = max|x|, q = 0 when A = 0; |x| <= 2^55 (fail loud beyond);
* encoding picks the nearest code of 74 + 8 log2|v| (never a tie: the
  midpoints are irrational), saturates at 127 and flushes codes below 1 to
  the zero byte 0x00; the sign bit is set only for non-zero codes;
* sampler weights are 2^-(beta d / 2^16) in Q31, d = s_max - s, beta the
  inverse temperature in Q16 (base 2), evaluated by the integer cubic
  ``pow2_neg_q31`` below (constants A1, A2, A3 fixed by a minimax fit with
  P(0) = 1 and P(1) = 1/2 exactly; relative error < 1.1e-4); top-p keeps the
  ranks whose preceding cumulative weight is below p * W, min-p the ranks
  whose weight is at least p * w_0 (both Q16); the draw is Lemire's
  nearly-divisionless bounded integer from the first 8 digest bytes (big
  endian) of SHA-256(seed_le64 || position_le64 || attempt_le32).
"""
from __future__ import annotations

import hashlib

import numpy as np

ACT_ABS_MAX = 1 << 55          # |x| bound of the quantiser (127|x| stays far inside int64)

# ---------------------------------------------------------------- quantise


def act_quant_i8(x):
    """(q int8[K], absmax) with q_i = round_half_away(127 x_i / A)."""
    xs = [int(v) for v in np.asarray(x).ravel()]
    for v in xs:
        if abs(v) > ACT_ABS_MAX:
            raise OverflowError("|x| > 2^55")
    a = max((abs(v) for v in xs), default=0)
    q = np.zeros(len(xs), dtype=np.int8)
    if a == 0:
        return q, 0
    for i, v in enumerate(xs):
        m = (254 * abs(v) + a) // (2 * a)
        q[i] = m if v >= 0 else -m
    return q, a


# ------------------------------------------------------------------ encode


def _code_at_least(mag: int, frac: int, c: int) -> bool:
    """Is |v| = mag / 2^frac at or above the lower edge 2^((c - 74.5)/8) of
    code c?  Exactly: mag^16 >= 2^(16 frac + 2c - 149)."""
    e = 16 * frac + 2 * c - 149
    if e >= 0:
        return mag ** 16 >= (1 << e)
    return (mag ** 16) << (-e) >= 1


def lns8_code(mag: int, frac: int) -> int:
    """Nearest code of 74 + 8 log2(mag / 2^frac), saturated at 127, 0 below 1."""
    if mag == 0:
        return 0
    c = 0
    for cand in range(1, 128):
        if _code_at_least(mag, frac, cand):
            c = cand
        else:
            break
    return c


def lns8_encode(x, frac: int) -> np.ndarray:
    """LNS8 bytes (bit 7 = sign, bits 6..0 = code) of int64 fixed-point x."""
    out = np.zeros(np.asarray(x).size, dtype=np.uint8)
    for i, v in enumerate(int(t) for t in np.asarray(x).ravel()):
        c = lns8_code(abs(v), frac)
        out[i] = 0 if c == 0 else (c | (0x80 if v < 0 else 0))
    return out


# ------------------------------------------------------------------ sample

POW2_A1 = 1484817034           # Q31 coefficients of P(x) = 1 - a1 x + a2 x^2 - a3 x^3
POW2_A2 = 495114803
POW2_A3 = 84039593
SAMPLE_GREEDY, SAMPLE_DRAW = 0, 1
MAX_DRAWS = 16


def pow2_neg_q31(u: int) -> int:
    """~ 2^31 * 2^(-u / 2^16) for 0 <= u < 2^16: integer Horner, floor shifts."""
    h = POW2_A3
    h = POW2_A2 - ((h * u) >> 16)
    h = POW2_A1 - ((h * u) >> 16)
    return (1 << 31) - ((h * u) >> 16)


def weight_q31(d: int, beta: int) -> int:
    """2^-(beta d / 2^16) in Q31 for d >= 0 (0 once the exponent reaches 32)."""
    t = d * beta
    n = t >> 16
    if n >= 32:
        return 0
    return pow2_neg_q31(t & 0xFFFF) >> n


def draw_u64(seed: int, position: int, attempt: int) -> int:
    msg = (seed.to_bytes(8, "little") + position.to_bytes(8, "little")
           + attempt.to_bytes(4, "little"))
    return int.from_bytes(hashlib.sha256(msg).digest()[:8], "big")


def lemire_bounded(seed: int, position: int, n: int):
    """(value in [0, n), attempts used): Lemire's nearly divisionless method,
    each attempt one counter-based 64-bit draw."""
    for a in range(MAX_DRAWS):
        m = draw_u64(seed, position, a) * n
        lo = m & ((1 << 64) - 1)
        if lo < n and lo < ((1 << 64) - n) % n:
            continue
        return m >> 64, a + 1
    raise RuntimeError("no accepted draw")


def sample_candidates(idx, score, mode: int, beta: int = 1 << 16, top_p: int = 1 << 16,
                      min_p: int = 0, seed: int = 0, position: int = 0) -> dict:
    """One token from the candidates (idx int32, score int64).  Returns the
    token, its rank in (score desc, index asc) order, the number of kept
    ranks, the kept weight total, the bounded draw and the SHA-256 attempts
    it took."""
    cand = sorted(zip((int(s) for s in score), (int(i) for i in idx)),
                  key=lambda p: (-p[0], p[1]))
    if not cand:
        raise ValueError("no candidates")
    if mode == SAMPLE_GREEDY:
        return {"token": cand[0][1], "rank": 0, "kept": 1, "total": 0, "draw": 0, "attempts": 0}
    s0 = cand[0][0]
    w = [weight_q31(s0 - s, beta) for s, _ in cand]
    wall = sum(w)
    kept, cum = 0, 0
    for r, wr in enumerate(w):
        if (cum << 16) >= top_p * wall or (wr << 16) < min_p * w[0]:
            break
        kept = r + 1
        cum += wr
    total = sum(w[:kept])
    v, attempts = lemire_bounded(seed, position, total)
    run = 0
    for r in range(kept):
        run += w[r]
        if run > v:
            return {"token": cand[r][1], "rank": r, "kept": kept, "total": total, "draw": v,
                    "attempts": attempts}
    raise AssertionError("unreachable")

