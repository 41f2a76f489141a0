"""Pins of the LNS8 eight-phase oracle ("BitState / HSDR PoC Technical Brief -
v0.5", sections 3, 3.1, 4, 5.1 and the Phase A checklist of section 7).

What pins it, besides agreement of its three forms with each other:
* the code facts the brief states (code 0 = 0, code 74 = 1.0, code 122 = 64,
  eight codes = x2) from a text fixture;
* correct rounding of F[p] = 2^((p-2)/8), checked with exact integer
  inequalities and against math.sqrt(2) for p = 6;
* the dyadic decomposition |x| = 2^-9 * 2^band * F[phase];
* C_s = N - 2*Nneg against a lane-by-lane count on random masks;
* closed forms: an all-code-74 activation makes S the plain signed dot of
  signs; code 1 and code 127 (the two ends of the range);
* the FP64 direct ternary dot of Phase A, to a few ulps per term.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_decode_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_codes():
    pins = []
    for line in open(os.path.join(GOLDEN, "lns8_code_pins.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            pins.append((int(c), float(v)))
    return pins


def test_page_code_facts():
    pins = _golden_codes()
    assert len(pins) == 3
    for code, value in pins:
        assert oracle.lns8_decode(code) == value


def test_eight_codes_double_exactly():
    for k in range(1, 120):
        assert oracle.lns8_decode(k + 8) == 2.0 * oracle.lns8_decode(k)


def test_f_hat_is_correctly_rounded():
    fh = oracle.f_hat()
    assert fh[2] == 1.0
    assert fh[6] == math.sqrt(2.0)          # IEEE sqrt is correctly rounded
    for p, f in enumerate(fh):
        m, e = math.frexp(f)                 # f = m * 2^e, 0.5 <= m < 1
        mi = int(m * (1 << 53))              # 53-bit integer mantissa
        ex = e - 53                          # f = mi * 2^ex
        # 2^((p-2)/8) lies within half an ulp of f:
        # (mi - 1/2)^8 * 2^(8 ex) <= 2^(p-2) <= (mi + 1/2)^8 * 2^(8 ex)
        lo = Fraction(2 * mi - 1) ** 8 * Fraction(2) ** (8 * ex - 8)
        hi = Fraction(2 * mi + 1) ** 8 * Fraction(2) ** (8 * ex - 8)
        target = Fraction(2) ** (p - 2)
        assert lo <= target <= hi, p
        # and libm agrees to within one ulp
        assert abs(f - 2.0 ** ((p - 2) / 8)) <= math.ulp(f)


def test_decode_is_dyadic_band_times_phase():
    fh = oracle.f_hat()
    for k in range(1, 128):
        band, phase = k >> 3, k & 7
        assert k == 8 * band + phase
        assert oracle.lns8_decode(k) == math.ldexp(fh[phase], band - 9)
    # anchor identity of section 5.2: k = (120 + phase) + 8*(band - 15)
    for k in range(1, 128):
        assert k == (120 + (k & 7)) + 8 * ((k >> 3) - 15)


def test_signed_population_identity():
    """C_s = N - 2*Nneg equals the sum of product signs over the selected
    lanes (section 4)."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        a_s, wnz, wneg_raw, sign = (int(v) for v in rng.integers(0, 2**63, 4, dtype=np.int64))
        a_s |= int(rng.integers(0, 2)) << 63
        wneg = wneg_raw & wnz
        m = a_s & wnz
        pneg = sign ^ wneg
        n = bin(m).count("1")
        nneg = bin(m & pneg).count("1")
        lane_sum = 0
        for lane in range(64):
            if (m >> lane) & 1:
                w = -1 if (wneg >> lane) & 1 else 1
                s = -1 if (sign >> lane) & 1 else 1
                lane_sum += w * s
        assert n - 2 * nneg == lane_sum


def _three_forms(t, x):
    a = oracle.lns8_direct(t, x)
    b = oracle.lns8_tile64(t, x)
    c, h = oracle.lns8_popcount(t, x, hist=True)
    assert (a == b).all()
    assert (a == c).all()
    # histogram-to-A equivalence, section 3.1
    assert (a == (h * (np.int64(1) << np.arange(16, dtype=np.int64))).sum(-1)).all()
    return a, h


def numpy_hist(t, x):
    """H[r][phase][band] = sum_i t_i * (-1)^S1_i over positions with that code."""
    code = (x & 0x7F).astype(np.int64)
    sgn = np.where(x >> 7, -1, 1).astype(np.int64)
    h = np.zeros((t.shape[0], 8, 16), np.int64)
    for c in range(1, 128):
        sel = code == c
        if sel.any():
            h[:, c & 7, c >> 3] += (t[:, sel].astype(np.int64) * sgn[sel]).sum(1)
    return h


@pytest.mark.parametrize("rows,k,seed", [(64, 256, 0), (70, 512, 1), (3, 128, 2)])
def test_random_three_forms_and_numpy_histogram(rows, k, seed):
    t, x = synth.lns8(rows, k, seed)
    a, h = _three_forms(t, x)
    assert (h == numpy_hist(t, x)).all()


def _adversarial_cases():
    rng = np.random.default_rng(7)
    k = 256
    t = rng.integers(-1, 2, (40, k)).astype(np.int8)
    yield "all_same_code", t, np.full(k, 80, np.uint8)
    yield "all_zero_code", t, np.zeros(k, np.uint8)
    yield "zero_code_sign_set", t, np.full(k, 0x80, np.uint8)
    yield "code_1", t, (rng.integers(0, 2, k).astype(np.uint8) << 7) | 1
    yield "code_127", t, (rng.integers(0, 2, k).astype(np.uint8) << 7) | 127
    yield "all_codes", t, rng.integers(0, 256, k).astype(np.uint8)
    # exactly cancelling products: same code, opposite product sign in pairs
    tc = np.ones((4, k), np.int8)
    xc = np.full(k, 90, np.uint8)
    xc[1::2] |= 0x80
    yield "cancel", tc, xc


@pytest.mark.parametrize("case", list(_adversarial_cases()), ids=lambda c: c[0])
def test_adversarial_three_forms(case):
    _, t, x = case
    a, h = _three_forms(t, x)
    assert (h == numpy_hist(t, x)).all()
    if case[0] in ("all_zero_code", "zero_code_sign_set", "cancel"):
        assert not a.any()


def test_code74_makes_s_the_signed_dot_of_signs():
    """code 74 = 1.0 (phase 2, band 9, F[2] = 1): S = sum_i t_i*(-1)^S1_i."""
    t, _ = synth.lns8(30, 512, 3)
    rng = np.random.default_rng(3)
    s1 = rng.integers(0, 2, 512).astype(np.uint8)
    x = (s1 << 7) | 74
    a, _ = _three_forms(t, x)
    assert not np.delete(a, 2, axis=1).any()
    dot = (t.astype(np.int64) * np.where(s1, -1, 1)).sum(1)
    assert (a[:, 2] == dot * 512).all()
    s = oracle.lns8_materialize(a)
    assert (s == dot.astype(np.float64)).all()


def test_code1_and_code127_ends():
    t, _ = synth.lns8(10, 128, 4)
    for code, phase, band in ((1, 1, 0), (127, 7, 15)):
        x = np.full(128, code, np.uint8)
        a, _ = _three_forms(t, x)
        dot = t.astype(np.int64).sum(1)
        assert (a[:, phase] == dot * (1 << band)).all()
        assert not np.delete(a, phase, axis=1).any()


def test_materialize_unit_vectors_and_zero():
    fh = oracle.f_hat()
    for p in range(8):
        a = np.zeros((1, 8), np.int64)
        a[0, p] = 1
        assert oracle.lns8_materialize(a)[0] == math.ldexp(fh[p], -9)
    assert oracle.lns8_materialize(np.zeros((1, 8), np.int64))[0] == 0.0


def test_materialize_matches_fp64_direct_dot():
    """Phase A: the FP64 direct ternary dot agrees with the dyadic S to the
    rounding of K fp64 additions."""
    t, x = synth.lns8(200, 4096, 5)
    a = oracle.lns8_direct(t, x)
    s = oracle.lns8_materialize(a)
    d = oracle.lns8_fp64_dot(t, x)
    code = (x & 0x7F).astype(np.float64)
    mag = np.where(code > 0, 2.0 ** ((code - 74) / 8), 0.0)
    bound = 4096 * 2.0 ** -52 * (np.abs(t) * mag).sum(1) + 1e-300
    assert (np.abs(s - d) <= bound).all()
    # S is zero exactly when every A[p] is zero (2^(p/8) are independent over Q)
    assert ((s == 0) == (~a.any(1))).all()


def test_direct_row_parallel_matches_single_thread():
    t, x = synth.lns8(257, 1024, 5)
    want = oracle.lns8_direct(t, x)
    for n in (2, 7):
        oracle.set_threads(n)
        assert (oracle.lns8_direct_mt(t, x) == want).all()
    oracle.set_threads(1)
