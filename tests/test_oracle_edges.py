"""Pins of the oracle for the steps on either side of the GEMV (CPU only).

Quantisation: a hand-worked example (tests/golden/act_quant_hand.json), the
rounding property |q - 127 x / A| <= 1/2 with halves away from zero, the
largest element at +-127, sign symmetry, scale invariance, the fail-loud
bound.  LNS8 encoding: the brief's code facts (code 74 = 1.0, code 122 = 64,
eight codes per factor of two, code 0 = zero), the nearest-code property
against a floating-point log2 away from the code edges, saturation,
underflow, the sign bit.  Sampler: the weight polynomial against 2^-x over
every input, exact powers of two, Lemire's bounded draw in closed form for
power-of-two ranges and its rejection path, greedy = argmax with the
lowest-index tie-break by brute force, filters, order independence, and
the draw distribution against the weights.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import edges

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- quantise

def test_quant_hand_example():
    for g in json.load(open(os.path.join(GOLDEN, "act_quant_hand.json")))["cases"]:
        q, a = edges.act_quant_i8(np.array(g["x_fixed"], np.int64))
        assert a == g["absmax"]
        assert q.tolist() == g["q"]


@pytest.mark.parametrize("seed", range(6))
def test_quant_rounding_property(seed):
    rng = np.random.default_rng(seed)
    mag = [1, 100, 1 << 20, 1 << 40, 1 << 55][seed % 5]
    x = rng.integers(-mag, mag + 1, 300).astype(np.int64)
    x[rng.integers(0, 300)] = mag * (1 if seed % 2 else -1)
    q, a = edges.act_quant_i8(x)
    assert a == int(np.abs(x).max())
    for xi, qi in zip(x.tolist(), q.tolist()):
        exact = Fraction(127 * xi, a)
        err = abs(Fraction(qi) - exact)
        assert err <= Fraction(1, 2)
        if err == Fraction(1, 2):
            assert abs(qi) > abs(exact)          # halves go away from zero
    assert np.abs(q).max() == 127


def test_quant_symmetry_scale_and_zero():
    rng = np.random.default_rng(7)
    x = rng.integers(-10 ** 6, 10 ** 6, 500).astype(np.int64)
    q, a = edges.act_quant_i8(x)
    qn, an = edges.act_quant_i8(-x)
    assert an == a and (qn == -q).all()
    q3, a3 = edges.act_quant_i8(3 * x)
    assert a3 == 3 * a and (q3 == q).all()
    z, az = edges.act_quant_i8(np.zeros(64, np.int64))
    assert az == 0 and not z.any()


def test_quant_fails_loud():
    with pytest.raises(OverflowError):
        edges.act_quant_i8(np.array([0, (1 << 55) + 1], np.int64))
    edges.act_quant_i8(np.array([-(1 << 55)], np.int64))


# ------------------------------------------------------------------ encode

@pytest.mark.parametrize("frac", [0, 8, 16, 30])
def test_encode_page_codes(frac):
    """Code 74 is 1.0 and code 122 is 64 (brief, sections 3 and 5.2); code 0
    is exact zero; the sign rides in bit 7."""
    one = 1 << frac
    assert edges.lns8_encode([one], frac)[0] == 74
    assert edges.lns8_encode([64 * one], frac)[0] == 122
    assert edges.lns8_encode([-64 * one], frac)[0] == 0x80 | 122
    assert edges.lns8_encode([0], frac)[0] == 0


@pytest.mark.parametrize("frac", [4, 20])
def test_encode_doubling_moves_eight_codes(frac):
    rng = np.random.default_rng(frac)
    for v in rng.integers(1, 1 << 40, 200).tolist():
        c = edges.lns8_code(v, frac)
        c2 = edges.lns8_code(2 * v, frac)
        if 1 <= c and c + 8 <= 127:
            assert c2 == c + 8


@pytest.mark.parametrize("frac", [0, 12, 24])
def test_encode_nearest_code(frac):
    """Away from the code edges (where double log2 decides safely), the code
    is the nearest integer to 74 + 8 log2 |v|, clamped to [1, 127] or 0."""
    rng = np.random.default_rng(frac + 1)
    xs = np.concatenate([rng.integers(-(1 << 62), 1 << 62, 300),
                         rng.integers(-(1 << 20), 1 << 20, 300),
                         rng.integers(-300, 300, 100)]).astype(np.int64)
    out = edges.lns8_encode(xs, frac)
    for v, b in zip(xs.tolist(), out.tolist()):
        if v == 0:
            assert b == 0
            continue
        t = 74 + 8 * (math.log2(abs(v)) - frac)
        if abs(t - math.floor(t) - 0.5) < 1e-6:
            continue
        want = int(math.floor(t + 0.5))
        want = 127 if want > 127 else (0 if want < 1 else want)
        assert (b & 0x7F) == want
        assert (b >> 7) == (1 if (v < 0 and want) else 0)


def test_encode_saturation_and_underflow():
    # frac 62: the smallest magnitude 2^-62 is far below code 1 (2^-9.2)
    assert edges.lns8_code(1, 62) == 0
    # code 1 starts at 2^((1 - 74.5)/8) = 2^-9.1875
    frac = 40
    edge = 2.0 ** (frac - 9.1875)
    lo, hi = int(math.floor(edge)), int(math.ceil(edge))
    assert edges.lns8_code(lo, frac) == 0 and edges.lns8_code(hi, frac) == 1
    # code 127 is 2^(53/8) ~ 98.7; far above saturates
    assert edges.lns8_code((1 << 62), 0) == 127
    assert edges.lns8_code(99, 0) == 127 and edges.lns8_code(95, 0) == 127
    assert edges.lns8_code(94, 0) == 126 and edges.lns8_code(87, 0) == 126


def test_encode_agrees_with_decode():
    """decode(code) (the oracle's correctly rounded 2^((k-74)/8)) lies within
    a factor 2^(1/16) of the encoded value."""
    import oracle
    frac = 30
    rng = np.random.default_rng(3)
    for v in rng.integers(1 << 21, 1 << 36, 200).tolist():   # codes 1..126
        c = edges.lns8_code(v, frac)
        ratio = (v / 2.0 ** frac) / oracle.lns8_decode(c)
        assert 2 ** (-1 / 16) - 1e-12 <= ratio <= 2 ** (1 / 16) + 1e-12


# ------------------------------------------------------------------ sample

def test_pow2_polynomial_every_input():
    u = np.arange(1 << 16)
    got = np.array([edges.pow2_neg_q31(int(v)) for v in u], np.float64)
    want = np.exp2(31.0 - u / 65536.0)
    assert got[0] == 2 ** 31
    assert np.max(np.abs(got / want - 1)) < 1.1e-4
    assert (np.diff(got) <= 0).all()
    # the constants put P(1) at 1/2 exactly: 1 - a1 + a2 - a3 = 1/2
    assert (1 << 31) - edges.POW2_A1 + edges.POW2_A2 - edges.POW2_A3 == 1 << 30


def test_weight_exact_powers_and_cutoff():
    assert edges.weight_q31(0, 12345) == 1 << 31
    for n in range(0, 33):
        assert edges.weight_q31(n, 1 << 16) == ((1 << 31) >> n if n < 32 else 0)
        assert edges.weight_q31(2 * n, 1 << 15) == ((1 << 31) >> n if n < 32 else 0)
    assert edges.weight_q31(10 ** 12, 0) == 1 << 31       # beta 0: uniform


def test_sha256_known_answer():
    """FIPS 180-2 example: SHA-256("abc")."""
    import hashlib
    assert hashlib.sha256(b"abc").hexdigest() == (
        "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad")


def test_lemire_power_of_two_closed_form():
    """For n = 2^k no draw is rejected and the value is the top k bits."""
    for k in (1, 5, 31, 63):
        for pos in range(20):
            v, a = edges.lemire_bounded(9, pos, 1 << k)
            assert a == 1 and v == edges.draw_u64(9, pos, 0) >> (64 - k)


def test_lemire_rejection_and_range():
    n = (1 << 63) + 1          # rejects about half of all draws
    attempts = []
    for pos in range(200):
        v, a = edges.lemire_bounded(1, pos, n)
        assert 0 <= v < n
        attempts.append(a)
    assert max(attempts) > 1 and min(attempts) == 1


def test_greedy_is_argmax_lowest_index():
    rng = np.random.default_rng(11)
    for trial in range(50):
        n = int(rng.integers(1, 60))
        idx = rng.permutation(100000)[:n].astype(np.int32)
        score = rng.integers(-5, 5, n).astype(np.int64)
        best = max(range(n), key=lambda i: (score[i], -idx[i]))
        r = edges.sample_candidates(idx, score, edges.SAMPLE_GREEDY)
        assert r["token"] == idx[best]


def test_filters_and_order_independence():
    idx = np.array([10, 3, 7, 5, 1], np.int32)
    score = np.array([100, 100, 40, 99, -1000], np.int64)
    # beta = 2^16: weight halves per unit of score below the top
    base = dict(mode=edges.SAMPLE_DRAW, beta=1 << 16, seed=5)
    r = edges.sample_candidates(idx, score, top_p=1, **base)
    assert r["kept"] == 1 and r["token"] == 3          # ties: lower index first
    r = edges.sample_candidates(idx, score, min_p=1 << 16, **base)
    assert r["kept"] == 2 and r["token"] in (3, 10)
    r = edges.sample_candidates(idx, score, **base)
    assert r["kept"] == 3 and r["total"] == (1 << 31) * 2 + (1 << 30)
    perm = np.array([4, 2, 0, 3, 1])
    for pos in range(30):
        a = edges.sample_candidates(idx, score, position=pos, **base)
        b = edges.sample_candidates(idx[perm], score[perm], position=pos, **base)
        assert a == b


def test_draw_distribution_follows_weights():
    idx = np.arange(4, dtype=np.int32)
    score = np.array([0, -1, -2, -3], np.int64)       # weights 8 : 4 : 2 : 1 at beta = 2^16
    counts = np.zeros(4)
    n = 6000
    for pos in range(n):
        counts[edges.sample_candidates(idx, score, edges.SAMPLE_DRAW, seed=77,
                                       position=pos)["rank"]] += 1
    p = np.array([8, 4, 2, 1]) / 15.0
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 16.3          # 3 degrees of freedom, p = 0.001


def test_sampler_rejection_golden():
    """tests/golden/sampler_rejection.json (written by make_sampler_rejection.py
    beside it): keys whose first draw Lemire's method rejects.  2^33 = -1 mod 683,
    so 2^64 mod (683 * 2^31) = 682 * 2^31, and each key's first draw falls
    below it."""
    import json
    path = os.path.join(os.path.dirname(__file__), "golden", "sampler_rejection.json")
    with open(path) as f:
        g = json.load(f)
    total = g["n"] << 31
    assert g["total"] == total and pow(2, 33, 683) == 682
    assert (1 << 64) % total == 682 << 31
    idx = list(range(g["first_index"], g["first_index"] + g["n"]))
    for c in g["cases"]:
        lo = (edges.draw_u64(c["seed"], c["position"], 0) * total) % (1 << 64)
        assert lo < (1 << 64) % total                     # the first attempt is rejected
        o = edges.sample_candidates(idx, [g["score"]] * g["n"], edges.SAMPLE_DRAW, beta=0,
                                    seed=c["seed"], position=c["position"])
        assert (o["attempts"], o["draw"], o["token"], o["rank"]) == (
            c["attempts"], c["draw"], c["token"], c["rank"])
        assert o["draw"] == (edges.draw_u64(c["seed"], c["position"], 1) * total) >> 64
