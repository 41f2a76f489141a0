"""Pins of the oracle's Q1_0 weight apply (integer-engine page, section 4.1):
a hand-worked golden case (floor shift of negative values included), the
ternary definition (signs are ternary weights without zeros, and that oracle
is pinned on its own), a NumPy brute force, and the page's masked form
2*pos_sum - block_total on the packed bits, which must agree exactly."""
import json
import os

import numpy as np
import pytest

import oracle
from bit_decode_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_case():
    g = json.load(open(os.path.join(GOLDEN, "q1_hand.json")))
    k = g["k"]
    x = np.full(k, g["x_all"], np.int8)
    s = -np.ones((len(g["rows"]), k), np.int8)
    sc = np.zeros((len(g["rows"]), 1), np.int16)
    for r, row in enumerate(g["rows"]):
        a, b = row["plus"]
        s[r, a:b] = 1
        sc[r, 0] = row["scale"]
    for frac, want in g["expected"].items():
        assert oracle.q1_gemv_def(s, sc, x, int(frac)).tolist() == want
        bits = oracle.q1_pack(s)
        assert oracle.q1_gemv_masked(bits, oracle.scales_pack(sc), x, 2, k,
                                     int(frac)).tolist() == want


@pytest.mark.parametrize("rows,k,seed", [(3, 128, 0), (70, 384, 1), (129, 1280, 2)])
@pytest.mark.parametrize("frac", [0, 5, 31, 62])
def test_definition_equals_ternary_definition(rows, k, seed, frac):
    s, sc, x = synth.q1(rows, k, seed)
    rng = np.random.default_rng(seed + 100)
    sc = rng.integers(-32768, 32768, sc.shape).astype(np.int16)   # negative scales too
    assert (oracle.q1_gemv_def(s, sc, x, frac) == oracle.ternary_gemv_def(s, sc, x, frac)).all()


@pytest.mark.parametrize("seed", range(3))
def test_numpy_brute_force(seed):
    s, sc, x = synth.q1(9, 256, seed)
    frac = 3 * seed
    groups = (s.astype(np.int64).reshape(9, 2, 128) * x.astype(np.int64).reshape(2, 128)).sum(2)
    want = np.floor_divide(groups * sc.astype(np.int64), 1 << frac).sum(1)
    assert (oracle.q1_gemv_def(s, sc, x, frac) == want).all()


@pytest.mark.parametrize("rows,k,seed", [(1, 128, 0), (64, 256, 1), (65, 512, 2), (200, 2560, 3)])
@pytest.mark.parametrize("frac", [0, 7, 30])
def test_masked_form_equals_definition(rows, k, seed, frac):
    s, sc, x = synth.q1(rows, k, seed)
    y = oracle.q1_gemv_masked(oracle.q1_pack(s), oracle.scales_pack(sc), x, rows, k, frac)
    assert (y == oracle.q1_gemv_def(s, sc, x, frac)).all()


def test_extremes_and_layout():
    k = 256
    x = np.full(k, -128, np.int8)
    s = np.ones((2, k), np.int8)
    s[1] = -1
    sc = np.full((2, 2), -32768, np.int16)
    # per group 128 * (-128) * (-32768) = 2^29, two groups: +-2^30
    assert oracle.q1_gemv_def(s, sc, x).tolist() == [1 << 30, -(1 << 30)]
    bits = oracle.q1_pack(s)
    assert bits.size == 64 * k // 8
    assert (bits[:16] == 0xFF).all() and (bits[16:32] == 0).all()       # rows 0, 1 of group 0
    assert (bits[1024:1040] == 0xFF).all()                              # row 0 of group 1
    with pytest.raises(ValueError):
        oracle.q1_pack(np.zeros((1, 128), np.int8))                     # 0 is not a sign
