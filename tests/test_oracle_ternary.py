"""Pins of the ternary-GEMV oracle against facts that do not come from it.

The oracle follows "A standalone deterministic integer inference engine for
BitNet-style LLMs", section 4.2 (ternary signed sum with per-group integer
scale and floor shift).  Each test below would fail on a plausible mistake:
a hand-worked example, closed forms (all zero, all +1, one-hot activations),
the 1-bit identity of section 4.1 (2*pos_sum - block_total), the floor rule of
section 3.3 on negative values, and a brute force written with NumPy.
"""
import json
import os

import numpy as np
import pytest

import oracle
from bit_decode_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def numpy_brute(t, scales, x, frac=0):
    rows, k = t.shape
    g = k // 128
    s = (t.astype(np.int64).reshape(rows, g, 128) * x.astype(np.int64).reshape(1, g, 128)).sum(-1)
    p = s * scales.astype(np.int64)
    return np.floor_divide(p, np.int64(1) << frac).sum(-1)


def test_hand_worked_example():
    spec = json.load(open(os.path.join(GOLDEN, "ternary_hand.json")))
    k = spec["k"]
    x = (np.arange(k) - 64).astype(np.int8)
    rows = spec["rows"]
    t = np.zeros((len(rows), k), np.int8)
    sc = np.zeros((len(rows), k // 128), np.int16)
    for r, row in enumerate(rows):
        t[r, row["plus"][0]:row["plus"][1]] = 1
        t[r, row["minus"][0]:row["minus"][1]] = -1
        sc[r, :] = row["scale"]
    y0 = oracle.ternary_gemv_def(t, sc, x, frac=0)
    y3 = oracle.ternary_gemv_def(t, sc, x, frac=3)
    assert list(y0) == [row["y_frac0"] for row in rows]
    assert list(y3) == [row["y_frac3"] for row in rows]
    # the packed masked-sum form reads the same numbers back
    ym = oracle.ternary_gemv_masked(oracle.ternary_pack(t), oracle.scales_pack(sc), x,
                                    len(rows), k, frac=3)
    assert list(ym) == [row["y_frac3"] for row in rows]


def test_all_zero_weights_give_zero():
    t = np.zeros((70, 256), np.int8)
    _, sc, x = synth.ternary(70, 256, seed=1)
    assert not oracle.ternary_gemv_def(t, sc, x).any()


def test_all_plus_one_unit_scale_is_sum_of_x():
    _, _, x = synth.ternary(3, 384, seed=2, act="uniform127")
    t = np.ones((3, 384), np.int8)
    sc = np.ones((3, 3), np.int16)
    y = oracle.ternary_gemv_def(t, sc, x)
    assert (y == int(x.astype(np.int64).sum())).all()


def test_one_hot_activation_reads_a_column():
    t, sc, _ = synth.ternary(65, 256, seed=3, p_zero=1 / 3)
    for i in (0, 1, 7, 8, 127, 128, 200, 255):
        x = np.zeros(256, np.int8)
        x[i] = 1
        y = oracle.ternary_gemv_def(t, sc, x)
        assert (y == t[:, i].astype(np.int64) * sc[:, i // 128]).all()
        ym = oracle.ternary_gemv_masked(oracle.ternary_pack(t), oracle.scales_pack(sc), x, 65, 256)
        assert (ym == y).all()


def test_binary_rows_match_pos_sum_identity():
    """With no zero weights the signed sum is 2*pos_sum - block_total
    (integer-engine page, section 4.1)."""
    rng = np.random.default_rng(5)
    t = np.where(rng.random((40, 256)) < 0.5, 1, -1).astype(np.int8)
    x = rng.integers(-128, 128, 256).astype(np.int8)
    sc = rng.integers(-32768, 32768, (40, 2)).astype(np.int16)
    pos = (t == 1)
    xs = x.astype(np.int64)
    expect = np.zeros(40, np.int64)
    for g in range(2):
        sl = slice(128 * g, 128 * g + 128)
        pos_sum = (pos[:, sl] * xs[sl]).sum(1)
        total = xs[sl].sum()
        expect += (2 * pos_sum - total) * sc[:, g].astype(np.int64)
    assert (oracle.ternary_gemv_def(t, sc, x) == expect).all()


@pytest.mark.parametrize("product,frac,expect", [(-3, 1, -2), (3, 1, 1), (-1, 5, -1),
                                                 (-32, 5, -1), (-33, 5, -2), (31, 5, 0)])
def test_floor_shift_rounds_toward_minus_infinity(product, frac, expect):
    t = np.zeros((1, 128), np.int8)
    t[0, 0] = 1
    x = np.zeros(128, np.int8)
    x[0] = 1
    sc = np.array([[product]], np.int16)
    assert oracle.ternary_gemv_def(t, sc, x, frac=frac)[0] == expect


def test_floor_is_per_group_before_the_sum():
    # two groups each with product -1 and frac 1: floor(-1/2) + floor(-1/2) = -2,
    # whereas a floor after the sum would give floor(-2/2) = -1
    t = np.zeros((1, 256), np.int8)
    t[0, 0] = t[0, 128] = 1
    x = np.zeros(256, np.int8)
    x[0] = x[128] = -1
    sc = np.ones((1, 2), np.int16)
    assert oracle.ternary_gemv_def(t, sc, x, frac=1)[0] == -2


@pytest.mark.parametrize("rows,k,seed,frac", [(256, 512, 0, 0), (67, 384, 1, 0),
                                              (130, 1280, 2, 4), (1, 128, 3, 0)])
def test_random_matches_numpy_brute_force(rows, k, seed, frac):
    t, sc, x = synth.ternary(rows, k, seed, p_zero=0.4)
    y = oracle.ternary_gemv_def(t, sc, x, frac)
    assert (y == numpy_brute(t, sc, x, frac)).all()
    ym = oracle.ternary_gemv_masked(oracle.ternary_pack(t), oracle.scales_pack(sc), x, rows, k, frac)
    assert (ym == y).all()


def test_extreme_values():
    # x = -128 everywhere (int8 minimum), weights -1, scale -32768: the largest
    # magnitude per group, 128*128*32768 = 2^29
    t = -np.ones((2, 256), np.int8)
    x = np.full(256, -128, np.int8)
    sc = np.full((2, 2), -32768, np.int16)
    y = oracle.ternary_gemv_def(t, sc, x)
    assert (y == -2 * (1 << 29)).all()
    assert (y == numpy_brute(t, sc, x)).all()


def test_pack_bit_positions():
    """Hand-placed bits of the tiled layout: block (tile, g) of 2048 bytes,
    W_nonzero row j at 16j, W_negative at 1024 + 16j, weight i at bit i%8 of
    byte i/8."""
    rows, k = 66, 256
    t = np.zeros((rows, k), np.int8)
    t[0, 0] = 1          # tile 0, g 0, row 0: nz byte 0 bit 0
    t[0, 9] = -1         # nz byte 1 bit 1, neg byte 1024+1 bit 1
    t[1, 127] = 1        # row 1: nz byte 16+15 bit 7
    t[2, 128] = -1       # g 1: block 1, row 2: nz byte 2048+32, neg 2048+1024+32
    t[65, 255] = 1       # tile 1 (row 1 of it), g 1: block 3: byte 3*2048+16+15 bit 7
    p = oracle.ternary_pack(t)
    assert p.size == 128 * 256 // 4
    want = {0: 0x01, 1: 0x02, 1024 + 1: 0x02, 16 + 15: 0x80, 2048 + 32: 0x01,
            2048 + 1024 + 32: 0x01, 3 * 2048 + 16 + 15: 0x80}
    nz = np.nonzero(p)[0]
    assert sorted(nz.tolist()) == sorted(want)
    for off, v in want.items():
        assert p[off] == v


def test_pack_unpack_roundtrip_and_rejects():
    t, _, _ = synth.ternary(100, 384, seed=9, p_zero=1 / 3)
    p = oracle.ternary_pack(t)
    assert (oracle.ternary_unpack(p, 100, 384) == t).all()
    # a W_negative bit whose W_nonzero bit is clear is not a ternary code
    z = oracle.ternary_pack(np.zeros((3, 128), np.int8))
    z[1024 + 16 * 2 + 3] = 0x10
    with pytest.raises(ValueError):
        oracle.ternary_unpack(z, 3, 128)
    t2 = t.copy()
    t2[5, 5] = 2
    with pytest.raises(ValueError):
        oracle.ternary_pack(t2)


def test_scales_pack_positions():
    sc = np.arange(70 * 3, dtype=np.int16).reshape(70, 3)
    ps = oracle.scales_pack(sc)
    assert ps.size == 128 * 3
    assert ps[(0 * 3 + 2) * 16 + 5] == sc[5, 2]
    assert ps[(4 * 3 + 1) * 16 + 3] == sc[67, 1]
    assert ps[(4 * 3 + 0) * 16 + 6] == 0      # padding row 70
    assert ps[(7 * 3 + 2) * 16 + 15] == 0     # last padding row 127


def test_row_parallel_form_matches_single_thread():
    """The all-core baseline's row-parallel form returns the single-thread
    definition form's bytes, at several thread counts, including a ragged
    row count and an out-of-range trit (rejected before any row runs)."""
    t, sc, x = synth.ternary(301, 1024, 3)
    want = oracle.ternary_gemv_def(t, sc, x, 2)
    for n in (1, 3, 8):
        assert oracle.set_threads(n) == n
        assert (oracle.ternary_gemv_def_mt(t, sc, x, 2) == want).all()
    bad = t.copy()
    bad[150, 7] = 2
    with pytest.raises(Exception):
        oracle.ternary_gemv_def_mt(bad, sc, x)
    oracle.set_threads(1)
