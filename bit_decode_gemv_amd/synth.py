"""Seeded synthetic inputs for the ternary decode-GEMV workloads.

This module only draws random numbers and arranges them into arrays; it holds
none of the method's arithmetic.  Both the product path (through its codec)
and the oracle consume the arrays it returns, so neither side generates its
own inputs.

Every generator takes a seed and draws from NumPy's PCG64 through
``default_rng(SeedSequence(seed).spawn(n))``: one independent stream per
array, in the order the arrays are listed (weights, scales, activations).

Workloads (shapes from the BitNet b1.58 2B decode projections and the larger
LLaMA-like projections; the models themselves are not used):

* ``ternary``  -- iid trits with P(0) = p_zero and equiprobable signs, int16
  group scales uniform in [1, 4096], int8 activations either uniform in
  [-127, 127] or N(0, 32^2) rounded half-to-even and clipped to +-127;
* ``lns8``     -- iid uniform trits and LNS8 activation bytes: sign bit
  uniform, code 0 with probability 0.05, else uniform in 60..100;
* ``lmhead``   -- eight iid uniform trit planes per row, int32 row scales
  uniform in [1, 4096], int8 hidden state from rounded N(0, 32^2);
* ``q1``       -- iid equiprobable signs {-1, +1}, int16 group scales uniform
  in [1, 4096], int8 activations from rounded N(0, 32^2).
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# BitNet-b1.58-2B-shaped decode projections (N x K): q/o, k/v, gate/up, down.
BITNET2B_SHAPES = {
    "q": (2560, 2560), "k": (640, 2560), "v": (640, 2560), "o": (2560, 2560),
    "gate": (6912, 2560), "up": (6912, 2560), "down": (2560, 6912),
}
# Larger-K projections.
LARGE_K_SHAPES = [(11008, 4096), (4096, 11008), (13824, 5120), (5120, 13824)]
TINY_SHAPE = (256, 512)
LNS8_SHAPE = (4096, 4096)
LMHEAD_SHAPE = (128256, 2560)


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _trits(rng, shape, p_zero: float) -> np.ndarray:
    """iid trits; p_zero = 1/3 gives uniform {-1,0,+1}; p_zero = 0.4 gives
    P(0) = 0.4 and P(+1) = P(-1) = 0.3; any other p_zero in [0, 1] gives
    P(0) = p_zero with equiprobable signs."""
    if abs(p_zero - 1.0 / 3.0) < 1e-12:
        t = rng.integers(0, 3, size=shape, dtype=np.int8)
        t -= 1
        return t
    if abs(p_zero - 0.4) < 1e-12:
        u = rng.integers(0, 10, size=shape, dtype=np.int8)
        lut = np.array([0, 0, 0, 0, 1, 1, 1, -1, -1, -1], dtype=np.int8)
        return lut[u]
    if not 0.0 <= p_zero <= 1.0:
        raise ValueError("p_zero must be in [0, 1]")
    # any other zero density (the Phase B sweeps): P(+1) = P(-1)
    u = rng.random(size=shape)
    t = np.where(u < p_zero, 0, np.where(u < p_zero + (1.0 - p_zero) / 2.0, 1, -1))
    return t.astype(np.int8)


def _act_normal32(rng, k: int) -> np.ndarray:
    v = np.rint(rng.normal(0.0, 32.0, size=k))
    return np.clip(v, -127, 127).astype(np.int8)


def ternary(rows: int, k: int, seed: int, p_zero: float = 0.4, act: str = "normal32"):
    """(t int8[rows][k], scales int16[rows][k/128], x int8[k])."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 128")
    rt, rs, rx = _streams(seed, 3)
    t = _trits(rt, (rows, k), p_zero)
    scales = rs.integers(1, 4097, size=(rows, k // GROUP), dtype=np.int16)
    if act == "normal32":
        x = _act_normal32(rx, k)
    elif act == "uniform127":
        x = rx.integers(-127, 128, size=k, dtype=np.int8)
    else:
        raise ValueError(act)
    return t, scales, x


def q1(rows: int, k: int, seed: int):
    """(s int8[rows][k] in {-1, +1}, scales int16[rows][k/128], x int8[k])."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 128")
    rs_, rsc, rx = _streams(seed, 3)
    s = rs_.integers(0, 2, size=(rows, k), dtype=np.int8) * 2 - 1
    scales = rsc.integers(1, 4097, size=(rows, k // GROUP), dtype=np.int16)
    return s.astype(np.int8), scales, _act_normal32(rx, k)


def tiny(seed: int = 0):
    """256 x 512, uniform trits, uniform int8 activations."""
    return ternary(*TINY_SHAPE, seed=seed, p_zero=1.0 / 3.0, act="uniform127")


def lns8(rows: int, k: int, seed: int):
    """(t int8[rows][k] uniform trits, x uint8[k] LNS8 bytes S1<<7 | code)."""
    rt, rsign, rzero, rcode = _streams(seed, 4)
    t = _trits(rt, (rows, k), 1.0 / 3.0)
    sign = rsign.integers(0, 2, size=k, dtype=np.uint8)
    is_zero = rzero.random(size=k) < 0.05
    code = rcode.integers(60, 101, size=k, dtype=np.uint8)
    code = np.where(is_zero, np.uint8(0), code).astype(np.uint8)
    x = ((sign << 7) | code).astype(np.uint8)
    return t, x


def lns8_sweep(rows: int, k: int, seed: int, p_zero: float, n_codes: int):
    """LNS8 inputs for the Phase B sweeps: ternary weights with P(0) = p_zero
    (signs equiprobable), activations with 5% zero codes and the rest uniform
    over ``n_codes`` distinct non-zero codes evenly spread over 1..127 (41
    codes over 60..100 is the workload's own recipe), signs uniform."""
    if not 1 <= n_codes <= 127:
        raise ValueError("n_codes must be in 1..127")
    rt, rsign, rzero, rcode = _streams(seed, 4)
    t = _trits(rt, (rows, k), p_zero)
    codes = np.unique(np.rint(np.linspace(1, 127, n_codes)).astype(np.int64)).astype(np.uint8)
    sign = rsign.integers(0, 2, size=k, dtype=np.uint8)
    is_zero = rzero.random(size=k) < 0.05
    code = codes[rcode.integers(0, codes.size, size=k)]
    code = np.where(is_zero, np.uint8(0), code).astype(np.uint8)
    return t, ((sign << 7) | code).astype(np.uint8)


def lmhead(vocab: int, dim: int, seed: int):
    """(trits int8[vocab][8][dim], row_scale int32[vocab], h int8[dim])."""
    rt, rs, rh = _streams(seed, 3)
    trits = _trits(rt, (vocab, 8, dim), 1.0 / 3.0)
    row_scale = rs.integers(1, 4097, size=vocab, dtype=np.int32)
    h = _act_normal32(rh, dim)
    return trits, row_scale, h


def lmhead_planted(vocab: int, dim: int, seed: int, n_peaks: int = 64):
    """As ``lmhead`` but with ``n_peaks`` rows whose plane-0 trits copy
    sign(h) on a random half of the positions, so a few rows stand far above
    the rest and the candidate set stays small."""
    trits, row_scale, h = lmhead(vocab, dim, seed)
    rp, rpos = _streams(seed + 1_000_003, 2)
    peaks = rp.choice(vocab, size=n_peaks, replace=False)
    sgn = np.sign(h).astype(np.int8)
    for r in peaks:
        pos = rpos.random(size=dim) < 0.5
        trits[r, 0, pos] = sgn[pos]
    return trits, row_scale, h, np.sort(peaks)
