"""Seeded random-shape parity sweep: every entry point on the hot path and
its next rows against the oracle, at shapes drawn from one fixed seed (rows
log-uniform, K any multiple of 128 up to past the pipelined kernel's 128
groups, ragged everywhere), with random zero densities, activation
distributions, frac, internal precisions, k and cap.  Each case is small
enough for the oracle to finish in well under a second; the fixed cases of
the per-entry-point files pin the configurations themselves."""
import numpy as np
import pytest

from bit_decode_gemv_amd import synth

import test_gpu_flns
import test_gpu_lmhead
import test_gpu_lns8
import test_gpu_q1
import test_gpu_ternary

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)


def _rows(lo, hi):
    return int(np.exp(_rng.uniform(np.log(lo), np.log(hi))))


def _groups(hi):
    return int(_rng.integers(1, hi + 1))


def _shape(rows_hi, groups_hi, max_weights=8 << 20):
    """rows log-uniform, K uniform in groups, rows cut so the oracle stays fast"""
    rows, k = _rows(1, rows_hi), 128 * _groups(groups_hi)
    return max(1, min(rows, max_weights // k)), k


TERNARY = [_shape(6000, 140) + (int(_rng.integers(0, 1 << 20)),
                                float(_rng.choice([0.0, 1 / 3, 0.4, 0.9, 1.0])),
                                str(_rng.choice(["normal32", "uniform127"])),
                                int(_rng.choice([0, 0, 3, 17, 40])))
           for _ in range(24)]
Q1 = [_shape(6000, 140) + (int(_rng.integers(0, 1 << 20)), int(_rng.choice([0, 0, 5, 31])))
      for _ in range(16)]
LNS8 = [(_rows(1, 700), 128 * _groups(80), int(_rng.integers(0, 1 << 20)),
         float(_rng.choice([0.0, 1 / 3, 0.9])), int(_rng.choice([1, 8, 41, 127])))
        for _ in range(12)]
FLNS = [(_rows(1, 300), 128 * _groups(40), int(_rng.integers(0, 1 << 20)),
         int(_rng.integers(0, 13))) for _ in range(10)]
LMHEAD = []
for _ in range(12):
    _v = _rows(40, 20000)
    _k = int(_rng.integers(1, min(40, _v) + 1))
    _cap = int(_rng.integers(_k, 513))
    LMHEAD.append((_v, 128 * int(_rng.integers(1, 5)), _k, _cap, int(_rng.integers(0, 1 << 20))))


@pytest.mark.parametrize("rows,k,seed,p_zero,act,frac", TERNARY)
def test_ternary_random(rows, k, seed, p_zero, act, frac):
    test_gpu_ternary.check(*synth.ternary(rows, k, seed, p_zero=p_zero, act=act), frac)


@pytest.mark.parametrize("rows,k,seed,frac", Q1)
def test_q1_random(rows, k, seed, frac):
    test_gpu_q1.check(*synth.q1(rows, k, seed), frac)


@pytest.mark.parametrize("rows,k,seed,p_zero,n_codes", LNS8)
def test_lns8_random(rows, k, seed, p_zero, n_codes):
    test_gpu_lns8.check(*synth.lns8_sweep(rows, k, seed, p_zero, n_codes))


@pytest.mark.parametrize("rows,k,seed,f", FLNS)
def test_flns_random(rows, k, seed, f):
    t, x = synth.lns8(rows, k, seed)
    test_gpu_flns.check(t, x, f)


# long K for the chunked kernels (LNS8 popcount: 64 units per chunk; pure
# LNS: 32 Tile128s per chunk), from a generator of their own so the cases
# above stay as they were
_rng2 = np.random.default_rng(20261203)
LNS8_LONG = [(int(_rng2.integers(1, 80)), 128 * int(_rng2.integers(81, 320)),
              int(_rng2.integers(0, 1 << 20)), float(_rng2.choice([0.0, 1 / 3])),
              int(_rng2.choice([8, 41, 127]))) for _ in range(6)]
FLNS_LONG = [(int(_rng2.integers(1, 70)), 128 * int(_rng2.integers(41, 200)),
              int(_rng2.integers(0, 1 << 20)), int(_rng2.integers(0, 13))) for _ in range(6)]


@pytest.mark.parametrize("rows,k,seed,p_zero,n_codes", LNS8_LONG)
def test_lns8_random_long_k(rows, k, seed, p_zero, n_codes):
    test_gpu_lns8.check(*synth.lns8_sweep(rows, k, seed, p_zero, n_codes))


@pytest.mark.parametrize("rows,k,seed,f", FLNS_LONG)
def test_flns_random_long_k(rows, k, seed, f):
    t, x = synth.lns8(rows, k, seed)
    test_gpu_flns.check(t, x, f)


@pytest.mark.parametrize("V,K,top_k,cap,seed", LMHEAD)
def test_lmhead_random(V, K, top_k, cap, seed):
    test_gpu_lmhead.check(*synth.lmhead(V, K, seed), top_k, cap)
