"""GPU parity of bs_ternary_gemv against the oracle (bit-exact int64).

Covers the tiny case, the BitNet-2B decode projection shapes (seeds 0..4) and
the larger-K shapes (seeds 0..4) at full size in the launch configuration the
benchmark times, plus ragged and degenerate cases: single rows, row counts
off the 64-row tile, K = 128, all-zero weights, x = -128, extreme scales,
every frac, workspace reuse across shapes, and run-to-run byte identity.
"""
import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu


def run(t, sc, x, frac=0, dev=None):
    dev = dev or device()
    rows, k = t.shape
    planes = to_dev(bs.ternary_pack(t), dev)
    scales = to_dev(bs.ternary_pack_scales(sc), dev)
    xd = to_dev(x, dev)
    note("ternary_gemv rows=%d k=%d frac=%d" % (rows, k, frac))
    y = bs.ternary_gemv(planes, scales, xd, rows, k, frac)
    import torch
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(t, sc, x, frac=0):
    y = run(t, sc, x, frac)
    want = oracle.ternary_gemv_def(t, sc, x, frac)
    bad = np.nonzero(y != want)[0]
    assert bad.size == 0, "first mismatch row %d: got %d want %d (%d bad)" % (
        bad[0], y[bad[0]], want[bad[0]], bad.size)


def test_tiny_config():
    check(*synth.tiny(0))


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_bitnet2b_projections(name, seed):
    rows, k = synth.BITNET2B_SHAPES[name]
    check(*synth.ternary(rows, k, seed))


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("rows", [3840, 13824])
def test_fused_launches(rows, seed):
    """The benchmark's launches: q|k|v (3840 x 2560) and gate|up (13824 x 2560)
    stored concatenated by rows."""
    check(*synth.ternary(rows, 2560, seed))


@pytest.mark.parametrize("rows,k", [(9600, 2560), (9601, 3072), (12800, 3200), (12863, 6144),
                                    (13800, 2560), (12800, 640), (14000, 128),
                                    (9536, 4096), (9600, 4096), (9601, 4224), (12800, 8192),
                                    (12737, 8320), (4999, 4224), (5000, 4224)])
def test_tall_shapes(rows, k):
    """Tall shapes with 1 to 65 groups around 150 and 200 tiles and 5000 rows:
    ragged last tiles and blocks, fewer groups than wavefronts."""
    check(*synth.ternary(rows, k, seed=rows ^ k, p_zero=1 / 3, act="uniform127"))


@pytest.mark.parametrize("rows,k", [(1024, 2560), (1025, 2560), (2047, 2560), (2048, 2560),
                                    (4096, 2560), (4097, 2560), (4097, 256), (8191, 2560),
                                    (8192, 2560), (10239, 2560), (10240, 2560), (10240, 128),
                                    (10240, 1152), (12000, 3072), (10239, 4096), (10240, 4096),
                                    (6399, 5120), (6400, 5120), (10240, 5120), (8192, 8192),
                                    (8192, 8320), (8255, 1024), (2000, 16384), (2000, 16512),
                                    (1023, 128 * 127), (300, 16384), (7, 2560), (9, 1152),
                                    (17, 4224), (1, 16384), (4096, 3072), (4097, 3072),
                                    (4097, 128), (13824, 2560)])
def test_pipelined_launch_rule(rows, k):
    """Either side of the pipelined kernel's launch-shape bounds: up to 24
    groups 8-row blocks under 2048 rows, 16-row blocks to 4096, 32-row blocks
    to 10240 and whole 64-row tiles from there (1 to 6 groups per slice); up
    to 40 groups whole tiles from 10240 rows, 32-row blocks from 6400, else
    16-row blocks with 2 groups per slice; 8 wavefronts of 16-row blocks up
    to 96 groups, 32-row blocks of 8 up to 128 (129 takes the row-block
    kernel); ragged blocks and tiles, fewer groups than slices."""
    check(*synth.ternary(rows, k, seed=rows + k, p_zero=1 / 3, act="uniform127"))


@pytest.mark.parametrize("groups", [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 40, 63, 64, 65,
                                    86, 100, 108, 120, 127, 128])
@pytest.mark.parametrize("rows", [40, 1500, 8200, 10300])
def test_pipelined_wavefront_counts(groups, rows):
    """Every wavefront count and groups-per-slice of the pipelined kernel
    (padding slots past K, partly filled last rounds)."""
    check(*synth.ternary(rows, 128 * groups, seed=groups * 7 + rows, p_zero=0.4))


@pytest.mark.parametrize("rows,k", [(4999, 16512), (5000, 16512), (5001, 20480)])
def test_row_block_kernel_beyond_128_groups(rows, k):
    """K > 16384 takes the row-block kernel: 16-row blocks below 5000 rows,
    32-row blocks from 5000 (ragged last block)."""
    check(*synth.ternary(rows, k, seed=rows + k, p_zero=1 / 3, act="uniform127"))


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("shape", synth.LARGE_K_SHAPES)
def test_large_k(shape, seed):
    check(*synth.ternary(shape[0], shape[1], seed))


@pytest.mark.parametrize("rows,k", [(1, 128), (63, 128), (65, 256), (130, 384), (1, 2560),
                                    (127, 6912), (200, 128 * 100)])
def test_ragged_shapes(rows, k):
    check(*synth.ternary(rows, k, seed=rows + k, p_zero=1 / 3, act="uniform127"))


@pytest.mark.parametrize("rows", [130, 9700])
@pytest.mark.parametrize("frac", [0, 1, 3, 16, 29, 30, 31, 32, 62])
def test_frac_with_negative_scales(frac, rows):
    t, _, x = synth.ternary(rows, 640, seed=frac, p_zero=1 / 3, act="uniform127")
    rng = np.random.default_rng(frac)
    sc = rng.integers(-32768, 32768, (rows, 5)).astype(np.int16)
    check(t, sc, x, frac)


def test_degenerate_values():
    for rows, k in ((96, 512), (9664, 512)):
        _degenerate(rows, k)


def _degenerate(rows, k):
    # all-zero weights
    check(np.zeros((rows, k), np.int8), np.ones((rows, 4), np.int16),
          np.full(k, 7, np.int8))
    # largest magnitudes: t = -1, x = -128, scale = -32768
    check(-np.ones((rows, k), np.int8), np.full((rows, 4), -32768, np.int16),
          np.full(k, -128, np.int8))
    # one-hot activations pin the bit order of the codec on the device
    t, sc, _ = synth.ternary(rows, k, seed=3, p_zero=1 / 3)
    for i in (0, 1, 31, 32, 63, 64, 127, 128, 300, 511):
        x = np.zeros(k, np.int8)
        x[i] = 1
        check(t, sc, x)


def test_determinism():
    for t, sc, x in [synth.ternary(13824, 5120, 7), synth.ternary(640, 2560, 8),
                     synth.ternary(2560, 6912, 9), synth.ternary(65, 256, 10)]:
        a = run(t, sc, x)
        b = run(t, sc, x)
        assert (a == b).all()
        assert (a == oracle.ternary_gemv_def(t, sc, x)).all()


@pytest.mark.parametrize("k", [128 * 216, 128 * 217, 128 * 450])
def test_k_beyond_one_lds_chunk(k):
    """K larger than the activation planes one workgroup keeps in LDS."""
    check(*synth.ternary(80, k, seed=k, p_zero=1 / 3, act="uniform127"))


def check_acc(t, sc, x, frac=0, times=1, seed=0):
    """y0 + times * (W x) through bs_ternary_gemv_acc, against the oracle."""
    import torch
    dev = device()
    rows, k = t.shape
    y0 = np.random.default_rng(seed).integers(-(1 << 50), 1 << 50, rows).astype(np.int64)
    planes = to_dev(bs.ternary_pack(t), dev)
    scales = to_dev(bs.ternary_pack_scales(sc), dev)
    xd = to_dev(x, dev)
    y = to_dev(y0, dev)
    note("ternary_gemv_acc rows=%d k=%d frac=%d times=%d" % (rows, k, frac, times))
    for _ in range(times):
        bs.ternary_gemv_acc(planes, scales, xd, rows, k, y, frac)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = y0 + times * oracle.ternary_gemv_def(t, sc, x, frac)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "first mismatch row %d: got %d want %d (%d bad)" % (
        bad[0], got[bad[0]], want[bad[0]], bad.size)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("rows,k", [(2560, 2560), (2560, 6912), (640, 2560), (3840, 2560),
                                    (13824, 2560), (6912, 2560)])
def test_acc_bitnet2b_shapes(rows, k, seed):
    """y += W x on the decode layer's shapes (o and down add into the residual)."""
    check_acc(*synth.ternary(rows, k, seed), seed=seed)


@pytest.mark.parametrize("shape", synth.LARGE_K_SHAPES)
def test_acc_large_k(shape):
    check_acc(*synth.ternary(shape[0], shape[1], 1), seed=1)


@pytest.mark.parametrize("rows,k", [(1, 128), (63, 128), (65, 256), (130, 384), (200, 12800),
                                    (80, 128 * 450), (9700, 640), (13800, 2560)])
def test_acc_ragged_and_repeated(rows, k):
    t, sc, x = synth.ternary(rows, k, seed=rows + k, p_zero=1 / 3, act="uniform127")
    check_acc(t, sc, x, times=3, seed=rows)


@pytest.mark.parametrize("frac", [0, 3, 31, 62])
def test_acc_frac_and_extremes(frac):
    t, _, x = synth.ternary(2560, 1280, seed=frac, p_zero=1 / 3, act="uniform127")
    sc = np.random.default_rng(frac).integers(-32768, 32768, (2560, 10)).astype(np.int16)
    check_acc(t, sc, x, frac, seed=frac)
    rows, k = 640, 2560
    check_acc(-np.ones((rows, k), np.int8), np.full((rows, 20), -32768, np.int16),
              np.full(k, -128, np.int8), frac, times=2)


@pytest.mark.parametrize("rows,k", [(13824, 2560), (2560, 6912), (640, 2560), (11008, 4096),
                                    (5120, 13824)])
def test_launch_geometry_invariance(rows, k):
    """The storing kernels (row blocks or one workgroup per tile) and the
    accumulating kernel (runs of groups over many workgroups, atomics) split
    the same sum differently; integer addition makes their bytes identical
    (integer-engine page, sections 3.2 and 11)."""
    import torch
    dev = device()
    t, sc, x = synth.ternary(rows, k, seed=rows % 97)
    planes = to_dev(bs.ternary_pack(t), dev)
    scales = to_dev(bs.ternary_pack_scales(sc), dev)
    xd = to_dev(x, dev)
    note("launch geometry rows=%d k=%d" % (rows, k))
    y_store = bs.ternary_gemv(planes, scales, xd, rows, k)
    y_acc = torch.zeros(rows, dtype=torch.int64, device=dev)
    bs.ternary_gemv_acc(planes, scales, xd, rows, k, y_acc)
    torch.cuda.synchronize()
    a, b = y_store.cpu().numpy(), y_acc.cpu().numpy()
    assert a.tobytes() == b.tobytes()
    assert (a == oracle.ternary_gemv_def(t, sc, x)).all()


def test_max_k():
    """K = 2^24, the largest the int64 accumulation bound allows: one row, the
    storing and the accumulating kernels."""
    k = 1 << 24
    t, sc, x = synth.ternary(1, k, seed=24, p_zero=1 / 3, act="uniform127")
    sc = np.full_like(sc, -32768)
    x[::3] = -128
    check(t, sc, x)
    check_acc(t, sc, x, seed=24)
