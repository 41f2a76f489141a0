"""GPU parity of bs_q1_gemv (Q1_0 weight apply) against the oracle's
definition form, bit-exact int64: the BitNet-2B projection shapes and the
larger-K shapes at full size, ragged shapes, every frac with negative scales,
and the extremes (all +1, all -1, x = -128, scale -32768, one-hot x)."""
import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu


def check(s, sc, x, frac=0):
    import torch
    dev = device()
    rows, k = s.shape
    note("q1_gemv rows=%d k=%d frac=%d" % (rows, k, frac))
    y = bs.q1_gemv(to_dev(bs.q1_pack(s), dev), to_dev(bs.ternary_pack_scales(sc), dev),
                   to_dev(x, dev), rows, k, frac)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    want = oracle.q1_gemv_def(s, sc, x, frac)
    bad = np.nonzero(y != want)[0]
    assert bad.size == 0, "first mismatch row %d: got %d want %d (%d bad)" % (
        bad[0], y[bad[0]], want[bad[0]], bad.size)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("rows,k", [(2560, 2560), (640, 2560), (6912, 2560), (2560, 6912),
                                    (3840, 2560), (13824, 2560)])
def test_bitnet2b_shapes(rows, k, seed):
    check(*synth.q1(rows, k, seed))


@pytest.mark.parametrize("shape", synth.LARGE_K_SHAPES)
def test_large_k(shape):
    check(*synth.q1(shape[0], shape[1], 0))


@pytest.mark.parametrize("rows,k", [(9600, 3840), (9601, 3968), (12800, 6144), (12801, 6272),
                                    (4999, 4224), (5000, 4224), (5001, 12800)])
def test_mapping_edges(rows, k):
    """Tall shapes with 30 to 100 groups (ragged last blocks, more groups than
    one wavefront's slices)."""
    check(*synth.q1(rows, k, rows ^ k))


@pytest.mark.parametrize("rows,k", [(4999, 16512), (5000, 16512), (5001, 20480)])
def test_row_block_kernel_beyond_128_groups(rows, k):
    """K > 16384 takes the row-block kernel: 16-row blocks below 5000 rows,
    32-row blocks with two groups per slice and round from 5000."""
    check(*synth.q1(rows, k, rows + k))


@pytest.mark.parametrize("rows,k", [(4096, 3072), (4097, 3072), (4097, 128), (1, 128),
                                    (13824, 2560), (10239, 2560), (10240, 2560), (10240, 128),
                                    (10240, 256), (10240, 1152), (12000, 3072), (6399, 5120),
                                    (6400, 5120), (10239, 5120), (10240, 5120), (300, 16384),
                                    (1, 16384), (2000, 16512), (9, 1152), (17, 4224)])
def test_pipelined_launch_rule(rows, k):
    """Either side of the Q1_0 table of the pipelined kernel: up to 24 groups
    16-row blocks with 2 groups per slice up to 4096 rows, whole 64-row tiles
    of 4 wavefronts from 10240 (1 to 3 groups in flight), 32-row blocks of 4
    between; the ternary table's blocks beyond; 129 groups take the row-block
    kernel."""
    check(*synth.q1(rows, k, rows + k))


@pytest.mark.parametrize("rows,k", [(1, 128), (63, 128), (65, 256), (130, 384), (127, 6912),
                                    (200, 128 * 100), (80, 128 * 217), (9600, 2560),
                                    (13800, 2560), (12863, 6144), (14000, 128)])
def test_ragged(rows, k):
    check(*synth.q1(rows, k, rows + k))


@pytest.mark.parametrize("rows", [130, 9700])
@pytest.mark.parametrize("frac", [0, 1, 16, 31, 32, 62])
def test_frac_with_negative_scales(frac, rows):
    s, _, x = synth.q1(rows, 640, frac)
    sc = np.random.default_rng(frac).integers(-32768, 32768, (rows, 5)).astype(np.int16)
    check(s, sc, x, frac)


def test_extremes():
    rows, k = 96, 512
    x = np.full(k, -128, np.int8)
    sc = np.full((rows, 4), -32768, np.int16)
    check(np.ones((rows, k), np.int8), sc, x)
    check(-np.ones((rows, k), np.int8), sc, x)
    s, sc, _ = synth.q1(rows, k, 5)
    for i in (0, 31, 64, 127, 128, 511):      # one-hot x pins the bit order on the device
        xo = np.zeros(k, np.int8)
        xo[i] = 1
        check(s, sc, xo)


def test_max_k():
    """K = 2^24, the largest the int64 accumulation bound allows."""
    s, sc, x = synth.q1(1, 1 << 24, 24)
    check(s, np.full_like(sc, -32768), x)
