"""GPU parity of bs_flns_phase_gemv (pure fractional-LNS reduction) against
the oracle.  The method is an approximation whose every rounding is
specified, so both sides compute the same integers: (sign, L) must match
bit for bit on every row, at every internal precision.  Sizes span several
16-row workgroups, ragged rows, K over one or several 32-Tile128 chunks
(the tile tree continued across the chunks), the largest K, and the
degenerate inputs of the LNS8 path."""
import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu

_tables = {}


def table_dev(f, dev):
    if f not in _tables:
        _tables[f] = to_dev(bs.flns_table(f), dev)
    return _tables[f]


def check(t, x, f, d=1):
    import torch
    dev = device()
    rows, k = t.shape
    want = oracle.flns_gemv(t, x, f, d)
    planes = to_dev(bs.ternary_pack(t), dev)
    xd = to_dev(x, dev)
    tb = table_dev(f, dev)
    note("flns rows=%d k=%d f=%d d=%d" % (rows, k, f, d))
    out = bs.flns_phase_gemv(planes, xd, rows, k, f, tb, scale_d=d)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.nonzero((got != want).any(1))[0]
    assert bad.size == 0, "%d rows differ, first row %d: %s vs oracle %s" % (
        bad.size, bad[0], got[bad[0]], want[bad[0]])
    return got


@pytest.mark.parametrize("f,seed", [(8, 0), (8, 1), (4, 0), (12, 0)])
def test_flns_config(f, seed):
    """4096 x 4096 ternary weights against LNS8 activations."""
    check(*synth.lns8(4096, 4096, seed), f)


@pytest.mark.parametrize("f", range(13))
def test_flns_every_precision(f):
    check(*synth.lns8(130, 2048, 100 + f), f)


@pytest.mark.parametrize("rows,k", [(1, 128), (63, 256), (65, 1152), (130, 1024), (2000, 128),
                                    (200, 8192), (64, 65408), (16, 4096), (33, 4224),
                                    (17, 12416)])
def test_flns_ragged_and_split(rows, k):
    """One Tile128; nine Tile128s (k = 1152: five wavefronts with a tile,
    one of them with only the first of its pair); eight (1024); one full
    chunk of 32 (4096); 32 + 1 (4224: the second chunk holds one Tile128);
    64 (8192: two chunks); 97 (12416: four chunks, the last short); the
    largest K (511 Tile128s: sixteen chunks).  The last 16-row block is cut
    short at 1, 63, 65, 130, 33 and 17 rows."""
    check(*synth.lns8(rows, k, rows + k), 8)


@pytest.mark.parametrize("d", [3, 1000, 65535, 4294967295])
def test_flns_scale(d):
    check(*synth.lns8(70, 1152, d % 1000), 6, d)


def _adversarial():
    rng = np.random.default_rng(23)
    k = 1152
    t = rng.integers(-1, 2, (70, k)).astype(np.int8)
    yield "all_same_code", t, np.full(k, 80, np.uint8)
    yield "all_zero_code", t, np.zeros(k, np.uint8)
    yield "zero_code_sign_set", t, np.full(k, 0x80, np.uint8)
    yield "code_1", t, (rng.integers(0, 2, k).astype(np.uint8) << 7) | 1
    yield "code_127", t, (rng.integers(0, 2, k).astype(np.uint8) << 7) | 127
    yield "all_bytes", t, rng.integers(0, 256, k).astype(np.uint8)
    tc = np.ones((64, k), np.int8)
    xc = np.full(k, 90, np.uint8)
    xc[1::2] |= 0x80
    yield "cancel_in_tile", tc, xc
    xt = np.zeros(k, np.uint8)
    xt[0:128] = 90
    xt[128:256] = 90 | 0x80
    yield "cancel_across_tiles", tc, xt
    yield "full_tiles_max", -np.ones((64, k), np.int8), np.full(k, 0xFF, np.uint8)
    yield "zero_weights", np.zeros((64, k), np.int8), rng.integers(0, 256, k).astype(np.uint8)


@pytest.mark.parametrize("f", [0, 8])
@pytest.mark.parametrize("case", list(_adversarial()), ids=lambda c: c[0])
def test_flns_adversarial(case, f):
    got = check(case[1], case[2], f)
    if case[0] in ("all_zero_code", "zero_code_sign_set", "cancel_in_tile",
                   "cancel_across_tiles", "zero_weights"):
        assert (got == 0).all()


def _adversarial_long():
    """Adversarial activations over K = 8320 (65 Tile128s: three 32-tile
    chunks, the last holding one), 33 rows."""
    rng = np.random.default_rng(31)
    k = 8320
    t = rng.integers(-1, 2, (33, k)).astype(np.int8)
    yield "all_same_code", t, np.full(k, 80, np.uint8)
    yield "all_bytes", t, rng.integers(0, 256, k).astype(np.uint8)
    xc = np.full(k, 90, np.uint8)
    xc[1::2] |= 0x80
    yield "cancel", np.ones((33, k), np.int8), xc
    yield "full_tiles_max", -np.ones((33, k), np.int8), np.full(k, 0xFF, np.uint8)


@pytest.mark.parametrize("f", [0, 8, 12])
@pytest.mark.parametrize("case", list(_adversarial_long()), ids=lambda c: c[0])
def test_flns_adversarial_long_k(case, f):
    got = check(case[1], case[2], f)
    if case[0] == "cancel":
        assert (got == 0).all()


def test_flns_repeated_calls_share_a_workspace():
    """One workspace serves back-to-back calls of different shapes, every
    result exact; the reduction never writes it, so it stays zero."""
    import torch
    dev = device()
    shapes = ((300, 4096, 1), (300, 4096, 2), (130, 2048, 3), (64, 1024, 5), (1000, 3072, 6),
              (300, 4096, 4), (1000, 3072, 7))
    need = max(int(bs.lib().bs_flns_workspace_bytes(r, k)) for r, k, _ in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for rows, k, seed in shapes:
        t, x = synth.lns8(rows, k, seed)
        want = oracle.flns_gemv(t, x, 8)
        note("flns repeated rows=%d k=%d" % (rows, k))
        out = bs.flns_phase_gemv(to_dev(bs.ternary_pack(t), dev), to_dev(x, dev), rows, k, 8,
                                 table_dev(8, dev), workspace=ws)
        torch.cuda.synchronize()
        assert (out.cpu().numpy() == want).all()
        assert int(ws.count_nonzero().item()) == 0      # left zero for the next call
