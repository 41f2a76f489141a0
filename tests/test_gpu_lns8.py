"""GPU parity of bs_lns8_phase_gemv against the oracle.

A[p] (int32) must be bit-exact for each of the DIRECT, POPCOUNT and MATRIX paths;
S (binary64) must agree with the oracle's exact-then-rounded value within
1e-12 relative, the bound the task sets for the materialised fp64 result.
Both sides evaluate S as the exact sum over the correctly rounded F[p]
rounded once, so they are expected to agree bit for bit; the test states
the 1e-12 bar and reports any inexact row.
"""
import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu
REL_TOL = 1e-12


def run(t, x, path):
    import torch
    dev = device()
    rows, k = t.shape
    planes = to_dev(bs.ternary_pack(t), dev)
    xd = to_dev(x, dev)
    note("lns8 rows=%d k=%d path=%d" % (rows, k, path))
    acc, s = bs.lns8_phase_gemv(planes, xd, rows, k, path)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), s.cpu().numpy()


def check(t, x):
    want_a = oracle.lns8_direct(t, x)
    want_s = oracle.lns8_materialize(want_a)
    results = []
    for path in (bs.LNS8_DIRECT, bs.LNS8_POPCOUNT, bs.LNS8_MATRIX):
        a, s = run(t, x, path)
        bad = np.nonzero((a != want_a).any(1))[0]
        assert bad.size == 0, "path %d row %d: %s vs %s" % (path, bad[0], a[bad[0]], want_a[bad[0]])
        err = np.abs(s - want_s)
        assert (err <= REL_TOL * np.abs(want_s)).all(), "path %d: max rel err %g" % (
            path, (err / np.maximum(np.abs(want_s), 1e-300)).max())
        assert ((s == 0) == (want_s == 0)).all()
        results.append((a, s))
    # the paths return identical bytes
    for a, s in results[1:]:
        assert (results[0][0] == a).all()
        assert (results[0][1].view(np.int64) == s.view(np.int64)).all()
    return results[0][1], want_s


@pytest.mark.parametrize("seed", range(5))
def test_lns8_config(seed):
    s, want = check(*synth.lns8(4096, 4096, seed))
    # exact-then-round on both sides: report, and expect, bit equality
    assert (s.view(np.int64) == want.view(np.int64)).all()


@pytest.mark.parametrize("rows,k", [(1, 128), (63, 256), (65, 128), (130, 1024)])
def test_lns8_ragged(rows, k):
    check(*synth.lns8(rows, k, seed=rows))


def _adversarial():
    rng = np.random.default_rng(17)
    k = 512
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
    yield "cancel", tc, xc
    yield "max_magnitude", -np.ones((64, k), np.int8), np.full(k, 0xFF, np.uint8)


@pytest.mark.parametrize("case", list(_adversarial()), ids=lambda c: c[0])
def test_lns8_adversarial(case):
    check(case[1], case[2])


def _adversarial_long():
    """The adversarial activations over K = 8320 (three 64-unit chunks of the
    popcount kernel, the last holding two units), 33 rows."""
    rng = np.random.default_rng(29)
    k = 8320
    t = rng.integers(-1, 2, (33, k)).astype(np.int8)
    yield "all_same_code", t, np.full(k, 80, np.uint8)
    yield "code_127_signs", t, (rng.integers(0, 2, k).astype(np.uint8) << 7) | 127
    yield "all_bytes", t, rng.integers(0, 256, k).astype(np.uint8)
    xc = np.full(k, 90, np.uint8)
    xc[1::2] |= 0x80
    yield "cancel", np.ones((33, k), np.int8), xc
    yield "max_magnitude", -np.ones((33, k), np.int8), np.full(k, 0xFF, np.uint8)


@pytest.mark.parametrize("case", list(_adversarial_long()), ids=lambda c: c[0])
def test_lns8_adversarial_long_k(case):
    check(case[1], case[2])


@pytest.mark.parametrize("rows,k", [(64, 65408), (200, 8192), (2000, 128), (70, 2048)])
def test_lns8_split_and_long_rows(rows, k):
    """K split over several workgroups per tile (partials combined by the
    last workgroup of each tile) and the largest K whose |A| fits int32;
    2000 x 128 keeps one wavefront per tile."""
    check(*synth.lns8(rows, k, seed=k + rows))


@pytest.mark.parametrize("rows,k", [(17, 4224), (33, 8320), (16, 4096), (15, 256), (48, 384),
                                    (1, 640), (129, 4096), (3, 65408)])
def test_lns8_popcount_chunks(rows, k):
    """The popcount kernel's geometry: 16-row workgroups (ragged last block),
    one to sixteen wavefronts (up to 64 units per chunk), and K beyond one
    chunk with a partly filled last chunk (4224: 64 + 2 units; 8320: 64 + 64
    + 2; 65408: sixteen chunks).  Every path against the oracle."""
    check(*synth.lns8(rows, k, seed=rows * 7 + k))


def test_lns8_max_k_extremes():
    """k = 65408 with every product +2^15 into one phase: |A| reaches
    65408 * 2^15 = 2^31 - 2^22, the int32 bound the shape limit keeps."""
    k = 65408
    t = np.ones((64, k), np.int8)
    check(t, np.full(k, 127, np.uint8))


def test_split_k_counters_reused_across_calls():
    """The split-K reduction's last-workgroup counters live in the caller's
    workspace: one zeroed workspace, many calls of several shapes (all
    paths, growing and shrinking tile counts), every result exact and the
    used workspace zero again after each call."""
    import torch
    dev = device()
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)
    cases = [synth.lns8(4096, 4096, 7), synth.lns8(1000, 2560, 8), synth.lns8(8192, 1024, 9),
             synth.lns8(64, 8192, 10)]
    want = [oracle.lns8_direct(t, x) for t, x in cases]
    dev_in = [(to_dev(bs.ternary_pack(t), dev), to_dev(x, dev)) for t, x in cases]
    for rep in range(6):
        for ci, ((t, x), (pd, xd)) in enumerate(zip(cases, dev_in)):
            rows, k = t.shape
            need = bs.lib().bs_lns8_workspace_bytes(rows, k)
            assert need <= ws.numel()
            path = (rep + ci) % 3
            note("lns8 reuse rep=%d case=%d path=%d" % (rep, ci, path))
            acc, _ = bs.lns8_phase_gemv(pd, xd, rows, k, path, s=False, workspace=ws)
            torch.cuda.synchronize()
            assert (acc.cpu().numpy() == want[ci]).all(), (rep, ci, path)
            assert int(ws[:need].view(torch.int32).abs().sum().item()) == 0, (rep, ci)


@pytest.mark.parametrize("p_zero,n_codes", [(0.0, 41), (0.9, 41), (1 / 3, 1), (1 / 3, 8),
                                            (1 / 3, 127), (0.6, 127)])
def test_phase_b_inputs(p_zero, n_codes):
    """The inputs of the benchmark's Phase B sweeps (weight zero density,
    number of distinct activation codes)."""
    check(*synth.lns8_sweep(512, 4096, 3, p_zero, n_codes))
