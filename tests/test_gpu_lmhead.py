"""GPU parity of bs_lmhead_planes_topk against the oracle.

The GPU result (top-k indices, exact int64 scores, |C| and the cap flag)
must equal the oracle's step-by-step two-stage algorithm bit for bit on every
input.  Where the cap does not engage the oracle's result equals the brute
force (pinned in the oracle tests), so the GPU result is then the exact
top-k; where it engages, agreement with brute force is recorded.
"""
import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu
_NO_T1 = -(1 << 63)   # the workspace's T1 when every candidate is rescored


def run(trits, rs, h, top_k, cap, packed=None):
    import torch
    dev = device()
    V, _, K = trits.shape
    p03, p47 = packed if packed is not None else bs.planes_pack(trits)
    note("lmhead V=%d K=%d k=%d cap=%d" % (V, K, top_k, cap))
    idx, sc, info = bs.lmhead_planes_topk(to_dev(p03, dev), to_dev(p47, dev), to_dev(rs, dev),
                                          to_dev(h, dev), V, K, top_k, cap)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy(), info.cpu().numpy()


def check(trits, rs, h, top_k, cap, packed=None):
    idx, sc, info = run(trits, rs, h, top_k, cap, packed)
    widx, wsc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, top_k, cap,
                                                         certificate=True)
    assert list(info) == [n, capped, cert], (info, n, capped, cert)
    assert (idx == widx).all(), (idx[:10], widx[:10])
    assert (sc == wsc).all()
    return idx, sc, n, capped


@pytest.mark.parametrize("V,K,k,cap,seed", [(300, 128, 40, 200, 0), (257, 256, 7, 50, 1),
                                             (64, 128, 1, 1, 2), (100, 128, 100, 100, 3),
                                             (1000, 256, 40, 200, 4), (2049, 384, 16, 32, 5),
                                             (5000, 128, 40, 4096, 6),
                                             # the top-k by S' includes a row the cap
                                             # drops (the finishing pass falls back to
                                             # ranking every gathered row) / does not
                                             (4000, 256, 20, 20, 91), (3000, 256, 10, 10, 92)])
def test_small_random(V, K, k, cap, seed):
    check(*synth.lmhead(V, K, seed), k, cap)


def test_planted_exact_branch():
    trits, rs, h, peaks = synth.lmhead_planted(4000, 512, 1, n_peaks=64)
    idx, sc, n, capped = check(trits, rs, h, 40, 200)
    assert capped == 0
    bi, bsc = oracle.lmhead_brute(trits, rs, h, 40)
    assert (idx == bi).all() and (sc == bsc).all()


def test_exactly_ternary_source():
    trits, rs, h = synth.lmhead(700, 256, 7)
    trits[:, 1:, :] = 0
    idx, sc, _, _ = check(trits, rs, h, 40, 200)
    bi, bsc = oracle.lmhead_brute(trits, rs, h, 40)
    assert (idx == bi).all() and (sc == bsc).all()


def test_all_zero_planes_ties():
    trits = np.zeros((450, 8, 128), np.int8)
    _, rs, h = synth.lmhead(450, 128, 8)
    idx, sc, n, capped = check(trits, rs, h, 40, 200)
    assert n == 450 and capped == 1
    assert (idx == np.arange(40)).all() and not sc.any()


def test_negative_row_scales():
    trits, rs, h = synth.lmhead(600, 256, 9)
    rs = rs * np.where(np.arange(600) % 3 == 0, -1, 1).astype(np.int32)
    check(trits, rs, h, 20, 100)


@pytest.mark.slow
def test_full_vocab_config():
    """vocab 128256 x dim 2560, k = 40, cap = 200, seed 0; the benchmark's
    lm_head workload, where the select kernel names the rescoring bound T1
    (its intermediate values are checked against the oracle's stage 1)."""
    import torch
    trits, rs, h = synth.lmhead(*synth.LMHEAD_SHAPE, seed=0)
    V, _, K = trits.shape
    dev = device()
    ws = torch.zeros(bs.lib().bs_lmhead_workspace_bytes(V, K, 40, 200), dtype=torch.uint8,
                     device=dev)
    p03, p47 = bs.planes_pack(trits)
    note("lmhead full vocab V=%d K=%d" % (V, K))
    bs.lmhead_planes_topk(to_dev(p03, dev), to_dev(p47, dev), to_dev(rs, dev), to_dev(h, dev),
                          V, K, 40, 200, workspace=ws)
    torch.cuda.synchronize()
    lk_gpu, habs_gpu, t1 = (int(v) for v in ws[:24].view(torch.int64).cpu().tolist())
    s1, bnd = oracle.lmhead_stage1(trits, rs, h)
    assert habs_gpu == int(np.abs(h.astype(np.int64)).sum())
    assert lk_gpu == int(np.sort(s1 - bnd)[::-1][39])
    assert t1 != _NO_T1 and t1 >= lk_gpu and int((s1 >= t1).sum()) >= 200
    assert t1 <= int(np.sort(s1)[::-1][199])
    check(trits, rs, h, 40, 200, packed=(p03, p47))


@pytest.mark.slow
@pytest.mark.parametrize("seed", range(5))
def test_full_vocab_seeds_against_recorded_brute_force(seed):
    """The full-vocabulary workload, seeds 0..4, against the oracle's results
    recorded in tests/golden/lmhead_c5_record.json (written by
    make_lmhead_c5_record.py from the oracle alone): the GPU equals the
    two-stage decode bit for bit (indices, scores, |C|, capped, certificate),
    and where the record shows the two-stage result equal to the brute-force
    exact top-k, the GPU result is asserted equal to the brute force too."""
    import json
    import os
    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "lmhead_c5_record.json")))["seeds"][str(seed)]
    trits, rs, h = synth.lmhead(*synth.LMHEAD_SHAPE, seed=seed)
    idx, sc, info = run(trits, rs, h, 40, 200)
    del trits
    assert list(info) == [rec["n_candidates"], rec["capped"], rec["certified"]]
    assert idx.tolist() == rec["two_stage_idx"] and sc.tolist() == rec["two_stage_score"]
    assert rec["equals_brute_force"] == (rec["two_stage_idx"] == rec["brute_idx"] and
                                         rec["two_stage_score"] == rec["brute_score"])
    if rec["equals_brute_force"]:
        assert idx.tolist() == rec["brute_idx"] and sc.tolist() == rec["brute_score"]


def test_workspace_shared_across_shapes():
    """One workspace serves calls of different shapes and needs no
    initialisation: it starts filled with 0xFF bytes, and each call leaves
    scratch that a later call of another shape must not read (regression: a
    candidate counter once moved with the shape and landed on scratch left by
    a larger call)."""
    import torch
    dev = device()
    ws = torch.full((bs.lib().bs_lmhead_workspace_bytes(3000, 256, 40, 200),), 255,
                    dtype=torch.uint8, device=dev)
    for V, K, k, cap, seed in [(3000, 256, 40, 200, 11), (257, 256, 7, 50, 12),
                               (2000, 128, 40, 200, 13), (300, 128, 40, 200, 14)]:
        trits, rs, h = synth.lmhead(V, K, seed)
        p03, p47 = bs.planes_pack(trits)
        note("lmhead shared workspace V=%d K=%d" % (V, K))
        idx, sc, info = bs.lmhead_planes_topk(to_dev(p03, dev), to_dev(p47, dev),
                                              to_dev(rs, dev), to_dev(h, dev), V, K, k, cap,
                                              workspace=ws)
        torch.cuda.synchronize()
        widx, wsc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, k, cap,
                                                             certificate=True)
        assert (idx.cpu().numpy() == widx).all() and (sc.cpu().numpy() == wsc).all()
        assert list(info.cpu().numpy()) == [n, capped, cert]


@pytest.mark.parametrize("V,cap", [(4096, 4096), (4097, 4096), (5000, 200)])
def test_all_zero_planes_candidate_counts(V, cap):
    """Every row ties, so |C| = V: at 4096 candidates the finishing pass holds
    them in registers, above that it reads them from the workspace."""
    trits = np.zeros((V, 8, 128), np.int8)
    _, rs, h = synth.lmhead(V, 128, 15)
    idx, sc, n, capped = check(trits, rs, h, 40, cap)
    assert n == V and capped == int(V > cap)
    assert (idx == np.arange(40)).all() and not sc.any()


def test_many_lower_bounds():
    """top_k = 500 over 40 stage-1 workgroups: 20000 lower bounds, more than
    the selection pass keeps in registers."""
    check(*synth.lmhead(20000, 128, 16), 500, 1000)


@pytest.mark.parametrize("zero", [False, True])
def test_more_filter_regions_than_one_pass(zero):
    """270000 rows: 1055 filter workgroups, more than the finishing pass scans
    at once, so the candidates are compacted first.  With all-zero planes
    every row ties: the selection pass then finds every tile at the bound and
    selects over the whole vocabulary."""
    V, K = 270000, 128
    trits, rs, h = synth.lmhead(V, K, 17)
    if zero:
        trits[:] = 0
    idx, sc, n, capped = check(trits, rs, h, 40, 200)
    if zero:
        assert n == V and (idx == np.arange(40)).all()


def test_max_dim():
    """dim = 10112, the largest the int64 score bound allows (79 groups)."""
    check(*synth.lmhead(300, 10112, 17), 40, 200)


# The selection kernel may name a bound T1 <= the cap-th largest S1' such that
# every row with S1' >= T1 is a candidate; the filter then rescores only those
# rows.  T1 is the workspace's third int64 (INT64_MIN when every candidate is
# rescored); the cases below pin which way each input goes, so each branch of
# the finishing pass is reached, and check the result against the oracle.


def _copies_of_top(V, K, seed, n, levels=None):
    """n random rows replaced by the row with the largest S1' (its trits; its
    row scale, or one drawn from `levels`): ties and near-ties at the top."""
    trits, rs, h = synth.lmhead(V, K, seed)
    s1, _ = oracle.lmhead_stage1(trits, rs, h)
    top = int(np.argmax(s1))
    rng = np.random.default_rng(seed + 7)
    rows = rng.choice(V, n, replace=False)
    trits[rows] = trits[top]
    rs[rows] = rs[top] if levels is None else rng.choice(levels, n).astype(np.int32)
    return trits, rs, h


@pytest.mark.parametrize("case", ["rand_k10_cap64", "rand_k10_cap100", "levels_head_prune",
                                  "ties_list_overflow", "zero_few_regions", "zero_many",
                                  "rand_bound_below_lk"])
def test_rescore_bound_branches(case):
    import torch
    trits = None
    if case == "rand_k10_cap64":          # T1 named, ~72 rows rescored
        (trits, rs, h), k, cap, named = synth.lmhead(20000, 2560, 33), 10, 64, True
    elif case == "rand_k10_cap100":       # T1 named, ~119 rows rescored
        (trits, rs, h), k, cap, named = synth.lmhead(30000, 2560, 43), 10, 100, True
    elif case == "levels_head_prune":     # 600 rescored; region heads prune to ~200
        trits, rs, h = _copies_of_top(20000, 2560, 71, 600, [4094, 4095, 4096])
        k, cap, named = 10, 64, True
    elif case == "ties_list_overflow":    # 600 exact ties: past the LDS list
        trits, rs, h = _copies_of_top(20000, 2560, 51, 600)
        k, cap, named = 10, 64, True
    elif case == "zero_few_regions":      # every row ties, 12 regions < cap
        _, rs, h = synth.lmhead(3000, 128, 52)
        trits, k, cap, named = np.zeros((3000, 8, 128), np.int8), 10, 40, True
    elif case == "zero_many":             # every row ties, 20000 rescored
        _, rs, h = synth.lmhead(20000, 128, 53)
        trits, k, cap, named = np.zeros((20000, 8, 128), np.int8), 10, 40, True
    else:                                 # enough tiles, but T1 < L_k
        (trits, rs, h), k, cap, named = synth.lmhead(13000, 2560, 31), 40, 200, False
    dev = device()
    V, _, K = trits.shape
    p03, p47 = bs.planes_pack(trits)
    ws = torch.zeros(bs.lib().bs_lmhead_workspace_bytes(V, K, k, cap), dtype=torch.uint8,
                     device=dev)
    note("lmhead rescore bound %s V=%d K=%d k=%d cap=%d" % (case, V, K, k, cap))
    idx, sc, info = bs.lmhead_planes_topk(to_dev(p03, dev), to_dev(p47, dev), to_dev(rs, dev),
                                          to_dev(h, dev), V, K, k, cap, workspace=ws)
    torch.cuda.synchronize()
    lk_gpu, habs_gpu, t1 = (int(v) for v in ws[:24].view(torch.int64).cpu().tolist())
    assert (t1 != _NO_T1) == named, t1
    # the intermediate values against the oracle's stage 1: sum|h| and L_k
    # exactly, and a named T1 where the rescoring argument needs it (every row
    # with S1' >= T1 a candidate, at least cap rows reaching it, so the cap
    # lies among them)
    s1, bnd = oracle.lmhead_stage1(trits, rs, h)
    assert habs_gpu == int(np.abs(h.astype(np.int64)).sum())
    lk = int(np.sort(s1 - bnd)[::-1][k - 1])
    assert lk_gpu == lk
    if named:
        assert t1 >= lk
        assert int((s1 >= t1).sum()) >= cap
        assert t1 <= int(np.sort(s1)[::-1][cap - 1])
    widx, wsc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, k, cap, certificate=True)
    assert list(info.cpu().numpy()) == [n, capped, cert]
    assert (idx.cpu().numpy() == widx).all()
    assert (sc.cpu().numpy() == wsc).all()


@pytest.mark.parametrize("case", ["vocab_over_2p17", "score_span_over_2p47"])
def test_finish_ranked_list_edges(case):
    """Capped inputs whose gathered list the finishing pass ranks directly
    (at most 512 rows): a vocabulary above 2^17 rows, and row scales near
    2^31 so S1' spans about 2^53."""
    if case == "vocab_over_2p17":       # 118 candidates, cap 100
        (trits, rs, h), k, cap = synth.lmhead(140000, 128, 81), 40, 100
    else:                               # row scales near 2^31: S1' spans ~2^53
        trits, _, h = synth.lmhead(3000, 256, 82)
        rs = np.random.default_rng(83).integers(1 << 28, (1 << 31) - 1, 3000).astype(np.int32)
        k, cap = 20, 50
    _, _, n, capped = check(trits, rs, h, k, cap)
    assert capped == 1 and n <= 512, n
