"""GPU parity of the steps on either side of the GEMV against the oracle
(oracle/edges.py): absmax int8 quantisation, LNS8 encoding, the candidate
sampler; each also chained into the kernel it feeds or follows."""
import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from oracle import edges as oe
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu


def _quant(x):
    import torch
    dev = device()
    note("act_quant_i8 k=%d" % x.size)
    q, a, st = bs.act_quant_i8(to_dev(x, dev))
    torch.cuda.synchronize()
    return q.cpu().numpy(), int(a.item()), int(st.item())


@pytest.mark.parametrize("k,mag,seed", [(2560, 1 << 20, 0), (6912, 1 << 40, 1), (1, 5, 2),
                                        (4097, 1 << 55, 3), (65537, 1000, 4), (13824, 3, 5)])
def test_quant_matches_oracle(k, mag, seed):
    x = np.random.default_rng(seed).integers(-mag, mag + 1, k).astype(np.int64)
    q, a, st = _quant(x)
    wq, wa = oe.act_quant_i8(x)
    assert st == bs.BS_OK and a == wa
    assert (q == wq).all()


def test_quant_hand_cases_zero_and_overflow():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "act_quant_hand.json")))
    for case in g["cases"]:
        q, a, st = _quant(np.array(case["x_fixed"], np.int64))
        assert st == 0 and a == case["absmax"] and q.tolist() == case["q"]
    q, a, st = _quant(np.zeros(3000, np.int64))
    assert st == 0 and a == 0 and not q.any()
    x = np.zeros(5000, np.int64)
    x[4321] = (1 << 55) + 1
    q, a, st = _quant(x)
    assert st == bs.BS_E_OVERFLOW and a == -1 and not q.any()
    x[4321] = np.iinfo(np.int64).min
    q, a, st = _quant(x)
    assert st == bs.BS_E_OVERFLOW and a == -1
    x[4321] = -(1 << 55)
    q, a, st = _quant(x)
    assert st == 0 and a == 1 << 55 and q[4321] == -127


def test_quant_feeds_the_ternary_gemv():
    import torch
    dev = device()
    rows, k = 2560, 2560
    t, sc, _ = synth.ternary(rows, k, 11)
    x = np.random.default_rng(12).integers(-(1 << 30), 1 << 30, k).astype(np.int64)
    note("act_quant_i8 -> ternary_gemv %dx%d" % (rows, k))
    q, _, _ = bs.act_quant_i8(to_dev(x, dev))
    y = bs.ternary_gemv(to_dev(bs.ternary_pack(t), dev), to_dev(bs.ternary_pack_scales(sc), dev),
                        q, rows, k)
    torch.cuda.synchronize()
    wq, _ = oe.act_quant_i8(x)
    assert (y.cpu().numpy() == oracle.ternary_gemv_def(t, sc, wq)).all()


def _encode(x, frac):
    import torch
    dev = device()
    note("lns8_encode k=%d frac=%d" % (x.size, frac))
    out = bs.lns8_encode(to_dev(x, dev), frac)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("frac,seed", [(0, 0), (8, 1), (16, 2), (30, 3), (62, 4)])
def test_encode_matches_oracle(frac, seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.integers(-(1 << 62), 1 << 62, 700),
                        (rng.standard_normal(700) * 2.0 ** (frac - 2)).astype(np.int64),
                        rng.integers(-3, 4, 100),
                        np.array([0, 1, -1, np.iinfo(np.int64).max, np.iinfo(np.int64).min])]
                       ).astype(np.int64)
    assert (_encode(x, frac) == oe.lns8_encode(x, frac)).all()


@pytest.mark.parametrize("frac", [0, 5, 24, 50])
def test_encode_at_every_code_edge(frac):
    """Magnitudes at, just below and just above each code edge (the edges
    pick the inputs; the oracle decides the codes)."""
    e = bs.lns8_encode_edges(frac)
    xs = []
    for c in range(1, 128):
        t = int(e[c])
        if t > 1 << 62:
            continue
        for v in (t - 1, t, t + 1):
            if 0 < v < 1 << 63:
                xs += [v, -v]
    x = np.array(xs, np.int64)
    assert (_encode(x, frac) == oe.lns8_encode(x, frac)).all()


def test_encode_feeds_the_lns8_gemv():
    import torch
    dev = device()
    rows, k, frac = 256, 1024, 20
    t, _ = synth.lns8(rows, k, 5)
    x = (np.random.default_rng(6).standard_normal(k) * 2.0 ** (frac + 1)).astype(np.int64)
    x[::17] = 0
    note("lns8_encode -> lns8_phase_gemv %dx%d" % (rows, k))
    enc = bs.lns8_encode(to_dev(x, dev), frac)
    acc, _ = bs.lns8_phase_gemv(to_dev(bs.ternary_pack(t), dev), enc, rows, k, bs.LNS8_POPCOUNT)
    torch.cuda.synchronize()
    assert (acc.cpu().numpy() == oracle.lns8_direct(t, oe.lns8_encode(x, frac))).all()


def _sample(idx, score, **kw):
    import torch
    dev = device()
    note("sample_candidates n=%d %s" % (len(idx), kw))
    r = bs.sample_candidates(to_dev(np.asarray(idx, np.int32), dev),
                             to_dev(np.asarray(score, np.int64), dev), **kw)
    torch.cuda.synchronize()
    return r.cpu().numpy().tolist()


def _want(idx, score, mode, **kw):
    o = oe.sample_candidates(idx, score, mode, **kw)
    return [o["token"], o["rank"], o["kept"], o["total"], o["draw"], o["attempts"]]


@pytest.mark.parametrize("n,seed", [(1, 0), (40, 1), (200, 2), (1024, 3), (77, 4), (64, 5),
                                    (65, 6), (960, 7), (961, 8)])
def test_sampler_matches_oracle(n, seed):
    """64/65: the last one-wavefront ranking and the first through LDS;
    960/961: the last workgroup with a wavefront of its own for the hashing
    and the first that hashes in the candidates' first wavefront."""
    rng = np.random.default_rng(seed)
    idx = rng.permutation(200000)[:n].astype(np.int32)
    score = rng.integers(-40, 40, n).astype(np.int64) * (1 << 10)
    if n > 4:
        idx[3] = idx[2]            # a repeated index: ties fall back to input order
        score[3] = score[2]
    for mode in (oe.SAMPLE_GREEDY, oe.SAMPLE_DRAW):
        for kw in (dict(beta=1 << 6), dict(beta=0), dict(beta=1 << 16, top_p=30000),
                   dict(beta=3000, min_p=2000), dict(beta=123, top_p=65535, min_p=65536),
                   dict(beta=(1 << 32) - 1)):
            for pos in (0, 1, 2 ** 64 - 1):
                args = dict(seed=seed * 1000 + 7, position=pos, **kw)
                want = _want(idx, score, mode, **args)
                got = _sample(idx, score, mode=mode, beta_q16=args["beta"],
                              top_p_q16=args.get("top_p", 1 << 16),
                              min_p_q16=args.get("min_p", 0), seed=args["seed"], position=pos)
                assert got == want, (mode, args)


def test_sampler_extreme_scores():
    idx = np.array([5, 9, 2, 7], np.int32)
    score = np.array([np.iinfo(np.int64).max, np.iinfo(np.int64).min, 0,
                      np.iinfo(np.int64).max - 1], np.int64)
    for beta in (0, 1, 1 << 16, (1 << 32) - 1):
        for pos in range(4):
            want = _want(idx, score, oe.SAMPLE_DRAW, beta=beta, seed=3, position=pos)
            got = _sample(idx, score, mode=bs.SAMPLE_DRAW, beta_q16=beta, seed=3, position=pos)
            assert got == want


def test_sampler_after_lmhead():
    """Top-k of the BITNET_PLANES lm_head, then a draw, all on the device."""
    import torch
    dev = device()
    trits, rs, h = synth.lmhead(3000, 256, 2)
    p03, p47 = bs.planes_pack(trits)
    note("lmhead 3000x256 -> sample_candidates")
    ti, ts, _ = bs.lmhead_planes_topk(to_dev(p03, dev), to_dev(p47, dev), to_dev(rs, dev),
                                      to_dev(h, dev), 3000, 256, 40, 200)
    outs = [bs.sample_candidates(ti, ts, bs.SAMPLE_DRAW, beta_q16=1 << 4, seed=9, position=p)
            for p in range(8)]
    torch.cuda.synchronize()
    widx, wsc, _, _ = oracle.lmhead_two_stage(trits, rs, h, 40, 200)
    for p, o in enumerate(outs):
        assert o.cpu().numpy().tolist() == _want(widx, wsc, oe.SAMPLE_DRAW, beta=1 << 4, seed=9,
                                                 position=p)


def test_sampler_rejected_first_draw():
    """Keys whose first draw is rejected (tests/golden/sampler_rejection.json):
    the kernel hashes the attempts in parallel lanes and must report the
    second attempt's value and two attempts used, as the oracle does."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "sampler_rejection.json")
    with open(path) as f:
        g = json.load(f)
    idx = np.arange(g["first_index"], g["first_index"] + g["n"], dtype=np.int32)
    score = np.full(g["n"], g["score"], np.int64)
    for c in g["cases"]:
        want = _want(idx, score, oe.SAMPLE_DRAW, beta=0, seed=c["seed"], position=c["position"])
        got = _sample(idx, score, mode=bs.SAMPLE_DRAW, beta_q16=0, seed=c["seed"],
                      position=c["position"])
        assert got == want
        assert got[5] == c["attempts"] == 2 and got[4] == c["draw"]
