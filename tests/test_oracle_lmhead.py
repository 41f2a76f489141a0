"""Pins of the BITNET_PLANES lm_head oracle ("[bitnet] T2: lm_head via
BITNET_PLANES weight format (WeightForm) + two-stage top-k decode").

What pins it: a NumPy brute force of the exact eight-plane score; the
bound invariant |S' - S1'| <= B' on every row and the page's truncation
figure; exactness of the two-stage result whenever the cap does not engage
(the page says the bound-driven rescoring equals the exact top-k);
special cases: an exactly-ternary source (planes 1..7 zero, which plane 0
captures losslessly), a single plane (which reduces to the ternary GEMV with
scale 3^(7-p)*rowScale), all-zero planes (ties resolved by lowest index).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_decode_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
POW3 = np.array([3 ** (7 - p) for p in range(8)], np.int64)


def numpy_scores(trits, rs, h):
    dots = np.einsum("vpk,k->vp", trits.astype(np.int64), h.astype(np.int64))
    return rs.astype(np.int64) * (dots @ POW3)


def numpy_topk(scores, k):
    order = np.lexsort((np.arange(scores.size), -scores))
    return order[:k].astype(np.int32), scores[order[:k]]


def small_case(V, K, seed):
    trits, rs, h = synth.lmhead(V, K, seed)
    return trits, rs, h


@pytest.mark.parametrize("V,K,k,seed", [(300, 128, 40, 0), (257, 256, 7, 1), (64, 128, 1, 2),
                                         (100, 128, 100, 3)])
def test_brute_matches_numpy(V, K, k, seed):
    trits, rs, h = small_case(V, K, seed)
    idx, sc, allsc = oracle.lmhead_brute(trits, rs, h, k, all_scores=True)
    want = numpy_scores(trits, rs, h)
    assert (allsc == want).all()
    wi, ws = numpy_topk(want, k)
    assert (idx == wi).all() and (sc == ws).all()


@pytest.mark.parametrize("V,K,seed", [(300, 128, 0), (290, 256, 5)])
def test_bound_invariant_and_candidate_superset(V, K, seed):
    trits, rs, h = small_case(V, K, seed)
    s1, b = oracle.lmhead_stage1(trits, rs, h)
    exact = numpy_scores(trits, rs, h)
    assert (np.abs(exact - s1) <= b).all()
    habs = int(np.abs(h.astype(np.int64)).sum())
    assert (b == 40 * np.abs(rs.astype(np.int64)) * habs).all()
    for k in (1, 10, 40):
        lower = np.sort(s1 - b)[::-1]
        lk = lower[k - 1]
        cand = np.nonzero(s1 + b >= lk)[0]
        ti, _ = numpy_topk(exact, k)
        assert len(cand) >= k
        assert set(ti.tolist()) <= set(cand.tolist())
        idx, sc, n, capped = oracle.lmhead_two_stage(trits, rs, h, k, cap=V)
        assert n == len(cand) and capped == 0
        assert (idx == ti).all() and (sc == exact[ti]).all()


def test_page_truncation_figure():
    vals = {}
    for line in open(os.path.join(GOLDEN, "planes_bound.txt")):
        line = line.split("#")[0].strip()
        if line:
            key, v = line.split()
            vals[key] = float(v)
    tail = Fraction(int(vals["tail_numerator"]), int(vals["tail_denominator"]))
    finite = Fraction(int(vals["finite_numerator"]), int(vals["finite_denominator"]))
    assert sum(Fraction(1, 3 ** p) for p in range(4, 8)) == finite
    assert abs(float(tail) * 100 - vals["page_truncation_percent"]) < 0.005
    assert finite < tail
    # the oracle's bound, in units of 3^-7 * |rowScale| * sum|h|, is exactly 40/2187
    trits, rs, h = small_case(80, 128, 9)
    _, b = oracle.lmhead_stage1(trits, rs, h)
    habs = int(np.abs(h.astype(np.int64)).sum())
    for r in range(80):
        assert Fraction(int(b[r]), 3 ** 7 * int(rs[r]) * habs) == finite


def test_planted_peaks_exact_branch():
    trits, rs, h, peaks = synth.lmhead_planted(600, 256, 4, n_peaks=16)
    idx, sc, n, capped = oracle.lmhead_two_stage(trits, rs, h, 10, cap=200)
    bi, bs = oracle.lmhead_brute(trits, rs, h, 10)
    assert capped == 0 and n <= 200
    assert (idx == bi).all() and (sc == bs).all()
    assert set(idx.tolist()) <= set(peaks.tolist())


def test_exactly_ternary_source():
    """Planes 1..7 zero: plane 0 carries the codes, stage 1 is already exact."""
    trits, rs, h = small_case(200, 128, 6)
    trits[:, 1:, :] = 0
    s1, _ = oracle.lmhead_stage1(trits, rs, h)
    assert (s1 == numpy_scores(trits, rs, h)).all()
    idx, sc, n, capped = oracle.lmhead_two_stage(trits, rs, h, 20, cap=200)
    bi, bs = oracle.lmhead_brute(trits, rs, h, 20)
    assert (idx == bi).all() and (sc == bs).all()


def test_single_plane_is_the_ternary_gemv():
    trits, rs, h = small_case(130, 256, 7)
    trits[:, 1:, :] = 0
    rs = (np.arange(130) % 14 + 1).astype(np.int32)   # 2187*rs fits int16
    _, _, allsc = oracle.lmhead_brute(trits, rs, h, 5, all_scores=True)
    scale = np.repeat((2187 * rs).astype(np.int16)[:, None], 2, axis=1)
    y = oracle.ternary_gemv_def(trits[:, 0, :], scale, h)
    assert (allsc == y).all()


def test_all_zero_planes_tie_break():
    trits = np.zeros((250, 8, 128), np.int8)
    _, rs, h = small_case(250, 128, 8)
    idx, sc, n, capped = oracle.lmhead_two_stage(trits, rs, h, 40, cap=200)
    assert (idx == np.arange(40)).all() and not sc.any()
    assert n == 250 and capped == 1
    bi, bs = oracle.lmhead_brute(trits, rs, h, 40)
    assert (bi == np.arange(40)).all()


def test_equal_rows_tie_break_lowest_index():
    trits, rs, h = small_case(50, 128, 10)
    trits[30] = trits[7]
    rs[30] = rs[7]
    trits[7, 0] = np.sign(h)          # make row 7 (and 30) the best
    trits[30, 0] = np.sign(h)
    idx, sc, _, _ = oracle.lmhead_two_stage(trits, rs, h, 3, cap=50)
    assert idx[0] == 7 and idx[1] == 30 and sc[0] == sc[1]


def test_cap_branch_keeps_top_stage1_rows():
    trits, rs, h = small_case(400, 128, 11)
    k, cap = 5, 8
    s1, b = oracle.lmhead_stage1(trits, rs, h)
    idx, sc, n, capped = oracle.lmhead_two_stage(trits, rs, h, k, cap)
    lk = np.sort(s1 - b)[::-1][k - 1]
    cand = np.nonzero(s1 + b >= lk)[0]
    assert n == len(cand) and n > cap and capped == 1
    order = np.lexsort((cand, -s1[cand]))
    kept = cand[order[:cap]]
    exact = numpy_scores(trits, rs, h)
    want = kept[np.lexsort((kept, -exact[kept]))][:k]
    assert (idx == want).all() and (sc == exact[want]).all()


def test_planes_pack_layout_positions():
    """Hand-placed trits land where the packed layout puts them, as the
    balanced-ternary digit sums 27*T_0 + 9*T_1 + 3*T_2 + T_3 (planes 0-3) and
    27*T_4 + 9*T_5 + 3*T_6 + T_7 (planes 4-7)."""
    V, K = 65, 256
    trits = np.zeros((V, 8, K), np.int8)
    trits[0, 0, 0] = 1                    # D03 = 27: tile 0, g 0, run 0, row 0, byte 0
    trits[1, 3, 9] = -1                   # D03 = -1: run 0, row 1 (16), byte 9
    trits[64, 2, 130] = 1                 # D03 = 3: tile 1, g 1 (block 3), run 0, row 0, byte 2
    trits[5, 0:4, 17] = [1, -1, 0, 1]     # D03 = 27 - 9 + 1 = 19: run 1 (1024), row 5 (80), byte 1
    trits[2, 4, 0] = 1                    # D47 = 27 at 2*256
    trits[3, 7, 255] = -1                 # D47 = -1 at 3*256 + 255
    trits[6, 4:8, 100] = -1               # D47 = -40 at 6*256 + 100
    p03, p47 = oracle.planes_pack(trits)
    assert p03.size == 128 * K and p47.size == V * K
    want03 = {0: 27, 16 + 9: 0xFF, 3 * 8192 + 2: 3, 1024 + 80 + 1: 19}
    want47 = {2 * 256: 27, 3 * 256 + 255: 0xFF, 6 * 256 + 100: 256 - 40}
    assert sorted(np.nonzero(p03)[0].tolist()) == sorted(want03)
    assert sorted(np.nonzero(p47)[0].tolist()) == sorted(want47)
    for off, v in want03.items():
        assert p03[off] == v
    for off, v in want47.items():
        assert p47[off] == v


def test_planes_digits_keep_every_trit():
    """The packed digit sums determine the eight trits: balanced-ternary
    decoding of D03 and D47 gives back planes 0-3 and 4-7."""
    V, K = 70, 256
    trits, _, _ = synth.lmhead(V, K, 21)
    p03, p47 = oracle.planes_pack(trits)
    blk = p03.view(np.int8).reshape(-1, K // 128, 8, 64, 16)      # tile, g, run, row, byte
    d03 = blk.transpose(0, 3, 1, 2, 4).reshape(-1, K)[:V].astype(np.int64)
    d47 = p47.view(np.int8).reshape(V, K).astype(np.int64)

    def digits(d):
        out = []
        for _ in range(4):
            t = (d + 1) % 3 - 1
            out.append(t)
            d = (d - t) // 3
        assert not d.any()
        return np.stack(out[::-1], axis=1)

    assert (digits(d03) == trits[:, 0:4, :]).all()
    assert (digits(d47) == trits[:, 4:8, :]).all()


def test_brute_row_parallel_matches_single_thread():
    trits, rs, h = synth.lmhead(700, 256, 9)
    wi, ws = oracle.lmhead_brute(trits, rs, h, 40)
    for n in (2, 5):
        oracle.set_threads(n)
        gi, gs = oracle.lmhead_brute_mt(trits, rs, h, 40)
        assert (gi == wi).all() and (gs == ws).all()
    oracle.set_threads(1)


def numpy_certificate(trits, rs, h, k, cap):
    """The exactness certificate from its definition, in NumPy: stage-1
    scores S1' = 81*rs*E1 and bounds B' = 40*|rs|*sum|h| per row, L_k the
    k-th largest S1' - B', C = {U >= L_k}; when |C| > cap the rows of C past
    the top `cap` by (S1' desc, row asc) are dropped, and the certificate
    holds iff max U over them < the k-th output score (which the brute
    force gives whenever the result is exact, and the two-stage oracle
    gives always)."""
    t = trits.astype(np.int64)
    hh = h.astype(np.int64)
    e1 = sum(3 ** (3 - p) * (t[:, p, :] @ hh) for p in range(4))
    s1 = 81 * rs.astype(np.int64) * e1
    b = 40 * np.abs(rs.astype(np.int64)) * int(np.abs(hh).sum())
    lk = np.sort(s1 - b)[::-1][k - 1]
    c = np.nonzero(s1 + b >= lk)[0]
    if c.size <= cap:
        return c.size, 0, None
    order = c[np.lexsort((c, -s1[c]))]
    return c.size, 1, (s1 + b)[order[cap:]].max()


@pytest.mark.parametrize("V,K,k,cap,seed", [(3000, 256, 10, 10, 92), (4000, 256, 20, 20, 91),
                                             (2000, 128, 5, 8, 11), (1500, 256, 3, 6, 12),
                                             (800, 128, 40, 200, 13), (2500, 256, 8, 12, 14)])
def test_certificate_matches_its_definition_and_is_sound(V, K, k, cap, seed):
    trits, rs, h = synth.lmhead(V, K, seed)
    idx, sc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, k, cap, certificate=True)
    nn, ncapped, umax = numpy_certificate(trits, rs, h, k, cap)
    assert (n, capped) == (nn, ncapped)
    assert cert == (1 if not capped else int(umax < sc[-1]))
    bi, bsc = oracle.lmhead_brute(trits, rs, h, k)
    if cert:   # soundness: a certified result is the exact top-k
        assert (idx == bi).all() and (sc == bsc).all()


def test_certificate_zero_where_the_cap_drops_a_top_row():
    """The (4000, 256, k = cap = 20) case has a true top-20 row outside the
    capped set: the result differs from brute force and is not certified."""
    trits, rs, h = synth.lmhead(4000, 256, 91)
    idx, sc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, 20, 20, certificate=True)
    bi, bsc = oracle.lmhead_brute(trits, rs, h, 20)
    assert capped == 1 and not ((idx == bi).all() and (sc == bsc).all())
    assert cert == 0


def test_certificate_capped_and_certified():
    """Planted peaks far above the rest, cap below the number of candidates:
    the cap engages and the dropped candidates' upper bounds stay below the
    k-th score, so the capped result is certified (and equals brute force)."""
    trits, rs, h, _ = synth.lmhead_planted(2000, 512, 1, n_peaks=64)
    idx, sc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, 3, 6, certificate=True)
    bi, bsc = oracle.lmhead_brute(trits, rs, h, 3)
    assert capped == 1 and n == 7 and cert == 1
    assert (idx == bi).all() and (sc == bsc).all()


def test_recorded_full_vocab_results_are_consistent():
    """tests/golden/lmhead_c5_record.json (written by make_lmhead_c5_record.py
    from the oracle alone): five seeds of the full-vocabulary workload, each
    with the two-stage result, its info, the brute-force top-k and the
    equality flag, which must agree with the recorded arrays; a certified
    result must equal the brute force."""
    import json
    rec = json.load(open(os.path.join(GOLDEN, "lmhead_c5_record.json")))
    assert sorted(rec["seeds"]) == ["0", "1", "2", "3", "4"]
    for seed, r in rec["seeds"].items():
        assert len(r["two_stage_idx"]) == len(r["brute_idx"]) == 40
        same = r["two_stage_idx"] == r["brute_idx"] and r["two_stage_score"] == r["brute_score"]
        assert r["equals_brute_force"] == same, seed
        assert r["capped"] == int(r["n_candidates"] > 200)
        if r["certified"]:
            assert same, seed
        # brute force: scores descending, ties by lower index
        s, i = r["brute_score"], r["brute_idx"]
        assert all((s[j], -i[j]) > (s[j + 1], -i[j + 1]) for j in range(39))
