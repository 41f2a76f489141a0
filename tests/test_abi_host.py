"""Host-side checks of the C-ABI library that need no GPU.

* the shared library loads and exports every function include/bs.h declares;
* the load-time codec (host C++) is byte-identical to the oracle's own
  implementation of the documented layouts, and rejects invalid input;
* argument validation returns the documented BS_E_* code before any HIP call
  (only calls that fail validation are made here, so nothing reaches the
  GPU runtime).
"""
import ctypes

import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth

FAKE = ctypes.c_void_p(1 << 20)          # never dereferenced: validation fails first


def test_library_exports_every_header_symbol():
    lib = bs.lib()
    names = bs.header_symbols()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    assert lib.bs_abi_version() == 2


def test_probe_library_exports_its_header():
    """The benchmark's measurement kernels (include/bs_probe.h) are exported
    by libbsprobe.so; host validation runs without a GPU."""
    import re
    from bit_decode_gemv_amd import probe
    lib = probe.lib()
    names = sorted(set(re.findall(r"\b(bs_probe_[a-z0-9_]+)\s*\(", open(probe.HEADER).read())))
    assert names == ["bs_probe_empty", "bs_probe_read", "bs_probe_read_sink_count",
                     "bs_probe_read_strided"]
    for name in names:
        assert hasattr(lib, name), name
    assert lib.bs_probe_read_sink_count(4096 * 8, 8) == 256
    assert lib.bs_probe_read_sink_count(4096 * 8 + 1, 8) == 512
    assert lib.bs_probe_read_sink_count(0, 8) == -3
    assert lib.bs_probe_read_sink_count((1 << 31) - 15, 8) == -3
    assert lib.bs_probe_read_sink_count(4096, 3) == -3
    assert lib.bs_probe_read(None, 4096, 8, FAKE, None) == -1
    assert lib.bs_probe_read_strided(None, 4096, 512, FAKE, None) == -1
    assert lib.bs_probe_read_strided(FAKE, 0, 512, FAKE, None) == -3
    assert lib.bs_probe_read_strided(FAKE, 1 << 31, 512, FAKE, None) == -3
    assert lib.bs_probe_read_strided(FAKE, 4096, 0, FAKE, None) == -3
    assert lib.bs_probe_read_strided(FAKE, 4096, 65537, FAKE, None) == -3
    assert lib.bs_probe_read_strided(ctypes.c_void_p((1 << 20) + 8), 4096, 512, FAKE, None) == -3
    assert lib.bs_probe_empty(0, 64, None) == -3
    assert lib.bs_probe_empty(1, 100, None) == -3


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert bs.status_str(code)
    assert bs.status_str(-99) == "unknown status"


@pytest.mark.parametrize("rows,k,seed", [(256, 512, 0), (1, 128, 1), (63, 256, 2), (65, 384, 3),
                                         (130, 1280, 4)])
def test_ternary_codec_matches_oracle_layout(rows, k, seed):
    t, sc, _ = synth.ternary(rows, k, seed, p_zero=1 / 3)
    p = bs.ternary_pack(t)
    assert p.size == oracle.pad64(rows) * k // 4
    assert (p == oracle.ternary_pack(t)).all()
    assert (bs.ternary_unpack(p, rows, k) == t).all()
    ps = bs.ternary_pack_scales(sc)
    assert (ps == oracle.scales_pack(sc)).all()


def test_ternary_codec_rejects_invalid():
    t = np.zeros((4, 128), np.int8)
    t[2, 5] = -2
    with pytest.raises(bs.BsError) as e:
        bs.ternary_pack(t)
    assert e.value.status == bs.BS_E_RANGE
    z = bs.ternary_pack(np.zeros((3, 128), np.int8))
    z[1024 + 16 * 2 + 3] = 0x10          # W_negative without W_nonzero
    with pytest.raises(bs.BsError) as e:
        bs.ternary_unpack(z, 3, 128)
    assert e.value.status == bs.BS_E_RANGE
    with pytest.raises(bs.BsError) as e:
        bs.ternary_pack(np.zeros((3, 100), np.int8))
    assert e.value.status == bs.BS_E_SHAPE


@pytest.mark.parametrize("V,K,seed", [(65, 256, 0), (128, 128, 1), (3, 384, 2)])
def test_planes_codec_matches_oracle_layout(V, K, seed):
    trits, _, _ = synth.lmhead(V, K, seed)
    p03, p47 = bs.planes_pack(trits)
    o03, o47 = oracle.planes_pack(trits)
    assert (p03 == o03).all() and (p47 == o47).all()


def test_sizes():
    lib = bs.lib()
    assert lib.bs_ternary_planes_bytes(2560, 2560) == 2560 * 2560 // 4
    assert lib.bs_ternary_planes_bytes(65, 128) == 128 * 128 // 4
    assert lib.bs_ternary_scales_count(2560, 2560) == 2560 * 20
    assert lib.bs_ternary_planes_bytes(10, 100) == bs.BS_E_SHAPE
    assert lib.bs_planes03_bytes(128256, 2560) == 128256 * 2560
    assert lib.bs_planes47_bytes(100, 256) == 100 * 256
    assert lib.bs_lns8_workspace_bytes(4096, 4096) > 0
    assert lib.bs_lmhead_workspace_bytes(128256, 2560, 40, 200) > 0
    assert lib.bs_lmhead_workspace_bytes(128256, 2560, 201, 200) == 0


def _tgemv(planes=FAKE, scales=FAKE, x=FAKE, rows=64, k=128, frac=0, y=FAKE):
    return bs.lib().bs_ternary_gemv(planes, scales, x, rows, k, frac, y, None)


def test_ternary_gemv_validation():
    assert _tgemv(planes=None) == bs.BS_E_NULL
    assert _tgemv(y=None) == bs.BS_E_NULL
    assert _tgemv(k=100) == bs.BS_E_SHAPE
    assert _tgemv(k=0) == bs.BS_E_SHAPE
    assert _tgemv(rows=0) == bs.BS_E_SHAPE
    assert _tgemv(frac=-1) == bs.BS_E_RANGE
    assert _tgemv(frac=63) == bs.BS_E_RANGE
    assert _tgemv(k=(1 << 24) + 128) == bs.BS_E_OVERFLOW
    assert _tgemv(planes=ctypes.c_void_p((1 << 20) + 8)) == bs.BS_E_ALIGN
    assert _tgemv(x=ctypes.c_void_p((1 << 20) + 4)) == bs.BS_E_ALIGN
    assert _tgemv(y=ctypes.c_void_p((1 << 20) + 4)) == bs.BS_E_ALIGN


def _lns8(planes=FAKE, x=FAKE, rows=64, k=128, path=0, acc=FAKE, s=FAKE, ws=FAKE, wsn=1 << 20):
    return bs.lib().bs_lns8_phase_gemv(planes, x, rows, k, path, acc, s, ws, wsn, None)


def test_lns8_validation():
    assert _lns8(x=None) == bs.BS_E_NULL
    assert _lns8(acc=None) == bs.BS_E_NULL
    assert _lns8(k=64) == bs.BS_E_SHAPE
    assert _lns8(path=3) == bs.BS_E_RANGE
    assert _lns8(k=65536) == bs.BS_E_OVERFLOW       # |A| <= k*2^15 would not fit int32
    assert _lns8(ws=None) == bs.BS_E_WORKSPACE
    assert _lns8(wsn=8) == bs.BS_E_WORKSPACE


def _lmh(V=1000, dim=256, top_k=40, cap=200, ws=FAKE, wsn=1 << 26, **kw):
    a = dict(p03=FAKE, p47=FAKE, rs=FAKE, h=FAKE, idx=FAKE, score=FAKE, info=FAKE)
    a.update(kw)
    return bs.lib().bs_lmhead_planes_topk(a["p03"], a["p47"], a["rs"], a["h"], V, dim, top_k,
                                          cap, a["idx"], a["score"], a["info"], ws, wsn, None)


def test_lmhead_validation():
    assert _lmh(p47=None) == bs.BS_E_NULL
    assert _lmh(info=None) == bs.BS_E_NULL
    assert _lmh(dim=200) == bs.BS_E_SHAPE
    assert _lmh(top_k=0) == bs.BS_E_RANGE
    assert _lmh(top_k=201, cap=200) == bs.BS_E_RANGE
    assert _lmh(V=10, top_k=20, cap=20) == bs.BS_E_RANGE
    assert _lmh(cap=5000) == bs.BS_E_RANGE
    assert _lmh(dim=10240) == bs.BS_E_OVERFLOW      # int64 bound of the exact score
    assert _lmh(ws=None) == bs.BS_E_WORKSPACE
    assert _lmh(wsn=1024) == bs.BS_E_WORKSPACE


def test_alignment_validation():
    """Every device pointer's documented alignment is checked on the host."""
    off = lambda n: ctypes.c_void_p((1 << 20) + n)
    assert _lns8(planes=off(8)) == bs.BS_E_ALIGN
    assert _lns8(x=off(2)) == bs.BS_E_ALIGN
    assert _lns8(acc=off(2)) == bs.BS_E_ALIGN
    assert _lns8(s=off(4)) == bs.BS_E_ALIGN
    assert _lmh(p03=off(8)) == bs.BS_E_ALIGN
    assert _lmh(p47=off(4)) == bs.BS_E_ALIGN
    assert _lmh(rs=off(2)) == bs.BS_E_ALIGN
    assert _lmh(h=off(4)) == bs.BS_E_ALIGN
    assert _lmh(idx=off(2)) == bs.BS_E_ALIGN
    assert _lmh(score=off(4)) == bs.BS_E_ALIGN
    assert _lmh(info=off(2)) == bs.BS_E_ALIGN
    assert _lmh(ws=off(128)) == bs.BS_E_WORKSPACE    # the workspace is 256-byte aligned


def test_lmhead_vocab_limit():
    assert _lmh(V=(1 << 31) - 1023) == bs.BS_E_SHAPE
    assert bs.lib().bs_lmhead_workspace_bytes((1 << 31) - 1023, 256, 40, 200) == 0


def test_workspace_sizes_follow_the_launch_plans():
    lib = bs.lib()
    # LNS8: when K is split over workgroups, one int32 counter per 64-row tile
    # (256-byte aligned) and the partials int32[nsplit][R][8]
    assert lib.bs_lns8_workspace_bytes(2000, 128) == 256
    assert lib.bs_lns8_workspace_bytes(4096, 4096) == 256 + 4 * 4096 * 8 * 4
    assert lib.bs_lns8_workspace_bytes(64, 65408) == 256 + 64 * 64 * 8 * 4
    # lm_head: grows with the vocabulary, not with top_k beyond the bounds
    a = lib.bs_lmhead_workspace_bytes(128256, 2560, 40, 200)
    assert a == lib.bs_lmhead_workspace_bytes(128256, 2560, 200, 200) > 128256 * 40


@pytest.mark.parametrize("rows,k,seed", [(1, 128, 0), (64, 256, 1), (65, 384, 2), (130, 2560, 3)])
def test_q1_codec_matches_oracle_layout(rows, k, seed):
    s, _, _ = synth.q1(rows, k, seed)
    assert (bs.q1_pack(s) == oracle.q1_pack(s)).all()
    assert bs.lib().bs_q1_planes_bytes(rows, k) == -(-rows // 64) * 64 * k // 8
    bad = s.copy()
    bad[0, 5] = 0
    with pytest.raises(bs.BsError) as e:
        bs.q1_pack(bad)
    assert e.value.status == bs.BS_E_RANGE


def _q1(bits=FAKE, scales=FAKE, x=FAKE, rows=64, k=256, frac=0, y=FAKE):
    return bs.lib().bs_q1_gemv(bits, scales, x, rows, k, frac, y, None)


def test_q1_gemv_validation():
    assert _q1(bits=None) == bs.BS_E_NULL
    assert _q1(k=100) == bs.BS_E_SHAPE
    assert _q1(frac=63) == bs.BS_E_RANGE
    assert _q1(k=(1 << 24) + 128) == bs.BS_E_OVERFLOW
    assert _q1(bits=ctypes.c_void_p((1 << 20) + 8)) == bs.BS_E_ALIGN
    assert _q1(x=ctypes.c_void_p((1 << 20) + 4)) == bs.BS_E_ALIGN


# ---- steps around the GEMVs (host checks)

@pytest.mark.parametrize("frac", [0, 1, 9, 16, 30, 47, 62])
def test_lns8_encode_edges_match_oracle(frac):
    """Each library code edge is the least magnitude whose oracle code reaches
    that code: code(edge) >= c and code(edge - 1) < c."""
    from oracle import edges as oe
    e = bs.lns8_encode_edges(frac)
    assert e[0] == 0
    assert (np.diff(e[1:].astype(object)) >= 0).all()
    for c in range(1, 128):
        t = int(e[c])
        if t == (1 << 64) - 1:
            assert oe.lns8_code(1 << 63, frac) < c
            continue
        assert t <= 1 << 63
        assert oe.lns8_code(t, frac) >= c
        assert t == 1 or oe.lns8_code(t - 1, frac) < c


def test_edges_steps_validation():
    lib = bs.lib()
    assert lib.bs_act_quant_i8(None, 8, FAKE, FAKE, FAKE, None) == bs.BS_E_NULL
    assert lib.bs_act_quant_i8(FAKE, 0, FAKE, FAKE, FAKE, None) == bs.BS_E_SHAPE
    assert lib.bs_act_quant_i8(ctypes.c_void_p((1 << 20) + 4), 8, FAKE, FAKE, FAKE,
                               None) == bs.BS_E_ALIGN
    assert lib.bs_act_quant_i8(FAKE, 8, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 2),
                               None) == bs.BS_E_ALIGN
    assert lib.bs_lns8_encode(FAKE, 8, 63, FAKE, None) == bs.BS_E_RANGE
    assert lib.bs_lns8_encode(FAKE, 8, -1, FAKE, None) == bs.BS_E_RANGE
    assert lib.bs_lns8_encode(None, 8, 0, FAKE, None) == bs.BS_E_NULL
    assert lib.bs_lns8_encode(FAKE, 0, 0, FAKE, None) == bs.BS_E_SHAPE
    assert lib.bs_lns8_encode_edges(63, None) == bs.BS_E_NULL
    assert lib.bs_lns8_encode_edges(63, FAKE) == bs.BS_E_RANGE

    def smp(n=40, mode=1, top_p=65536, min_p=0, idx=FAKE, score=FAKE, res=FAKE):
        return lib.bs_sample_candidates(idx, score, n, mode, 1 << 16, top_p, min_p, 1, 2, res,
                                        None)
    assert smp(idx=None) == bs.BS_E_NULL
    assert smp(res=None) == bs.BS_E_NULL
    assert smp(n=0) == bs.BS_E_SHAPE
    assert smp(n=1025) == bs.BS_E_SHAPE
    assert smp(mode=2) == bs.BS_E_RANGE
    assert smp(top_p=0) == bs.BS_E_RANGE
    assert smp(top_p=65537) == bs.BS_E_RANGE
    assert smp(min_p=65537) == bs.BS_E_RANGE
    assert smp(score=ctypes.c_void_p((1 << 20) + 4)) == bs.BS_E_ALIGN
    assert smp(idx=ctypes.c_void_p((1 << 20) + 2)) == bs.BS_E_ALIGN


def test_row_counts_past_int32_indexing_are_rejected():
    """The kernels index rows (with the last tile's padding) in int32: row
    counts above 2^31 - 64 fail on the host with BS_E_SHAPE, before any HIP
    call (fake pointers are never dereferenced)."""
    lib = bs.lib()
    big = (1 << 31) - 63
    for rows in (big, 1 << 31, 1 << 40):
        assert lib.bs_ternary_gemv(FAKE, FAKE, FAKE, rows, 128, 0, FAKE, None) == bs.BS_E_SHAPE
        assert lib.bs_ternary_gemv_acc(FAKE, FAKE, FAKE, rows, 128, 0, FAKE, None) == \
            bs.BS_E_SHAPE
        assert lib.bs_q1_gemv(FAKE, FAKE, FAKE, rows, 128, 0, FAKE, None) == bs.BS_E_SHAPE
        assert lib.bs_lns8_phase_gemv(FAKE, FAKE, rows, 128, 0, FAKE, FAKE, FAKE, 1 << 20,
                                      None) == bs.BS_E_SHAPE
        assert lib.bs_lns8_workspace_bytes(rows, 128) == 0
