"""Host-side checks of the pure fractional-LNS entry points (no GPU):

* the table blob the library builds on the host (extended precision) holds
  exactly the oracle's binary128 tables, for every supported f;
* blob header and size, and the errors of bs_flns_table_build;
* argument validation of bs_flns_phase_gemv returns the documented BS_E_*
  code before any HIP call (only failing calls are made here);
* the workspace size is the interface's reserved 256 bytes for every
  valid shape (the reduction keeps every partial result on chip).
"""
import ctypes

import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle

FAKE = ctypes.c_void_p(1 << 20)          # never dereferenced: validation fails first


def _unpack(blob):
    """(header, fold table, kp, km, padding past each table)."""
    hdr = blob[:64].view(np.int32)
    nkp, nkm, elem, S = int(hdr[2]), int(hdr[3]), int(hdr[4]), int(hdr[6])
    assert S == max(nkp, nkm) + 1
    fold = blob[64:64 + 132 * 4].view(np.int32)
    corr = blob[592:592 + 2 * S * elem].view(np.int16 if elem == 2 else np.int32)
    pad = np.concatenate([corr[nkp:S], corr[S + nkm:2 * S]])
    return hdr, fold, corr[:nkp], corr[S:S + nkm], pad


@pytest.mark.parametrize("f", range(0, 13))
def test_table_blob_equals_oracle_tables(f):
    blob = bs.flns_table(f)
    hdr, fold, kp, km, pad = _unpack(blob)
    tb = oracle.flns_tables(f)
    assert hdr[0] == 0x534E4C46 and hdr[1] == f and hdr[5] == blob.size
    assert hdr[4] == (2 if f <= 8 else 4)
    assert blob.size % 16 == 0
    assert np.array_equal(fold[:129], tb["lc"])
    assert np.array_equal(kp, tb["kp"])
    assert km.size == tb["km"].size
    assert np.array_equal(km[1:], tb["km"][1:])
    assert (pad == 0).all() and pad.size >= 2      # a clamped index reads a zero correction


def test_table_bytes_and_build_errors():
    lib = bs.lib()
    assert lib.bs_flns_table_bytes(-1) == 0
    assert lib.bs_flns_table_bytes(13) == 0
    sizes = [lib.bs_flns_table_bytes(f) for f in range(13)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))     # the size identifies f
    buf = np.zeros(sizes[4], dtype=np.uint8)
    p = ctypes.c_void_p(buf.ctypes.data)
    assert lib.bs_flns_table_build(4, None, sizes[4]) == bs.BS_E_NULL
    assert lib.bs_flns_table_build(13, p, sizes[4]) == bs.BS_E_RANGE
    assert lib.bs_flns_table_build(4, p, sizes[4] - 16) == bs.BS_E_SHAPE
    assert lib.bs_flns_table_build(4, p, sizes[4]) == bs.BS_OK


def _flns(planes=FAKE, x=FAKE, rows=64, k=1024, f=8, d=1, table=FAKE, tbytes=None, out=FAKE,
          ws=FAKE, wsn=1 << 20):
    lib = bs.lib()
    if tbytes is None:
        tbytes = lib.bs_flns_table_bytes(f) if 0 <= f <= 12 else 4096
    return lib.bs_flns_phase_gemv(planes, x, rows, k, f, d, table, tbytes, out, ws, wsn, None)


def test_flns_validation():
    off = lambda n: ctypes.c_void_p((1 << 20) + n)
    lib = bs.lib()
    assert _flns(planes=None) == bs.BS_E_NULL
    assert _flns(x=None) == bs.BS_E_NULL
    assert _flns(table=None) == bs.BS_E_NULL
    assert _flns(out=None) == bs.BS_E_NULL
    assert _flns(rows=0) == bs.BS_E_SHAPE
    assert _flns(rows=1 << 28) == bs.BS_E_SHAPE               # launch grid limit (2^32 threads)
    assert _flns(k=100) == bs.BS_E_SHAPE
    assert _flns(k=65536) == bs.BS_E_OVERFLOW
    assert _flns(f=-1) == bs.BS_E_RANGE
    assert _flns(f=13) == bs.BS_E_RANGE
    assert _flns(d=0) == bs.BS_E_RANGE
    # a table of another precision is rejected by its size
    assert _flns(f=8, tbytes=lib.bs_flns_table_bytes(7)) == bs.BS_E_RANGE
    assert _flns(planes=off(8)) == bs.BS_E_ALIGN
    assert _flns(x=off(2)) == bs.BS_E_ALIGN
    assert _flns(table=off(8)) == bs.BS_E_ALIGN
    assert _flns(out=off(4)) == bs.BS_E_ALIGN
    assert _flns(ws=None) == bs.BS_E_WORKSPACE
    assert _flns(ws=off(16)) == bs.BS_E_WORKSPACE
    assert _flns(k=2048, wsn=16) == bs.BS_E_WORKSPACE


def test_flns_workspace_sizes():
    lib = bs.lib()
    assert lib.bs_flns_workspace_bytes(0, 128) == 0               # invalid shapes
    assert lib.bs_flns_workspace_bytes(64, 100) == 0
    assert lib.bs_flns_workspace_bytes(64, 65536) == 0
    for rows, k in ((1, 128), (64, 1024), (4096, 4096), (65, 1152), (64, 65408),
                    ((1 << 31) - 64, 4096)):
        assert lib.bs_flns_workspace_bytes(rows, k) == 256
