"""Oracle for the ternary decode-GEMV hot path (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports it,
and this package imports nothing from the product.

The integer loops live in ``bs_oracle.c`` (plain C11, built with gcc into
``liboracle.so`` next to it).  The few steps that need exact real arithmetic
are written here in pure Python with integers and ``fractions``:

* ``f_hat`` -- F[p] = 2^((p-2)/8) of the BitState/HSDR brief v0.5, section 3,
  correctly rounded to binary64 by an integer eighth-root;
* ``lns8_decode`` -- |x| = 2^((code-74)/8) of the same section, correctly
  rounded by the same integer method, but from the code's own exponent;
* ``lns8_materialize`` -- S = 2^-9 * sum_p A[p]*F[p] of section 3.1, the
  exact rational sum over the binary64 F values, rounded once.

The pure fractional-LNS reduction of section 5.2 lives in ``flns_oracle.c``;
its tables are evaluated in binary128 (libquadmath) and rounded to nearest.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bs_oracle.c")
_SRC_FLNS = os.path.join(_HERE, "flns_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no intrinsics) into liboracle.so.
    flns_oracle.c uses GCC's binary128 (libquadmath), hence gnu11; -fopenmp
    only for the row-parallel forms of the CPU baseline."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-Wall", "-Wextra", "-fopenmp",
                               "-shared", "-fPIC", _SRC, _SRC_FLNS, "-o", tmp, "-lquadmath",
                               "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
                os.path.getmtime(_SRC), os.path.getmtime(_SRC_FLNS)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        for name in ("or_ternary_gemv_def", "or_ternary_pack", "or_scales_pack",
                     "or_ternary_unpack", "or_ternary_gemv_masked", "or_lns8_direct",
                     "or_lns8_tile64", "or_lns8_popcount", "or_lns8_fp64_dot",
                     "or_lmhead_brute", "or_lmhead_two_stage", "or_lmhead_stage1",
                     "or_planes_pack", "or_q1_gemv_def", "or_q1_pack", "or_q1_gemv_masked",
                     "or_flns_tables", "or_flns_log_scale", "or_flns_add", "or_flns_tree",
                     "or_flns_gemv", "or_ternary_gemv_def_mt", "or_lns8_direct_mt",
                     "or_lmhead_brute_mt", "or_max_threads"):
            getattr(lib, name).restype = ctypes.c_int
        lib.or_pad64.restype = ctypes.c_int64
        lib.or_pad64.argtypes = [ctypes.c_int64]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _i64(v):
    return ctypes.c_int64(int(v))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def pad64(rows: int) -> int:
    return (rows + 63) // 64 * 64


# --------------------------------------------------------------------------
# Ternary GEMV (integer-engine page, section 4.2)
# --------------------------------------------------------------------------

def ternary_gemv_def(t: np.ndarray, scales: np.ndarray, x: np.ndarray, frac: int = 0):
    """Definition form over unpacked trits: int64 y[rows]."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.int16)
    x = np.ascontiguousarray(x, dtype=np.int8)
    rows, k = t.shape
    assert scales.shape == (rows, k // 128) and x.shape == (k,)
    y = np.zeros(rows, dtype=np.int64)
    _check(_load().or_ternary_gemv_def(_p(t), _p(scales), _p(x), _i64(rows), _i64(k),
                                       ctypes.c_int(frac), _p(y)), "ternary_gemv_def")
    return y


def set_threads(n: int) -> int:
    """Threads the row-parallel forms use (OpenMP); returns the maximum now
    in effect."""
    lib = _load()
    lib.or_set_threads(ctypes.c_int(int(n)))
    return int(lib.or_max_threads())


def ternary_gemv_def_mt(t: np.ndarray, scales: np.ndarray, x: np.ndarray, frac: int = 0):
    """The definition form with its rows on all OpenMP threads (identical
    results; the CPU baseline's all-core leg)."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.int16)
    x = np.ascontiguousarray(x, dtype=np.int8)
    rows, k = t.shape
    assert scales.shape == (rows, k // 128) and x.shape == (k,)
    y = np.zeros(rows, dtype=np.int64)
    _check(_load().or_ternary_gemv_def_mt(_p(t), _p(scales), _p(x), _i64(rows), _i64(k),
                                          ctypes.c_int(frac), _p(y)), "ternary_gemv_def_mt")
    return y


def ternary_pack(t: np.ndarray) -> np.ndarray:
    """The tiled W_nonzero/W_negative layout, written from its description."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    rows, k = t.shape
    out = np.zeros(pad64(rows) * k // 4, dtype=np.uint8)
    _check(_load().or_ternary_pack(_p(t), _i64(rows), _i64(k), _p(out)), "ternary_pack")
    return out


def scales_pack(scales: np.ndarray) -> np.ndarray:
    scales = np.ascontiguousarray(scales, dtype=np.int16)
    rows, groups = scales.shape
    out = np.zeros(pad64(rows) * groups, dtype=np.int16)
    _check(_load().or_scales_pack(_p(scales), _i64(rows), _i64(groups * 128), _p(out)),
           "scales_pack")
    return out


def ternary_unpack(planes: np.ndarray, rows: int, k: int) -> np.ndarray:
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    t = np.zeros((rows, k), dtype=np.int8)
    _check(_load().or_ternary_unpack(_p(planes), _i64(rows), _i64(k), _p(t)),
           "ternary_unpack")
    return t


def ternary_gemv_masked(planes, pscales, x, rows: int, k: int, frac: int = 0):
    """Masked signed-sum form over packed planes and packed scales."""
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    pscales = np.ascontiguousarray(pscales, dtype=np.int16)
    x = np.ascontiguousarray(x, dtype=np.int8)
    y = np.zeros(rows, dtype=np.int64)
    _check(_load().or_ternary_gemv_masked(_p(planes), _p(pscales), _p(x), _i64(rows),
                                          _i64(k), ctypes.c_int(frac), _p(y)),
           "ternary_gemv_masked")
    return y


# --------------------------------------------------------------------------
# LNS8 eight-phase accumulation (BitState/HSDR brief v0.5, sections 3-5)
# --------------------------------------------------------------------------

def _lns8_call(fn: str, t, x, hist=False):
    t = np.ascontiguousarray(t, dtype=np.int8)
    x = np.ascontiguousarray(x, dtype=np.uint8)
    rows, k = t.shape
    acc = np.zeros((rows, 8), dtype=np.int64)
    lib = _load()
    if fn == "or_lns8_popcount":
        h = np.zeros((rows, 8, 16), dtype=np.int64)
        _check(lib.or_lns8_popcount(_p(t), _p(x), _i64(rows), _i64(k), _p(acc), _p(h)), fn)
        return (acc, h) if hist else acc
    _check(getattr(lib, fn)(_p(t), _p(x), _i64(rows), _i64(k), _p(acc)), fn)
    return acc


def lns8_direct(t, x):
    """(i) scalar direct routing A[L3] += sign*(1 << E4)."""
    return _lns8_call("or_lns8_direct", t, x)


def lns8_direct_mt(t, x):
    """(i) with the rows on all OpenMP threads (identical results)."""
    return _lns8_call("or_lns8_direct_mt", t, x)


def lns8_tile64(t, x):
    """(ii) Tile64 x 2 phase-selector masks."""
    return _lns8_call("or_lns8_tile64", t, x)


def lns8_popcount(t, x, hist=False):
    """(iii) signed POPCOUNT histogram over all 127 states, then shift/add."""
    return _lns8_call("or_lns8_popcount", t, x, hist=hist)


def lns8_fp64_dot(t, x):
    t = np.ascontiguousarray(t, dtype=np.int8)
    x = np.ascontiguousarray(x, dtype=np.uint8)
    rows, k = t.shape
    out = np.zeros(rows, dtype=np.float64)
    _check(_load().or_lns8_fp64_dot(_p(t), _p(x), _i64(rows), _i64(k), _p(out)), "fp64_dot")
    return out


def _iroot8(n: int) -> int:
    """floor(n ** (1/8)) for a non-negative integer, by Newton's method."""
    if n < 2:
        return n
    r = 1 << ((n.bit_length() + 7) // 8)      # r >= the root
    while True:
        s = (7 * r + n // r ** 7) // 8
        if s >= r:
            break
        r = s
    while r ** 8 > n:
        r -= 1
    while (r + 1) ** 8 <= n:
        r += 1
    return r


def _pow2_eighths(n: int) -> float:
    """2^(n/8) correctly rounded to binary64 (round to nearest; ties cannot
    occur because 2^(n/8) is irrational unless 8 | n)."""
    e = n // 8                                 # 2^e <= 2^(n/8) < 2^(e+1)
    big = 1 << (n - 8 * e + 8 * 52)            # (2^(n/8 - e) * 2^52)^8
    m = _iroot8(big)                           # floor of the 53-bit mantissa
    # round up iff the true mantissa exceeds m + 1/2, i.e. (2m+1)^8 < 2^8*big
    if (2 * m + 1) ** 8 < (big << 8):
        m += 1
    return float(Fraction(m) * Fraction(2) ** (e - 52))


def f_hat() -> list:
    """F[p] = 2^((p-2)/8), p = 0..7, correctly rounded to binary64."""
    return [_pow2_eighths(p - 2) for p in range(8)]


def lns8_decode(code: int) -> float:
    """|x| of a 7-bit LNS8 code: 0 for code 0, else 2^((code-74)/8)."""
    if code == 0:
        return 0.0
    return _pow2_eighths(code - 74)


def lns8_materialize(acc: np.ndarray) -> np.ndarray:
    """S[r] = 2^-9 * sum_p A[r][p]*F[p]: the exact rational value of the sum
    over the binary64 F values, rounded once to binary64."""
    fs = [Fraction(v) for v in f_hat()]
    acc = np.asarray(acc, dtype=np.int64)
    out = np.zeros(acc.shape[0], dtype=np.float64)
    scale = Fraction(1, 512)
    for r in range(acc.shape[0]):
        s = Fraction(0)
        for p in range(8):
            s += int(acc[r, p]) * fs[p]
        out[r] = float(s * scale)
    return out


# --------------------------------------------------------------------------
# Q1_0 ("A standalone deterministic integer inference engine for BitNet-style
# LLMs", section 4.1)
# --------------------------------------------------------------------------

def q1_gemv_def(s, scale, x, frac: int = 0):
    """Definition: sum_g floorshift((sum_i s_i x_i) * scale[r][g], frac)."""
    s = np.ascontiguousarray(s, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.int16)
    x = np.ascontiguousarray(x, dtype=np.int8)
    rows, k = s.shape
    y = np.empty(rows, dtype=np.int64)
    _check(_load().or_q1_gemv_def(_p(s), _p(scale), _p(x), _i64(rows), _i64(k), frac, _p(y)),
           "q1_gemv_def")
    return y


def q1_pack(s):
    """signs[rows][k] in {-1, +1} -> packed bits (1 = +1), tiled like one
    ternary plane."""
    s = np.ascontiguousarray(s, dtype=np.int8)
    rows, k = s.shape
    bits = np.zeros(pad64(rows) * k // 8, dtype=np.uint8)
    _check(_load().or_q1_pack(_p(s), _i64(rows), _i64(k), _p(bits)), "q1_pack")
    return bits


def q1_gemv_masked(bits, pscale, x, rows: int, k: int, frac: int = 0):
    """The page's masked form 2*pos_sum - block_total on packed bits/scales."""
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    pscale = np.ascontiguousarray(pscale, dtype=np.int16)
    x = np.ascontiguousarray(x, dtype=np.int8)
    y = np.empty(rows, dtype=np.int64)
    _check(_load().or_q1_gemv_masked(_p(bits), _p(pscale), _p(x), _i64(rows), _i64(k), frac,
                                     _p(y)), "q1_gemv_masked")
    return y


# --------------------------------------------------------------------------
# BITNET_PLANES lm_head (SKaiNET-transformers issue "[bitnet] T2")
# --------------------------------------------------------------------------

def planes_pack(trits: np.ndarray):
    """trits[V][8][K] -> (planes03 tiled, planes47 row-major)."""
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    V, _, K = trits.shape
    p03 = np.zeros(pad64(V) * K, dtype=np.uint8)
    p47 = np.zeros(V * K, dtype=np.uint8)
    _check(_load().or_planes_pack(_p(trits), _i64(V), _i64(K), _p(p03), _p(p47)),
           "planes_pack")
    return p03, p47


def lmhead_brute(trits, row_scale, h, top_k: int, all_scores: bool = False):
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    row_scale = np.ascontiguousarray(row_scale, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.int8)
    V, _, K = trits.shape
    idx = np.zeros(top_k, dtype=np.int32)
    sc = np.zeros(top_k, dtype=np.int64)
    allsc = np.zeros(V, dtype=np.int64)
    _check(_load().or_lmhead_brute(_p(trits), _p(row_scale), _p(h), _i64(V), _i64(K),
                                   ctypes.c_int(top_k), _p(idx), _p(sc), _p(allsc)),
           "lmhead_brute")
    return (idx, sc, allsc) if all_scores else (idx, sc)


def lmhead_brute_mt(trits, row_scale, h, top_k: int):
    """Brute force with the per-row scores on all OpenMP threads (identical
    results; the CPU baseline's all-core leg)."""
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    row_scale = np.ascontiguousarray(row_scale, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.int8)
    V, _, K = trits.shape
    idx = np.zeros(top_k, dtype=np.int32)
    sc = np.zeros(top_k, dtype=np.int64)
    _check(_load().or_lmhead_brute_mt(_p(trits), _p(row_scale), _p(h), _i64(V), _i64(K),
                                      ctypes.c_int(top_k), _p(idx), _p(sc)), "lmhead_brute_mt")
    return idx, sc


def lmhead_two_stage(trits, row_scale, h, top_k: int, cap: int, certificate: bool = False):
    """Returns (top_idx int32[k], top_score int64[k], n_candidates, capped),
    and with certificate=True also the exactness certificate (1 when the
    result is provably the exact top-k: nothing dropped, or every dropped
    candidate's upper bound strictly below the k-th output score)."""
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    row_scale = np.ascontiguousarray(row_scale, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.int8)
    V, _, K = trits.shape
    idx = np.zeros(top_k, dtype=np.int32)
    sc = np.zeros(top_k, dtype=np.int64)
    info = np.zeros(3, dtype=np.int64)
    _check(_load().or_lmhead_two_stage(_p(trits), _p(row_scale), _p(h), _i64(V), _i64(K),
                                       ctypes.c_int(top_k), ctypes.c_int(cap), _p(idx),
                                       _p(sc), _p(info)), "lmhead_two_stage")
    if certificate:
        return idx, sc, int(info[0]), int(info[1]), int(info[2])
    return idx, sc, int(info[0]), int(info[1])


def lmhead_stage1(trits, row_scale, h):
    """(S1'[V], B'[V]) of every row."""
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    row_scale = np.ascontiguousarray(row_scale, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.int8)
    V, _, K = trits.shape
    s1 = np.zeros(V, dtype=np.int64)
    b = np.zeros(V, dtype=np.int64)
    _check(_load().or_lmhead_stage1(_p(trits), _p(row_scale), _p(h), _i64(V), _i64(K),
                                    _p(s1), _p(b)), "lmhead_stage1")
    return s1, b


# --------------------------------------------------------------------------
# Pure fractional-LNS reduction (BitState/HSDR brief v0.5, section 5.2 and
# section 7 Phase A); the C side documents the coordinates and the order.
# --------------------------------------------------------------------------

_flns_cache = {}


def flns_tables(f: int) -> dict:
    """The fold and pair-add tables for f fractional bits, built in
    binary128: {"lc": int32[129], "kp": int32[n_kp], "km": int32[n_km]
    (km[0] unused), "N": 8*2^f, "margin": least distance of an entry from a
    rounding tie}."""
    if f not in _flns_cache:
        N = 8 << f
        cap = N * (f + 8)
        lc = np.zeros(129, dtype=np.int32)
        kp = np.zeros(cap, dtype=np.int32)
        km = np.zeros(cap, dtype=np.int32)
        n_kp = ctypes.c_int64(0)
        n_km = ctypes.c_int64(0)
        margin = ctypes.c_double(0)
        _check(_load().or_flns_tables(ctypes.c_int(f), _p(lc), _p(kp), _i64(cap),
                                      ctypes.byref(n_kp), _p(km), ctypes.byref(n_km),
                                      ctypes.byref(margin)), "flns_tables")
        _flns_cache[f] = {"lc": lc, "kp": kp[:n_kp.value].copy(), "km": km[:n_km.value].copy(),
                          "N": N, "margin": margin.value}
    return _flns_cache[f]


def _flns_tab_args(f: int):
    tb = flns_tables(f)
    kp = tb["kp"] if tb["kp"].size else np.zeros(1, dtype=np.int32)
    km = tb["km"] if tb["km"].size else np.zeros(1, dtype=np.int32)
    return (_p(kp), _i64(tb["kp"].size), _p(km), _i64(tb["km"].size))


def flns_log_scale(f: int, d: int) -> int:
    """round(8*2^f * log2 d): the log-domain offset of the shared scale d."""
    out = ctypes.c_int64(0)
    _check(_load().or_flns_log_scale(ctypes.c_int(f), ctypes.c_uint32(d), ctypes.byref(out)),
           "flns_log_scale")
    return out.value


def flns_add(f: int, a, b):
    """One pair add of (sign, coordinate) values (sign -1/0/+1)."""
    so = ctypes.c_int(0)
    lo = ctypes.c_int64(0)
    _check(_load().or_flns_add(*_flns_tab_args(f), ctypes.c_int(a[0]), _i64(a[1]),
                               ctypes.c_int(b[0]), _i64(b[1]), ctypes.byref(so),
                               ctypes.byref(lo)), "flns_add")
    return so.value, lo.value


def flns_tree(f: int, signs, lams):
    """The balanced pairwise reduction of explicit leaves."""
    signs = np.ascontiguousarray(signs, dtype=np.intc)
    lams = np.ascontiguousarray(lams, dtype=np.int64)
    so = ctypes.c_int(0)
    lo = ctypes.c_int64(0)
    _check(_load().or_flns_tree(*_flns_tab_args(f), _p(signs), _p(lams), _i64(signs.size),
                                ctypes.byref(so), ctypes.byref(lo)), "flns_tree")
    return so.value, lo.value


def flns_gemv(t, x, f: int, scale_d: int = 1) -> np.ndarray:
    """The whole pure-LNS row reduction: int32 out[rows][2] = (sign, L)."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    x = np.ascontiguousarray(x, dtype=np.uint8)
    rows, k = t.shape
    tb = flns_tables(f)
    out = np.zeros((rows, 2), dtype=np.int32)
    _check(_load().or_flns_gemv(_p(t), _p(x), _i64(rows), _i64(k), ctypes.c_int(f),
                                ctypes.c_uint32(scale_d), _p(tb["lc"]), *_flns_tab_args(f),
                                _p(out)), "flns_gemv")
    return out


def flns_value(out: np.ndarray, f: int) -> np.ndarray:
    """binary64 magnitude of (sign, L) results: sign * 2^((L/2^f - 74)/8).
    For error measurement only (libm exp2)."""
    out = np.asarray(out)
    lam = out[:, 1].astype(np.float64) / float(1 << f)
    return out[:, 0].astype(np.float64) * np.exp2((lam - 74.0) / 8.0)
