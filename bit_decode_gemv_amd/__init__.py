"""Python binding of the gfx950 ternary decode-GEMV library (``libbitstate.so``).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels (or, for the load-time codec, its host C++).  PyTorch supplies
device memory and streams.  There is no fallback: if the shared library is
missing, every call raises.

Names follow the C ABI declared in ``include/bs.h``:

* codec (host, NumPy arrays): ``ternary_pack``, ``ternary_unpack``,
  ``ternary_pack_scales``, ``q1_pack``, ``planes_pack``, ``flns_table``;
* device (torch tensors on a HIP device): ``ternary_gemv``, ``q1_gemv``,
  ``lns8_phase_gemv``, ``flns_phase_gemv``, ``lmhead_planes_topk``.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbitstate.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "bs.h")

BS_OK, BS_E_NULL, BS_E_SHAPE, BS_E_RANGE, BS_E_OVERFLOW, BS_E_HIP, BS_E_WORKSPACE, BS_E_ALIGN = (
    0, -1, -2, -3, -4, -5, -6, -7)
LNS8_DIRECT, LNS8_POPCOUNT, LNS8_MATRIX = 0, 1, 2

_lib = None


class BsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_str(status), status))


def _declare(lib, only=None):
    """Result and argument types of the exported calls (of those in `only`,
    when given: a library built from a subset of the sources)."""
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "bs_abi_version": (I32, []),
        "bs_status_str": (ctypes.c_char_p, [I32]),
        "bs_ternary_planes_bytes": (I64, [I64, I64]),
        "bs_ternary_scales_count": (I64, [I64, I64]),
        "bs_ternary_pack": (I32, [P, I64, I64, P]),
        "bs_ternary_unpack": (I32, [P, I64, I64, P]),
        "bs_ternary_pack_scales": (I32, [P, I64, I64, P]),
        "bs_ternary_gemv": (I32, [P, P, P, I64, I64, I32, P, P]),
        "bs_ternary_gemv_acc": (I32, [P, P, P, I64, I64, I32, P, P]),
        "bs_q1_planes_bytes": (I64, [I64, I64]),
        "bs_q1_pack": (I32, [P, I64, I64, P]),
        "bs_q1_gemv": (I32, [P, P, P, I64, I64, I32, P, P]),
        "bs_lns8_workspace_bytes": (SZ, [I64, I64]),
        "bs_lns8_phase_gemv": (I32, [P, P, I64, I64, I32, P, P, P, SZ, P]),
        "bs_flns_table_bytes": (I64, [I32]),
        "bs_flns_table_build": (I32, [I32, P, I64]),
        "bs_flns_workspace_bytes": (SZ, [I64, I64]),
        "bs_flns_phase_gemv": (I32, [P, P, I64, I64, I32, ctypes.c_uint32, P, I64, P, P, SZ, P]),
        "bs_planes03_bytes": (I64, [I64, I64]),
        "bs_planes47_bytes": (I64, [I64, I64]),
        "bs_planes_pack": (I32, [P, I64, I64, P, P]),
        "bs_lmhead_workspace_bytes": (SZ, [I64, I64, I32, I32]),
        "bs_lmhead_planes_topk": (I32, [P, P, P, P, I64, I64, I32, I32, P, P, P, P, SZ, P]),
        "bs_lmhead_planes_topk_noalloc": (I32, [P, P, P, P, I64, I64, I32, I32, P, P, P, P]),
        "bs_act_quant_i8": (I32, [P, I64, P, P, P, P]),
        "bs_lns8_encode": (I32, [P, I64, I32, P, P]),
        "bs_lns8_encode_edges": (I32, [I32, P]),
        "bs_sample_candidates": (I32, [P, P, I32, I32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64, P, P]),
    }
    for name, (res, args) in sig.items():
        if only is not None and name not in only:
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libbitstate.so is not built (%s); run "
                              "`python -m bit_decode_gemv_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _lib = handle
    return _lib


def header_symbols() -> list:
    """Every function name declared in include/bs.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bs_[a-z0-9_]+)\s*\(", text)))


def status_str(status: int) -> str:
    return lib().bs_status_str(int(status)).decode()


def _check(rc: int, where: str):
    if rc != BS_OK:
        raise BsError(rc, where)


def _np_ptr(a: np.ndarray):
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("array must be C-contiguous")
    return ctypes.c_void_p(a.ctypes.data)


# --------------------------------------------------------------------- codec

def ternary_pack(t: np.ndarray) -> np.ndarray:
    """int8 trits [rows][k] -> packed W_nonzero/W_negative planes (uint8)."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    rows, k = t.shape
    n = lib().bs_ternary_planes_bytes(rows, k)
    if n < 0:
        raise BsError(int(n), "bs_ternary_planes_bytes")
    out = np.empty(n, dtype=np.uint8)
    _check(lib().bs_ternary_pack(_np_ptr(t), rows, k, _np_ptr(out)), "bs_ternary_pack")
    return out


def q1_pack(signs: np.ndarray) -> np.ndarray:
    """int8 signs [rows][k] in {-1, +1} -> packed sign bits (uint8)."""
    signs = np.ascontiguousarray(signs, dtype=np.int8)
    rows, k = signs.shape
    n = lib().bs_q1_planes_bytes(rows, k)
    if n < 0:
        raise BsError(int(n), "bs_q1_planes_bytes")
    out = np.empty(n, dtype=np.uint8)
    _check(lib().bs_q1_pack(_np_ptr(signs), rows, k, _np_ptr(out)), "bs_q1_pack")
    return out


def ternary_unpack(planes: np.ndarray, rows: int, k: int) -> np.ndarray:
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    need = lib().bs_ternary_planes_bytes(rows, k)
    if need < 0:
        raise BsError(int(need), "bs_ternary_planes_bytes")
    if planes.size < need:
        raise ValueError("planes buffer too small")
    t = np.empty((rows, k), dtype=np.int8)
    _check(lib().bs_ternary_unpack(_np_ptr(planes), rows, k, _np_ptr(t)), "bs_ternary_unpack")
    return t


def ternary_pack_scales(scales: np.ndarray) -> np.ndarray:
    """int16 scales [rows][k/128] -> packed int16 scales."""
    scales = np.ascontiguousarray(scales, dtype=np.int16)
    rows, groups = scales.shape
    n = lib().bs_ternary_scales_count(rows, groups * 128)
    if n < 0:
        raise BsError(int(n), "bs_ternary_scales_count")
    out = np.empty(n, dtype=np.int16)
    _check(lib().bs_ternary_pack_scales(_np_ptr(scales), rows, groups * 128, _np_ptr(out)),
           "bs_ternary_pack_scales")
    return out


def planes_pack(trits: np.ndarray):
    """int8 trits [vocab][8][dim] -> (planes03, planes47) uint8."""
    trits = np.ascontiguousarray(trits, dtype=np.int8)
    vocab, eight, dim = trits.shape
    if eight != 8:
        raise ValueError("trits must be [vocab][8][dim]")
    n03 = lib().bs_planes03_bytes(vocab, dim)
    n47 = lib().bs_planes47_bytes(vocab, dim)
    if n03 < 0 or n47 < 0:
        raise BsError(int(min(n03, n47)), "bs_planes_bytes")
    p03 = np.empty(n03, dtype=np.uint8)
    p47 = np.empty(n47, dtype=np.uint8)
    _check(lib().bs_planes_pack(_np_ptr(trits), vocab, dim, _np_ptr(p03), _np_ptr(p47)),
           "bs_planes_pack")
    return p03, p47


def flns_table(frac_bits: int) -> np.ndarray:
    """The pure fractional-LNS table blob for frac_bits (host uint8); copy it
    to the device as is for ``flns_phase_gemv``."""
    n = lib().bs_flns_table_bytes(int(frac_bits))
    if n <= 0:
        raise BsError(BS_E_RANGE, "bs_flns_table_bytes")
    blob = np.zeros(n, dtype=np.uint8)
    _check(lib().bs_flns_table_build(int(frac_bits), _np_ptr(blob), n), "bs_flns_table_build")
    return blob


# ------------------------------------------------------------------ device

def _torch():
    import torch
    return torch


def _dptr(t, dtype, name):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("%s must be a torch tensor on a HIP device" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


class Workspace:
    """Zero-filled device scratch, one per (entry point, device), grown on
    demand.  The split-K entry points (LNS8, pure fractional-LNS) need it
    zero before their first call and leave it zero; the others write every
    byte they read.  So one buffer serves every call of that entry point
    ordered on one stream; entry points never share a buffer."""

    _cache = {}

    @classmethod
    def get(cls, op: str, nbytes: int, device):
        torch = _torch()
        dev = torch.device(device)
        key = (op, dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
        buf = cls._cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
            cls._cache[key] = buf
        return buf


def _ws(op, ws, nbytes, device):
    torch = _torch()
    if ws is None:
        ws = Workspace.get(op, nbytes, device)
    if ws.dtype != torch.uint8 or ws.device.type != "cuda":
        raise TypeError("workspace must be a uint8 tensor on a HIP device")
    return ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())


def _need(t, n, name):
    """Device buffers are checked for size here, so a kernel never reads past
    the end of a tensor the caller passed."""
    if t is not None and t.numel() < n:
        raise ValueError("%s has %d elements, needs %d" % (name, t.numel(), n))


def ternary_gemv(planes, scales, x, rows: int, k: int, frac: int = 0, out=None,
                 stream=None):
    """y = bs_ternary_gemv(planes, scales, x): int64[rows] on x's device."""
    torch = _torch()
    if out is None:
        out = torch.empty(rows, dtype=torch.int64, device=x.device)
    nplanes = lib().bs_ternary_planes_bytes(rows, k)
    if nplanes < 0:
        raise BsError(int(nplanes), "bs_ternary_planes_bytes")
    _need(planes, nplanes, "planes")
    _need(scales, lib().bs_ternary_scales_count(rows, k), "scales")
    _need(x, k, "x")
    _need(out, rows, "y")
    rc = lib().bs_ternary_gemv(_dptr(planes, torch.uint8, "planes"),
                               _dptr(scales, torch.int16, "scales"),
                               _dptr(x, torch.int8, "x"), rows, k, frac,
                               _dptr(out, torch.int64, "y"),
                               _stream_handle(stream, x.device))
    _check(rc, "bs_ternary_gemv")
    return out


def ternary_gemv_acc(planes, scales, x, rows: int, k: int, y, frac: int = 0, stream=None):
    """y += bs_ternary_gemv(planes, scales, x) in place (int64[rows] on x's
    device); returns y."""
    torch = _torch()
    nplanes = lib().bs_ternary_planes_bytes(rows, k)
    if nplanes < 0:
        raise BsError(int(nplanes), "bs_ternary_planes_bytes")
    _need(planes, nplanes, "planes")
    _need(scales, lib().bs_ternary_scales_count(rows, k), "scales")
    _need(x, k, "x")
    _need(y, rows, "y")
    rc = lib().bs_ternary_gemv_acc(_dptr(planes, torch.uint8, "planes"),
                                   _dptr(scales, torch.int16, "scales"),
                                   _dptr(x, torch.int8, "x"), rows, k, int(frac),
                                   _dptr(y, torch.int64, "y"), _stream_handle(stream, x.device))
    _check(rc, "bs_ternary_gemv_acc")
    return y


def q1_gemv(bits, scales, x, rows: int, k: int, frac: int = 0, out=None, stream=None):
    """y = bs_q1_gemv(bits, scales, x): int64[rows] on x's device."""
    torch = _torch()
    if out is None:
        out = torch.empty(rows, dtype=torch.int64, device=x.device)
    nbits = lib().bs_q1_planes_bytes(rows, k)
    if nbits < 0:
        raise BsError(int(nbits), "bs_q1_planes_bytes")
    _need(bits, nbits, "bits")
    _need(scales, lib().bs_ternary_scales_count(rows, k), "scales")
    _need(x, k, "x")
    _need(out, rows, "y")
    rc = lib().bs_q1_gemv(_dptr(bits, torch.uint8, "bits"), _dptr(scales, torch.int16, "scales"),
                          _dptr(x, torch.int8, "x"), rows, k, frac, _dptr(out, torch.int64, "y"),
                          _stream_handle(stream, x.device))
    _check(rc, "bs_q1_gemv")
    return out


def lns8_phase_gemv(planes, x_lns8, rows: int, k: int, path: int = LNS8_DIRECT, acc=None,
                    s=True, workspace=None, stream=None):
    """(acc int32[rows][8], s float64[rows] or None).  ``workspace``, when
    given, is a uint8 device tensor of at least bs_lns8_workspace_bytes that
    is zero before its first use (every call leaves it zero); by default a
    zero-filled one is kept per device."""
    torch = _torch()
    dev = x_lns8.device
    if acc is None:
        acc = torch.empty((rows, 8), dtype=torch.int32, device=dev)
    if s is True:
        s = torch.empty(rows, dtype=torch.float64, device=dev)
    elif s is False:
        s = None
    need = lib().bs_lns8_workspace_bytes(rows, k)
    if need == 0:
        raise BsError(BS_E_SHAPE, "bs_lns8_workspace_bytes")
    _need(planes, lib().bs_ternary_planes_bytes(rows, k), "planes")
    _need(x_lns8, k, "x_lns8")
    _need(acc, rows * 8, "acc")
    _need(s, rows, "s")
    wp, wn = _ws("lns8_phase_gemv", workspace, need, dev)
    rc = lib().bs_lns8_phase_gemv(_dptr(planes, torch.uint8, "planes"),
                                  _dptr(x_lns8, torch.uint8, "x_lns8"), rows, k, int(path),
                                  _dptr(acc, torch.int32, "acc"),
                                  _dptr(s, torch.float64, "s") if s is not None else None,
                                  wp, wn, _stream_handle(stream, dev))
    _check(rc, "bs_lns8_phase_gemv")
    return acc, s


def flns_phase_gemv(planes, x_lns8, rows: int, k: int, frac_bits: int, table, scale_d: int = 1,
                    out=None, workspace=None, stream=None):
    """out int32[rows][2] = (sign, L) of the pure fractional-LNS reduction;
    ``table`` is the device copy of ``flns_table(frac_bits)``.  ``workspace``,
    when given, is a uint8 device tensor of at least bs_flns_workspace_bytes
    (reserved by the interface, never read or written); by default one is
    kept per device."""
    torch = _torch()
    dev = x_lns8.device
    if out is None:
        out = torch.empty((rows, 2), dtype=torch.int32, device=dev)
    need = lib().bs_flns_workspace_bytes(rows, k)
    if need == 0:
        raise BsError(BS_E_SHAPE, "bs_flns_workspace_bytes")
    _need(planes, lib().bs_ternary_planes_bytes(rows, k), "planes")
    _need(x_lns8, k, "x_lns8")
    _need(out, rows * 2, "out")
    wp, wn = _ws("flns_phase_gemv", workspace, need, dev)
    rc = lib().bs_flns_phase_gemv(_dptr(planes, torch.uint8, "planes"),
                                  _dptr(x_lns8, torch.uint8, "x_lns8"), rows, k, int(frac_bits),
                                  int(scale_d), _dptr(table, torch.uint8, "table"),
                                  table.numel(), _dptr(out, torch.int32, "out"), wp, wn,
                                  _stream_handle(stream, dev))
    _check(rc, "bs_flns_phase_gemv")
    return out


def lmhead_planes_topk(planes03, planes47, row_scale, h, vocab: int, dim: int,
                       top_k: int = 40, max_candidates: int = 200, top_idx=None,
                       top_score=None, info=None, workspace=None, stream=None):
    """(top_idx int32[top_k], top_score int64[top_k], info int32[3]: |C|,
    capped, certified exact)."""
    torch = _torch()
    dev = h.device
    if top_idx is None:
        top_idx = torch.empty(top_k, dtype=torch.int32, device=dev)
    if top_score is None:
        top_score = torch.empty(top_k, dtype=torch.int64, device=dev)
    if info is None:
        info = torch.empty(3, dtype=torch.int32, device=dev)
    need = lib().bs_lmhead_workspace_bytes(vocab, dim, top_k, max_candidates)
    if need == 0:
        raise BsError(BS_E_RANGE, "bs_lmhead_workspace_bytes")
    _need(planes03, lib().bs_planes03_bytes(vocab, dim), "planes03")
    _need(planes47, lib().bs_planes47_bytes(vocab, dim), "planes47")
    _need(row_scale, vocab, "row_scale")
    _need(h, dim, "h")
    _need(top_idx, top_k, "top_idx")
    _need(top_score, top_k, "top_score")
    _need(info, 3, "info")
    wp, wn = _ws("lmhead_planes_topk", workspace, need, dev)
    rc = lib().bs_lmhead_planes_topk(
        _dptr(planes03, torch.uint8, "planes03"), _dptr(planes47, torch.uint8, "planes47"),
        _dptr(row_scale, torch.int32, "row_scale"), _dptr(h, torch.int8, "h"), vocab, dim,
        top_k, max_candidates, _dptr(top_idx, torch.int32, "top_idx"),
        _dptr(top_score, torch.int64, "top_score"), _dptr(info, torch.int32, "info"),
        wp, wn, _stream_handle(stream, dev))
    _check(rc, "bs_lmhead_planes_topk")
    return top_idx, top_score, info


LMHEAD_NOALLOC_MAX_VOCAB = 262144     # BS_LMHEAD_NOALLOC_MAX_VOCAB


def lmhead_planes_topk_noalloc(planes03, planes47, row_scale, h, vocab: int, dim: int,
                               top_k: int = 40, max_candidates: int = 200, top_idx=None,
                               top_score=None, info=None, stream=None):
    """bs_lmhead_planes_topk_noalloc: the lm_head top-k with the library's own
    device scratch (no workspace).  Outputs as ``lmhead_planes_topk``; pass
    preallocated ``top_idx``/``top_score``/``info`` to allocate nothing here
    either."""
    torch = _torch()
    dev = h.device
    if top_idx is None:
        top_idx = torch.empty(top_k, dtype=torch.int32, device=dev)
    if top_score is None:
        top_score = torch.empty(top_k, dtype=torch.int64, device=dev)
    if info is None:
        info = torch.empty(3, dtype=torch.int32, device=dev)
    _need(planes03, lib().bs_planes03_bytes(vocab, dim), "planes03")
    _need(planes47, lib().bs_planes47_bytes(vocab, dim), "planes47")
    _need(row_scale, vocab, "row_scale")
    _need(h, dim, "h")
    _need(top_idx, top_k, "top_idx")
    _need(top_score, top_k, "top_score")
    _need(info, 3, "info")
    rc = lib().bs_lmhead_planes_topk_noalloc(
        _dptr(planes03, torch.uint8, "planes03"), _dptr(planes47, torch.uint8, "planes47"),
        _dptr(row_scale, torch.int32, "row_scale"), _dptr(h, torch.int8, "h"), vocab, dim,
        top_k, max_candidates, _dptr(top_idx, torch.int32, "top_idx"),
        _dptr(top_score, torch.int64, "top_score"), _dptr(info, torch.int32, "info"),
        _stream_handle(stream, dev))
    _check(rc, "bs_lmhead_planes_topk_noalloc")
    return top_idx, top_score, info


# ------------------------------------------------- steps around the GEMVs

SAMPLE_GREEDY, SAMPLE_DRAW = 0, 1


def lns8_encode_edges(frac: int) -> np.ndarray:
    """Host: the encoder's integer code edges for frac (uint64[128])."""
    e = np.zeros(128, dtype=np.uint64)
    _check(lib().bs_lns8_encode_edges(int(frac), _np_ptr(e)), "bs_lns8_encode_edges")
    return e


def act_quant_i8(x, q=None, absmax=None, status=None, stream=None):
    """(q int8[k], absmax int64[1], status int32[1]) on x's device."""
    torch = _torch()
    dev = x.device
    k = x.numel()
    if q is None:
        q = torch.empty(k, dtype=torch.int8, device=dev)
    if absmax is None:
        absmax = torch.empty(1, dtype=torch.int64, device=dev)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _need(q, k, "q")
    _need(absmax, 1, "absmax")
    _need(status, 1, "status")
    rc = lib().bs_act_quant_i8(_dptr(x, torch.int64, "x"), k, _dptr(q, torch.int8, "q"),
                               _dptr(absmax, torch.int64, "absmax"),
                               _dptr(status, torch.int32, "status"), _stream_handle(stream, dev))
    _check(rc, "bs_act_quant_i8")
    return q, absmax, status


def lns8_encode(x, frac: int, out=None, stream=None):
    """LNS8 bytes (uint8[k]) of the int64 fixed-point vector x."""
    torch = _torch()
    dev = x.device
    k = x.numel()
    if out is None:
        out = torch.empty(k, dtype=torch.uint8, device=dev)
    _need(out, k, "out")
    rc = lib().bs_lns8_encode(_dptr(x, torch.int64, "x"), k, int(frac),
                              _dptr(out, torch.uint8, "out"), _stream_handle(stream, dev))
    _check(rc, "bs_lns8_encode")
    return out


def sample_candidates(idx, score, mode: int, beta_q16: int = 1 << 16, top_p_q16: int = 1 << 16,
                      min_p_q16: int = 0, seed: int = 0, position: int = 0, n: int = None,
                      result=None, stream=None):
    """int64[6] on the device: token, rank, kept ranks, kept total, draw,
    SHA-256 attempts."""
    torch = _torch()
    dev = score.device
    n = score.numel() if n is None else int(n)
    if result is None:
        result = torch.empty(6, dtype=torch.int64, device=dev)
    _need(idx, n, "idx")
    _need(score, n, "score")
    _need(result, 6, "result")
    rc = lib().bs_sample_candidates(_dptr(idx, torch.int32, "idx"),
                                    _dptr(score, torch.int64, "score"), n, int(mode),
                                    int(beta_q16), int(top_p_q16), int(min_p_q16),
                                    int(seed) & ((1 << 64) - 1), int(position) & ((1 << 64) - 1),
                                    _dptr(result, torch.int64, "result"),
                                    _stream_handle(stream, dev))
    _check(rc, "bs_sample_candidates")
    return result
