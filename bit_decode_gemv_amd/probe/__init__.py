"""Binding of the benchmark's measurement kernels (``libbsprobe.so``,
declared in ``include/bs_probe.h``): a plain streaming read of a buffer and
an empty kernel.  Argument marshalling only; the kernels are HIP.  Used by
``bench.py`` to measure, in the same process and on the same stream as the
GEMVs, the read ceiling of each shape's bytes and the dispatch floor."""
from __future__ import annotations

import ctypes
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libbsprobe.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(_DIR)), "include", "bs_probe.h")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libbsprobe.so is not built (%s); run "
                              "`python -m bit_decode_gemv_amd.build`" % LIB_PATH)
        h = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        h.bs_probe_read_sink_count.restype = ctypes.c_int64
        h.bs_probe_read_sink_count.argtypes = [ctypes.c_uint64, ctypes.c_int32]
        h.bs_probe_read.restype = ctypes.c_int32
        h.bs_probe_read.argtypes = [P, ctypes.c_uint64, ctypes.c_int32, P, P]
        h.bs_probe_read_strided.restype = ctypes.c_int32
        h.bs_probe_read_strided.argtypes = [P, ctypes.c_uint64, ctypes.c_int32, P, P]
        h.bs_probe_empty.restype = ctypes.c_int32
        h.bs_probe_empty.argtypes = [ctypes.c_int32, ctypes.c_int32, P]
        _lib = h
    return _lib


def sink_for(nbytes: int, per_thread: int, device):
    """A sink tensor for ``read`` of ``nbytes`` with ``per_thread`` loads."""
    import torch
    n = lib().bs_probe_read_sink_count(int(nbytes), int(per_thread))
    if n < 0:
        raise ValueError("bs_probe_read_sink_count: status %d" % n)
    return torch.empty(n, dtype=torch.int64, device=device)


def read(src, nbytes: int, per_thread: int, sink, stream):
    """Stream ``nbytes`` of the tensor ``src`` once (bs_probe_read)."""
    if src.numel() * src.element_size() < nbytes:
        raise ValueError("src holds fewer than %d bytes" % nbytes)
    rc = lib().bs_probe_read(ctypes.c_void_p(src.data_ptr()), int(nbytes), int(per_thread),
                             ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("bs_probe_read: status %d" % rc)


def read_strided(src, nbytes: int, blocks: int, sink, stream):
    """Stream ``nbytes`` of ``src`` once with a fixed grid of ``blocks``
    workgroups (bs_probe_read_strided); ``sink`` holds blocks * 256 int64."""
    if src.numel() * src.element_size() < nbytes:
        raise ValueError("src holds fewer than %d bytes" % nbytes)
    if sink.numel() < blocks * 256:
        raise ValueError("sink holds fewer than %d values" % (blocks * 256))
    rc = lib().bs_probe_read_strided(ctypes.c_void_p(src.data_ptr()), int(nbytes), int(blocks),
                                     ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("bs_probe_read_strided: status %d" % rc)


def empty(blocks: int, threads: int, stream):
    rc = lib().bs_probe_empty(int(blocks), int(threads), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("bs_probe_empty: status %d" % rc)
