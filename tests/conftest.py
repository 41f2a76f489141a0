import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case")


# Sanitizer leg (test_sanitizers.py): the oracle and the host-only part of the
# library (codec, table builder), built by gcc/g++ with
# -fsanitize=address,undefined, replace the normal builds in a child pytest
# that runs with libasan preloaded.  Only host calls are made in that child.
HOST_ONLY_CALLS = ("bs_abi_version", "bs_status_str", "bs_ternary_planes_bytes",
                   "bs_ternary_scales_count", "bs_ternary_pack", "bs_ternary_unpack",
                   "bs_ternary_pack_scales", "bs_q1_planes_bytes", "bs_q1_pack",
                   "bs_planes03_bytes", "bs_planes47_bytes", "bs_planes_pack",
                   "bs_flns_table_bytes", "bs_flns_table_build")

if os.environ.get("BS_SANITIZED_ORACLE"):
    import oracle as _oracle
    _san = os.environ["BS_SANITIZED_ORACLE"]
    _oracle._LIB_PATH = _san
    _oracle.build = lambda force=True: _san
if os.environ.get("BS_SANITIZED_HOST"):
    import ctypes as _ctypes
    import bit_decode_gemv_amd as _bs
    _h = _ctypes.CDLL(os.environ["BS_SANITIZED_HOST"])
    _bs._declare(_h, HOST_ONLY_CALLS)
    _bs._lib = _h
