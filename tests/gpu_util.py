"""Shared helpers of the GPU parity tests (they call the library through the
C-ABI binding; the oracle supplies every expected value)."""
import os
import sys

import numpy as np
import pytest


def device():
    import torch
    if not torch.cuda.is_available():
        if os.environ.get("BS_REQUIRE_GPU") == "1":
            pytest.fail("BS_REQUIRE_GPU=1 but no HIP device is visible")
        pytest.skip("no HIP device")
    import bit_decode_gemv_amd as bs
    bs.lib()                      # a missing library is an error, never a skip
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def note(msg: str):
    """Name the case before each GPU step, flushed, so a crash still shows it."""
    print("[case] " + msg, file=sys.stderr, flush=True)
