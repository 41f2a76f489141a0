"""bs_lmhead_planes_topk_noalloc (the lm_head top-k on the library's own
device scratch, for callers that cannot allocate) against the workspace entry
point bs_lmhead_planes_topk, through the C ABI: identical indices, scores and
info on consecutive calls of shrinking size, which reuse the one scratch
array, and the size limit enforced on the host."""
import ctypes

import numpy as np
import pytest

import bit_decode_gemv_amd as bs
import oracle
from bit_decode_gemv_amd import synth
from gpu_util import device, note, to_dev


def _pair(trits, rs, h, k, cap, packed=None):
    import torch
    dev = device()
    V, _, K = trits.shape
    p03, p47 = packed if packed is not None else bs.planes_pack(trits)
    a = (to_dev(p03, dev), to_dev(p47, dev), to_dev(rs, dev), to_dev(h, dev))
    note("noalloc lmhead V=%d K=%d k=%d cap=%d" % (V, K, k, cap))
    i0, s0, f0 = bs.lmhead_planes_topk(*a, V, K, k, cap)
    torch.cuda.synchronize()
    # the no-alloc call writes into outputs poisoned beforehand
    i1 = torch.full((k,), -7, dtype=torch.int32, device=dev)
    s1 = torch.full((k,), -7, dtype=torch.int64, device=dev)
    f1 = torch.full((3,), -7, dtype=torch.int32, device=dev)
    bs.lmhead_planes_topk_noalloc(*a, V, K, k, cap, top_idx=i1, top_score=s1, info=f1)
    torch.cuda.synchronize()
    got = (i1.cpu().numpy(), s1.cpu().numpy(), f1.cpu().numpy())
    want = (i0.cpu().numpy(), s0.cpu().numpy(), f0.cpu().numpy())
    for g, w in zip(got, want):
        assert (g == w).all(), (g[:8], w[:8])
    return got


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_shrinking_calls():
    # largest accepted vocabulary first, then two smaller inputs: each call
    # reuses the scratch the previous one left behind
    V = bs.LMHEAD_NOALLOC_MAX_VOCAB
    trits, rs, h = synth.lmhead(V, 128, 11)
    _pair(trits, rs, h, 40, 200)
    del trits
    trits, rs, h = synth.lmhead(20000, 512, 12)
    idx, sc, info = _pair(trits, rs, h, 40, 200)
    widx, wsc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, 40, 200, certificate=True)
    assert (idx == widx).all() and (sc == wsc).all() and list(info) == [n, capped, cert]
    trits, rs, h = synth.lmhead(3000, 256, 13)
    idx, sc, info = _pair(trits, rs, h, 10, 10)
    widx, wsc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, 10, 10, certificate=True)
    assert (idx == widx).all() and (sc == wsc).all() and list(info) == [n, capped, cert]


@pytest.mark.gpu
def test_noalloc_planted_exact_branch_twice():
    # the uncapped branch, twice in a row on the same scratch
    trits, rs, h, _ = synth.lmhead_planted(4000, 512, 1, n_peaks=64)
    for _ in range(2):
        idx, sc, info = _pair(trits, rs, h, 40, 200)
        assert info[1] == 0 and info[2] == 1
        bi, bsc = oracle.lmhead_brute(trits, rs, h, 40)
        assert (idx == bi).all() and (sc == bsc).all()


def test_noalloc_rejects_vocab_beyond_scratch():
    # host validation only: the call returns before any HIP call, so fake
    # (aligned, never dereferenced) device pointers suffice
    lib = bs.lib()
    fake = ctypes.c_void_p(1 << 20)
    V = bs.LMHEAD_NOALLOC_MAX_VOCAB
    rc = lib.bs_lmhead_planes_topk_noalloc(fake, fake, fake, fake, V + 1, 128, 40, 200,
                                           fake, fake, fake, None)
    assert rc == bs.BS_E_WORKSPACE
    # the other checks come first and match the workspace entry point
    assert lib.bs_lmhead_planes_topk_noalloc(None, fake, fake, fake, V, 128, 40, 200, fake,
                                             fake, fake, None) == bs.BS_E_NULL
    assert lib.bs_lmhead_planes_topk_noalloc(fake, fake, fake, fake, V, 130, 40, 200, fake,
                                             fake, fake, None) == bs.BS_E_SHAPE
    assert lib.bs_lmhead_planes_topk_noalloc(fake, fake, fake, fake, V, 128, 201, 200, fake,
                                             fake, fake, None) == bs.BS_E_RANGE
