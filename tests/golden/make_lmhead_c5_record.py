"""Writes lmhead_c5_record.json: for the BITNET_PLANES lm_head workload
(vocab 128256 x dim 2560, k = 40, cap = 200; inputs from
bit_decode_gemv_amd.synth.lmhead, seeds 0..4) the two-stage decode's result
and info (|C|, capped, exactness certificate) and the brute-force exact
top-k, both from the oracle only ("[bitnet] T2: lm_head via BITNET_PLANES
weight format (WeightForm) + two-stage top-k decode": the result is checked
against an exact full eight-plane scoring), and whether they are equal.

    python tests/golden/make_lmhead_c5_record.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from bit_decode_gemv_amd import synth  # noqa: E402

K_TOP, CAP = 40, 200


def main():
    out = {"workload": "lm_head vocab 128256 x dim 2560, k = 40, cap = 200, synth.lmhead",
           "seeds": {}}
    oracle.set_threads(len(os.sched_getaffinity(0)))
    for seed in range(5):
        trits, rs, h = synth.lmhead(*synth.LMHEAD_SHAPE, seed=seed)
        idx, sc, n, capped, cert = oracle.lmhead_two_stage(trits, rs, h, K_TOP, CAP,
                                                           certificate=True)
        bi, bsc = oracle.lmhead_brute_mt(trits, rs, h, K_TOP)
        equal = bool((idx == bi).all() and (sc == bsc).all())
        out["seeds"][str(seed)] = {
            "n_candidates": n, "capped": capped, "certified": cert, "equals_brute_force": equal,
            "two_stage_idx": idx.tolist(), "two_stage_score": [int(v) for v in sc],
            "brute_idx": bi.tolist(), "brute_score": [int(v) for v in bsc]}
        print("seed %d: |C| = %d, capped = %d, certified = %d, equals brute force: %s"
              % (seed, n, capped, cert, equal), flush=True)
        del trits
    oracle.set_threads(1)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lmhead_c5_record.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
