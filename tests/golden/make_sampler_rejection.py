"""Writes sampler_rejection.json: draw keys (seed, position) whose first
attempt Lemire's method rejects, for the sampler's GPU parity test.  Uses
only the oracle (oracle/edges.py): the draw source, the bounded draw and the
sampler itself.

683 candidates of equal score with inverse temperature 0 all weigh 2^31
(Q31), so the kept total is T = 683 * 2^31 and 2^64 mod T = 682 * 2^31 (2^33
= -1 mod 683): a draw is rejected with probability about 2^-23.6, the
largest any total of at most 1024 candidates allows.  The search runs over
positions for a few seeds in parallel processes until it has found `want`
keys.

Run from the repository root:  python tests/golden/make_sampler_rejection.py
"""
import json
import multiprocessing as mp
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import edges  # noqa: E402

N_CAND = 683
TOTAL = N_CAND << 31
REJECT_BELOW = (1 << 64) % TOTAL


def _scan(args):
    seed, p0, p1 = args
    hits = []
    for pos in range(p0, p1):
        lo = (edges.draw_u64(seed, pos, 0) * TOTAL) & ((1 << 64) - 1)
        if lo < REJECT_BELOW:
            hits.append((seed, pos))
    return hits


def main(want=2, chunk=1 << 20):
    assert REJECT_BELOW == 682 << 31
    found = []
    with mp.Pool(8) as pool:
        tasks = ((seed, c * chunk, (c + 1) * chunk) for seed in (1, 2, 3) for c in range(64))
        for hits in pool.imap(_scan, tasks):
            found.extend(hits)
            if len(found) >= want:
                pool.terminate()
                break
    cases = []
    idx = list(range(1000, 1000 + N_CAND))
    score = [5] * N_CAND
    for seed, pos in found[:want]:
        o = edges.sample_candidates(idx, score, edges.SAMPLE_DRAW, beta=0, seed=seed, position=pos)
        assert o["attempts"] >= 2 and o["total"] == TOTAL
        cases.append({"seed": seed, "position": pos, "attempts": o["attempts"],
                      "draw": o["draw"], "token": o["token"], "rank": o["rank"]})
    out = {"note": "683 equal scores from index 1000, beta 0: first draw rejected",
           "n": N_CAND, "first_index": 1000, "score": 5, "total": TOTAL, "cases": cases}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sampler_rejection.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
