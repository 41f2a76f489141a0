#!/usr/bin/env python3
"""Benchmark of the batch-1 ternary decode GEMV hot path on one MI355X.

One step = one BitNet-b1.58-2B-shaped decode layer's projections: q, k, v
(2560, 640, 640 rows x 2560), o (2560 x 2560), gate and up (6912 x 2560 each)
and down (2560 x 6912), on packed ternary planes (0.25 B/weight) plus int16
group scales, int8 activations, exact int64 outputs.  The projections that
share an input are stored concatenated by rows, as decode engines store them:
q|k|v is one 3840 x 2560 matrix and gate|up one 13824 x 2560 matrix, so a step
is four dependent launches (qkv, o, gate_up, down) streaming the same bytes as
the seven separate GEMVs.  q|k|v and gate|up write fresh outputs
(bs_ternary_gemv); o and down add into the residual stream, as a decoder
layer's output projections do (bs_ternary_gemv_acc, y += W x).  The seven-launch form of the same
step (each projection a row range of the same buffers) is timed as well and
reported in `config`.  Steps walk a pool of distinct layers whose weights
total more than 1 GiB, so every GEMV streams its weights from HBM rather than
the 256 MB Infinity Cache; inputs are resident in HBM before the timed region.

Timing: the K timed steps are captured once in a HIP graph and replayed on one
stream between two HIP events (plus a host wall clock).  `value` is the
weight-stream throughput of the whole job: weight bytes of all K steps over
the elapsed time.  The roofline entry is for the dominant kernel (the one
with the largest share of step time): its algorithmic bytes per launch over
its average launch duration, measured with HIP events around a graph of
back-to-back launches of that kernel alone on the same stream.

Extra entries ("ops") time the other workloads of the path: the larger-K
GEMVs, the LNS8 eight-phase GEMV (both reductions) and the BITNET_PLANES
lm_head top-k.  `cpu_baseline` times the plain C oracle, single-threaded, on
a bounded sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
       python bench.py --trace-summary <rocprofv3 kernel_trace.csv>
       python bench.py --traffic-run NxK          (workload of the --pmc runs)
       python bench.py --traffic-summary FETCH.csv WRITE.csv NxK
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
METRIC = "ternary GEMV weight-stream GB/s & % HBM peak, batch-1, K=2560..5120"
LAYER = [("q", 2560, 2560), ("k", 640, 2560), ("v", 640, 2560), ("o", 2560, 2560),
         ("gate", 6912, 2560), ("up", 6912, 2560), ("down", 2560, 6912)]
# launches of one step: (name, member projections stored concatenated by rows)
FUSED = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
         ("down", ("down",))]
RESIDUAL = ("o", "down")        # output projections: y += W x into the residual stream


def weight_bytes(rows: int, k: int) -> int:
    """Algorithmic weight-stream bytes of one GEMV: planes (k/4 per row) plus
    int16 scales (2 bytes per 128 weights)."""
    return rows * k // 4 + rows * (k // 128) * 2


def log(msg: str):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Timer:
    """Graph replay timing on one stream with HIP events."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def graph(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    fn(i)
        return g

    def replay_us(self, g, reps=1):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(self.stream)
            for _ in range(reps):
                g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) * 1000.0, wall * 1e6


def per_launch_us(timer, fn, n=200, reps=5):
    g = timer.graph(fn, n)
    timer.replay_us(g)                         # warm
    us, _ = timer.replay_us(g, reps)
    return us / (n * reps)


def make_pool(torch, bs, synth, dev, rows, k, seed, min_bytes):
    """Packed planes/scales for one shape, replicated into distinct buffers
    totalling at least min_bytes."""
    t, sc, x = synth.ternary(rows, k, seed)
    p = torch.from_numpy(bs.ternary_pack(t)).to(dev)
    s = torch.from_numpy(bs.ternary_pack_scales(sc)).to(dev)
    n = max(2, -(-min_bytes // weight_bytes(rows, k)))
    return [p.clone() for _ in range(n)], [s.clone() for _ in range(n)], torch.from_numpy(x).to(dev)


def cpu_baseline(seconds_target: float):
    """The oracle's definition-form GEMV, single-threaded, over the step's
    seven shapes at full size (seed 0), repeated until about seconds_target
    of CPU time; reported in the metric's unit (weight-stream bytes per
    second of the packed format the GPU reads)."""
    import numpy as np
    import oracle
    from bit_decode_gemv_amd import synth
    cases = [synth.ternary(r, k, 0) for _, r, k in LAYER]
    step_bytes = sum(weight_bytes(r, k) for _, r, k in LAYER)
    done, t_cpu = 0, 0.0
    while t_cpu < seconds_target:
        for t, sc, x in cases:
            t0 = time.process_time()
            oracle.ternary_gemv_def(t, sc, x)
            t_cpu += time.process_time() - t0
        done += 1
    gbs = done * step_bytes / t_cpu / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full step(s) (q,k,v,o,gate,up,down at full size, seed 0) through "
                      "or_ternary_gemv_def on unpacked int8 trits, single thread, %.1f s CPU"
                      % (done, t_cpu),
            "cpu_model": _cpu_model(), "ms_per_step": round(1000.0 * t_cpu / done, 2),
            "per_config": _oracle_per_config()}


def _oracle_per_config():
    """The oracle's other entry points, single-threaded, each timed once on
    one seeded input (median of 3 where it takes under a second)."""
    import numpy as np
    import oracle
    from bit_decode_gemv_amd import synth

    def med(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.process_time()
            fn()
            ts.append(time.process_time() - t0)
        return statistics.median(ts)

    out = {}
    t, sc, x = synth.tiny(0)
    out["ternary_256x512_us"] = round(1e6 * med(lambda: oracle.ternary_gemv_def(t, sc, x), 3), 1)
    t, sc, x = synth.ternary(13824, 5120, 0)
    sec = med(lambda: oracle.ternary_gemv_def(t, sc, x), 3)
    out["ternary_13824x5120_us"] = round(1e6 * sec, 1)
    out["ternary_13824x5120_GBps"] = round(weight_bytes(13824, 5120) / sec / 1e9, 4)
    t8, x8 = synth.lns8(4096, 4096, 0)
    out["lns8_4096x4096_direct_us"] = round(1e6 * med(lambda: oracle.lns8_direct(t8, x8), 3), 1)
    out["lns8_4096x4096_popcount_us"] = round(
        1e6 * med(lambda: oracle.lns8_popcount(t8, x8), 1), 1)
    V = 16384
    trits, rs, h = synth.lmhead(V, 2560, 0)
    scale = synth.LMHEAD_SHAPE[0] / V
    out["lmhead_two_stage_us_scaled_from_16384_rows"] = round(
        1e6 * scale * med(lambda: oracle.lmhead_two_stage(trits, rs, h, 40, 200), 1), 1)
    out["lmhead_brute_us_scaled_from_16384_rows"] = round(
        1e6 * scale * med(lambda: oracle.lmhead_brute(trits, rs, h, 40), 1), 1)
    del np
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _source_digest():
    """Digest of the GEMV kernel's source: its file and the headers it
    includes (shared device helpers, status codes, the ABI header)."""
    h = hashlib.sha256()
    for rel in (("bit_decode_gemv_amd", "csrc", "ternary_gemv.hip"),
                ("bit_decode_gemv_amd", "csrc", "kcommon.h"),
                ("bit_decode_gemv_amd", "csrc", "bs_internal.h"),
                ("include", "bs.h")):
        with open(os.path.join(ROOT, *rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _recorded_traffic(shape_tag: str):
    """HBM bytes per launch recorded by rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, scaled by the copy-kernel calibration), stored as text under
    profiles/.  Returned only if the kernel source has not changed since."""
    path = os.path.join(ROOT, "profiles", "ternary_gemv_%s_hbm_traffic.txt" % shape_tag)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != _source_digest():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def context(torch, dev, timer):
    """The empty-launch floor (a one-element fill, back to back in a graph)
    and a 1 GiB read through torch's float32 sum, for scale."""
    one = torch.zeros(1, dtype=torch.int32, device=dev)
    floor_us = per_launch_us(timer, lambda i: one.fill_(i), n=200)
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    acc = torch.empty(1, dtype=torch.float32, device=dev)
    # eager, not graph-captured (a multi-block reduction may record memset nodes)
    with torch.cuda.stream(timer.stream):
        torch.sum(big, dim=0, keepdim=True, out=acc)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(timer.stream)
        for _ in range(10):
            torch.sum(big, dim=0, keepdim=True, out=acc)
        e1.record(timer.stream)
    torch.cuda.synchronize()
    read_us = e0.elapsed_time(e1) * 1000.0 / 10
    del big
    return {"launch_floor_us": round(floor_us, 3),
            "read_1GiB_GBps": round((1 << 30) / read_us / 1e3, 1),
            "read_1GiB_note": "torch.sum over 2^28 float32 (a reduction, so a lower bound on "
                              "the read ceiling), 10 eager launches between HIP events"}


def activation_reuse_sweep(torch, bs, synth, dev, timer, k=2560):
    """us and weight-stream GB/s of one launch as the rows sharing one staged
    activation vector grow (K = 2560): where the kernel turns bandwidth-bound."""
    out = {}
    for rows in (64, 256, 1024, 2560, 6912, 13824, 27648, 55296):
        ps, ss, x = make_pool(torch, bs, synth, dev, rows, k, 0, 1 << 30)
        y = torch.empty(rows, dtype=torch.int64, device=dev)
        us = per_launch_us(timer, lambda i: bs.ternary_gemv(ps[i % len(ps)], ss[i % len(ss)], x,
                                                            rows, k, out=y), n=100)
        wb = weight_bytes(rows, k)
        out[str(rows)] = {"us": round(us, 3), "GBps": round(wb / us / 1e3, 1)}
        del ps, ss
    log("activation-reuse sweep: " + ", ".join("%s rows %.0f GB/s" % (r, v["GBps"])
                                                for r, v in out.items()))
    return out


def run_extras(torch, bs, synth, dev, timer):
    ops = {}
    # larger-K GEMVs
    for rows, k in synth.LARGE_K_SHAPES:
        ps, ss, x = make_pool(torch, bs, synth, dev, rows, k, 0, 1 << 30)
        y = torch.empty(rows, dtype=torch.int64, device=dev)
        us = per_launch_us(timer, lambda i: bs.ternary_gemv(ps[i % len(ps)], ss[i % len(ss)], x,
                                                            rows, k, out=y), n=100)
        wb = weight_bytes(rows, k)
        ops["ternary_gemv_%dx%d" % (rows, k)] = {
            "us_per_gemv": round(us, 3), "weight_bytes": wb, "GBps": round(wb / us / 1e3, 1),
            "frac_hbm_peak": round(wb / us / 1e3 / HBM_PEAK_GBS, 4)}
        del ps, ss
        log("ternary %dx%d: %.2f us" % (rows, k, us))
    # Q1_0 (one sign bit per weight): the four launches of a BitNet-2B layer
    # and the largest K in range
    q1_bytes = lambda r, k: r * k // 8 + r * (k // 128) * 2
    for rows, k in [(3840, 2560), (2560, 2560), (13824, 2560), (2560, 6912), (13824, 5120)]:
        sgn, sc, x = synth.q1(rows, k, 0)
        b = torch.from_numpy(bs.q1_pack(sgn)).to(dev)
        s = torch.from_numpy(bs.ternary_pack_scales(sc)).to(dev)
        n = max(2, -(-(1 << 30) // q1_bytes(rows, k)))
        bp, sp = [b.clone() for _ in range(n)], [s.clone() for _ in range(n)]
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty(rows, dtype=torch.int64, device=dev)
        us = per_launch_us(timer, lambda i: bs.q1_gemv(bp[i % n], sp[i % n], xd, rows, k,
                                                       out=y), n=100)
        wb = q1_bytes(rows, k)
        ops["q1_gemv_%dx%d" % (rows, k)] = {
            "us_per_gemv": round(us, 3), "weight_bytes": wb, "GBps": round(wb / us / 1e3, 1),
            "frac_hbm_peak": round(wb / us / 1e3 / HBM_PEAK_GBS, 4)}
        del bp, sp
        log("q1 %dx%d: %.2f us" % (rows, k, us))
    # LNS8 eight-phase GEMV, 4096 x 4096
    t8, x8 = synth.lns8(4096, 4096, 0)
    p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
    pool8 = [p8.clone() for _ in range(-(-(1 << 30) // p8.numel()))]
    xd8 = torch.from_numpy(x8).to(dev)
    acc = torch.empty((4096, 8), dtype=torch.int32, device=dev)
    s8 = torch.empty(4096, dtype=torch.float64, device=dev)
    ws8 = torch.zeros(bs.lib().bs_lns8_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    for path, name in ((bs.LNS8_DIRECT, "direct"), (bs.LNS8_POPCOUNT, "popcount")):
        us = per_launch_us(timer, lambda i: bs.lns8_phase_gemv(pool8[i % len(pool8)], xd8, 4096,
                                                               4096, path, acc=acc, s=s8,
                                                               workspace=ws8), n=100)
        ops["lns8_4096x4096_" + name] = {
            "us_per_gemv": round(us, 3), "weight_bytes": p8.numel(),
            "GBps": round(p8.numel() / us / 1e3, 1),
            "frac_hbm_peak": round(p8.numel() / us / 1e3 / HBM_PEAK_GBS, 4),
            "weights_per_s": round(4096 * 4096 / us * 1e6, 1)}
        log("lns8 %s: %.2f us" % (name, us))
    # pure fractional-LNS reduction of the same products, by internal
    # precision: time per call and the error of the decoded result against the
    # exact dyadic S of the linear path above (sign * 2^((L/2^f - 74)/8))
    import numpy as np
    s_exact = s8.clone()
    bs.lns8_phase_gemv(p8, xd8, 4096, 4096, bs.LNS8_DIRECT, acc=acc, s=s_exact, workspace=ws8)
    torch.cuda.synchronize()
    s_ref = s_exact.cpu().numpy()
    wsf = torch.zeros(bs.lib().bs_flns_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    outf = torch.empty((4096, 2), dtype=torch.int32, device=dev)
    flns = {}
    for f in (0, 2, 4, 8, 12):
        tb = torch.from_numpy(bs.flns_table(f)).to(dev)
        us = per_launch_us(timer, lambda i: bs.flns_phase_gemv(pool8[i % len(pool8)], xd8, 4096,
                                                               4096, f, tb, out=outf,
                                                               workspace=wsf), n=50, reps=3)
        bs.flns_phase_gemv(p8, xd8, 4096, 4096, f, tb, out=outf, workspace=wsf)
        torch.cuda.synchronize()
        o = outf.cpu().numpy().astype(np.float64)
        val = o[:, 0] * np.exp2((o[:, 1] / float(1 << f) - 74.0) / 8.0) * (o[:, 0] != 0)
        big = np.abs(s_ref) >= 1e-3 * np.median(np.abs(s_ref))
        rel = np.abs(val[big] - s_ref[big]) / np.abs(s_ref[big])
        flns["f%d" % f] = {"us_per_gemv": round(us, 3),
                           "GBps": round(p8.numel() / us / 1e3, 1),
                           "rel_err_median": float("%.3g" % np.median(rel)),
                           "rel_err_p99": float("%.3g" % np.quantile(rel, 0.99)),
                           "rel_err_max": float("%.3g" % rel.max()),
                           "rows_compared": int(big.sum())}
        log("flns f=%d: %.2f us, median rel err %.3g" % (f, us, np.median(rel)))
    ops["flns_4096x4096"] = {"error_vs": "exact dyadic S of the linear eight-phase path "
                                         "(rows with |S| >= 1e-3 x median |S|)", **flns}
    del pool8
    # steps either side of the GEMVs: absmax int8 quantisation of the
    # activation vector (the q|k|v and down inputs), LNS8 encoding of the
    # eight-phase input, and the candidate sampler on a top-40 (one launch
    # each; a decode step runs them once per vector)
    rng = np.random.default_rng(0)
    for k in (2560, 6912):
        xq = torch.from_numpy(rng.integers(-(1 << 40), 1 << 40, k).astype(np.int64)).to(dev)
        qo = torch.empty(k, dtype=torch.int8, device=dev)
        am = torch.empty(1, dtype=torch.int64, device=dev)
        stq = torch.empty(1, dtype=torch.int32, device=dev)
        us = per_launch_us(timer, lambda i: bs.act_quant_i8(xq, q=qo, absmax=am, status=stq),
                           n=100)
        ops["act_quant_i8_k%d" % k] = {"us_per_call": round(us, 3)}
    xe = torch.from_numpy((rng.standard_normal(4096) * 2.0 ** 20).astype(np.int64)).to(dev)
    eo = torch.empty(4096, dtype=torch.uint8, device=dev)
    ops["lns8_encode_k4096"] = {"us_per_call": round(per_launch_us(
        timer, lambda i: bs.lns8_encode(xe, 16, out=eo), n=100), 3)}
    ci = torch.from_numpy(rng.permutation(128256)[:40].astype(np.int32)).to(dev)
    cs = torch.from_numpy(np.sort(rng.integers(0, 1 << 30, 40))[::-1].copy()).to(dev)
    res = torch.empty(6, dtype=torch.int64, device=dev)
    ops["sample_candidates_n40"] = {"us_per_call": round(per_launch_us(
        timer, lambda i: bs.sample_candidates(ci, cs, bs.SAMPLE_DRAW, beta_q16=1 << 10, seed=1,
                                              position=i, result=res), n=100), 3)}
    log("edges: quant %.2f us, encode %.2f us, sample %.2f us" % (
        ops["act_quant_i8_k2560"]["us_per_call"], ops["lns8_encode_k4096"]["us_per_call"],
        ops["sample_candidates_n40"]["us_per_call"]))
    # BITNET_PLANES lm_head, 128256 x 2560, top-40, cap 200
    V, K = synth.LMHEAD_SHAPE
    trits, rs, h = synth.lmhead(V, K, 0)
    p03, p47 = bs.planes_pack(trits)
    del trits
    d03, d47 = torch.from_numpy(p03).to(dev), torch.from_numpy(p47).to(dev)
    drs, dh = torch.from_numpy(rs).to(dev), torch.from_numpy(h).to(dev)
    pool03 = [d03] + [d03.clone() for _ in range(3)]       # > 1 GiB of planes 0-3
    idx = torch.empty(40, dtype=torch.int32, device=dev)
    sc = torch.empty(40, dtype=torch.int64, device=dev)
    info = torch.empty(2, dtype=torch.int32, device=dev)
    wsl = torch.zeros(bs.lib().bs_lmhead_workspace_bytes(V, K, 40, 200), dtype=torch.uint8,
                      device=dev)
    us = per_launch_us(timer, lambda i: bs.lmhead_planes_topk(
        pool03[i % 4], d47, drs, dh, V, K, 40, 200, top_idx=idx, top_score=sc, info=info,
        workspace=wsl), n=20, reps=3)
    stage1_bytes = p03.size + rs.nbytes
    ops["lmhead_planes_topk_128256x2560"] = {
        "us_per_call": round(us, 3), "stage1_bytes": stage1_bytes,
        "GBps_stage1_bytes": round(stage1_bytes / us / 1e3, 1),
        "frac_hbm_peak": round(stage1_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
        "n_candidates": int(info[0].item()), "capped": int(info[1].item())}
    log("lm_head: %.2f us" % us)
    return ops


def trace_summary(path: str):
    """Per (kernel, grid) durations from a rocprofv3 --kernel-trace CSV."""
    rows = list(csv.DictReader(open(path)))
    groups = {}
    for r in rows:
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
        key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = []
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append("%-70s grid %8d wg %4d calls %6d avg %8.3f us median %8.3f us min %8.3f us"
                   % (name[:70], grid, wg, len(d), statistics.mean(d) / 1e3,
                      statistics.median(d) / 1e3, min(d) / 1e3))
    return "\n".join(out)


CALIB_BYTES = 256 << 20         # the calibration kernel reads and writes this many bytes


def traffic_run(shape: str, launches: int = 20):
    """Workload for the rocprofv3 --pmc runs behind roofline.traffic: three
    launches of a plain elementwise kernel of known size (int32 negation,
    CALIB_BYTES read and CALIB_BYTES written: the counter calibration), then
    `launches` launches of the ternary GEMV of `shape` on distinct weight
    buffers (> 1 GiB in total, so they stream from HBM)."""
    import torch
    import bit_decode_gemv_amd as bs
    from bit_decode_gemv_amd import synth
    rows, k = (int(v) for v in shape.split("x"))
    dev = torch.device("cuda:0")
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    ps, ss, x = make_pool(torch, bs, synth, dev, rows, k, 0, 1 << 30)
    y = torch.empty(rows, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    for i in range(launches):
        bs.ternary_gemv(ps[i % len(ps)], ss[i % len(ss)], x, rows, k, out=y)
    torch.cuda.synchronize()
    log("traffic run done: 3 calibration launches, %d GEMV launches of %s" % (launches, shape))


def traffic_summary(fetch_csv: str, write_csv: str, shape: str):
    """HBM bytes per GEMV launch from two rocprofv3 counter CSVs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by the calibration kernel's
    reading of the same counter against its known byte count."""
    rows, k = (int(v) for v in shape.split("x"))

    def per_kernel(path, counter):
        calib, gemv = [], []
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            name = r["Kernel_Name"]
            if "ternary_rows_kernel" in name or "ternary_tile_kernel" in name:
                gemv.append(v)
            elif "neg" in name:
                calib.append(v)
        return calib, gemv

    fc, fg = per_kernel(fetch_csv, "FETCH_SIZE")
    wc, wg = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = CALIB_BYTES / statistics.mean(fc)
    w_scale = CALIB_BYTES / statistics.mean(wc)
    fetch = statistics.mean(fg) * f_scale
    write = statistics.mean(wg) * w_scale
    lines = [
        "shape: %s" % shape,
        "kernel_source_sha256_16: %s" % _source_digest(),
        "calibration_fetch_counter_bytes: %.0f (known %d, factor %.4f)"
        % (statistics.mean(fc), CALIB_BYTES, f_scale),
        "calibration_write_counter_bytes: %.0f (known %d, factor %.4f)"
        % (statistics.mean(wc), CALIB_BYTES, w_scale),
        "gemv_launches: %d fetch, %d write" % (len(fg), len(wg)),
        "fetch_bytes_per_launch: %.0f" % fetch,
        "write_bytes_per_launch: %.0f" % write,
        "hbm_bytes_per_launch: %.0f" % (fetch + write),
        "algorithmic_bytes_per_launch: %d (weights %d + activations %d + outputs %d)"
        % (weight_bytes(rows, k) + k + 8 * rows, weight_bytes(rows, k), k, 8 * rows),
    ]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extras", action="store_true", help="skip the non-headline workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--trace-summary", help="summarise a rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--traffic-run", metavar="NxK",
                    help="run the workload of the --pmc traffic measurement and exit")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "NxK"),
                    help="HBM bytes per launch from the two counter CSVs and exit")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary))
        return 0
    if args.traffic_run:
        traffic_run(args.traffic_run)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the GEMVs would "
              "shard by rows with one all-gather, or by K with one int64 all-reduce); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import bit_decode_gemv_amd as bs
    from bit_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    bs.lib()
    stream = torch.cuda.Stream(device=dev)
    timer = Timer(torch, stream)

    # layer pool: distinct weights for every layer, > 1 GiB in total.  Each
    # launch's matrix is its member projections' rows, concatenated; a member
    # is a row range of it (offsets are multiples of 64 rows, which is a
    # valid packed matrix in both the plane and the scale layout).
    import numpy as np
    shape = {name: (r, k) for name, r, k in LAYER}
    seed = {name: li for li, (name, _, _) in enumerate(LAYER)}
    step_bytes = sum(weight_bytes(r, k) for _, r, k in LAYER)
    n_layers = -(-(1 << 30) // step_bytes) + 1
    log("building %d layers of synthetic BitNet-2B projections (%.1f MB each)" % (
        n_layers, step_bytes / 1e6))
    base = {}
    for fname, members in FUSED:
        parts = [synth.ternary(*shape[m], seed[m]) for m in members]
        t = np.concatenate([pt[0] for pt in parts])
        sc = np.concatenate([pt[1] for pt in parts])
        k = shape[members[0]][1]
        base[fname] = (torch.from_numpy(bs.ternary_pack(t)).to(dev),
                       torch.from_numpy(bs.ternary_pack_scales(sc)).to(dev),
                       torch.from_numpy(parts[0][2]).to(dev), t.shape[0], k)
        del t, sc, parts
    layers = [{f: (base[f][0].clone(), base[f][1].clone()) for f, _ in FUSED}
              for _ in range(n_layers)]
    # outputs; the residual-stream accumulators start at zero and only grow by
    # |W x| < 2^35 per step, far from int64's range over the run
    ys = {f: torch.zeros(base[f][3], dtype=torch.int64, device=dev) for f, _ in FUSED}
    member_of = {}
    for fname, members in FUSED:
        row0 = 0
        for m in members:
            member_of[m] = (fname, row0)
            row0 += shape[m][0]

    def launch_fused(i, fname):
        p, s = layers[i % n_layers][fname]
        _, _, x, r, k = base[fname]
        if fname in RESIDUAL:
            bs.ternary_gemv_acc(p, s, x, r, k, ys[fname])
        else:
            bs.ternary_gemv(p, s, x, r, k, out=ys[fname])

    def launch_member(i, m):
        fname, row0 = member_of[m]
        p, s = layers[i % n_layers][fname]
        x, k = base[fname][2], base[fname][4]
        r = shape[m][0]
        pv = p[row0 * k // 4:(row0 + r) * k // 4]
        sv = s[row0 * (k // 128):(row0 + r) * (k // 128)]
        if fname in RESIDUAL:
            bs.ternary_gemv_acc(pv, sv, x, r, k, ys[fname][row0:row0 + r])
        else:
            bs.ternary_gemv(pv, sv, x, r, k, out=ys[fname][row0:row0 + r])

    def step(i):
        for fname, _ in FUSED:
            launch_fused(i, fname)

    def step7(i):
        for m, _, _ in LAYER:
            launch_member(i, m)

    # warmup, then the timed graph of exactly `steps` steps
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    g = timer.graph(lambda i: step(args.warmup + i), args.steps)
    timer.replay_us(g)                          # first replay uploads the graph
    us, wall_us = timer.replay_us(g)
    ms_per_step = us / 1000.0 / args.steps
    value = step_bytes * args.steps / (us * 1e-6) / 1e9
    log("step (4 launches): %.3f ms (events), %.3f ms (host wall) -> %.1f GB/s" % (
        ms_per_step, wall_us / 1000.0 / args.steps, value))
    del g
    g7 = timer.graph(lambda i: step7(args.warmup + i), args.steps)
    timer.replay_us(g7)
    us7, _ = timer.replay_us(g7)
    value7 = step_bytes * args.steps / (us7 * 1e-6) / 1e9
    log("step (7 launches): %.3f ms -> %.1f GB/s" % (us7 / 1000.0 / args.steps, value7))
    del g7

    # per-launch durations: the step's four launches and the seven members;
    # the dominant kernel is the step launch with the largest share
    launch_us = {f: per_launch_us(timer, lambda i, f=f: launch_fused(i, f)) for f, _ in FUSED}
    member_us = {}
    for m, r, k in LAYER:
        if "%dx%d" % (r, k) not in member_us:
            member_us["%dx%d" % (r, k)] = round(per_launch_us(
                timer, lambda i, m=m: launch_member(i, m)), 3)
    dom = max(launch_us, key=lambda f: launch_us[f])
    dom_us = launch_us[dom]
    dom_rows, dom_k = base[dom][3], base[dom][4]
    dom_bytes = weight_bytes(dom_rows, dom_k)
    achieved = dom_bytes / dom_us / 1e3
    tag = "%dx%d" % (dom_rows, dom_k)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": _recorded_traffic(tag),
                "kernel": "%s %s (%s, 1 launch per step)" % (
                    "bs_ternary_gemv_acc" if dom in RESIDUAL else "bs_ternary_gemv", tag, dom),
                "us_per_launch": round(dom_us, 3), "bytes_per_launch": dom_bytes}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": "bitnet-b1.58-2B decode projections q,k,v,o,gate,up,down, "
                               "batch 1; q|k|v and gate|up stored concatenated by rows: "
                               "4 dependent launches per step (qkv, gate_up: bs_ternary_gemv; "
                               "o, down: bs_ternary_gemv_acc into the residual stream)",
                   "launches": {f: "%dx%d" % (base[f][3], base[f][4]) for f, _ in FUSED},
                   "weight_bytes_per_step": step_bytes, "layers_in_pool": n_layers,
                   "pool_bytes": step_bytes * n_layers, "parallelism": "single GPU",
                   "frac_hbm_peak_whole_job": round(value / HBM_PEAK_GBS, 4),
                   "host_wall_ms_per_step": round(wall_us / 1000.0 / args.steps, 5),
                   "us_per_launch": {f: round(v, 3) for f, v in launch_us.items()},
                   "seven_launch_step": {"ms_per_step": round(us7 / 1000.0 / args.steps, 5),
                                         "GBps": round(value7, 1),
                                         "us_per_gemv": member_us}},
        "roofline": roofline,
    }
    if not args.no_extras:
        out["ops"] = run_extras(torch, bs, synth, dev, timer)
        out["ops"]["activation_reuse_sweep_k2560"] = activation_reuse_sweep(
            torch, bs, synth, dev, timer)
        out["context"] = context(torch, dev, timer)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (~%.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
