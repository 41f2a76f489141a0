#!/usr/bin/env python3
"""Benchmark of the batch-1 ternary decode GEMV hot path on one MI355X.

Headline (`value`): weight-stream GB/s of the per-configuration ternary GEMVs
with K in [2560, 5120], each a separate `bs_ternary_gemv` launch on its own
weights: the six K = 2560 projections of a BitNet-b1.58-2B decode layer (q,
k, v, o: 2560/640/640/2560 x 2560; gate, up: 6912 x 2560) and the larger-K
11008 x 4096 and 13824 x 5120.  One step = those eight launches (44.5 MB of
packed planes + int16 scales).  Weights are ternary with P(0) = 0.4, int16
group scales uniform in [1, 4096], int8 activations rint(N(0, 32^2))
clipped to +-127, seed 0.  Steps walk a pool of distinct weight sets of more
than 1.1 GB, so every launch streams its weights from HBM rather than the
256 MB Infinity Cache; inputs are resident in HBM before the timed region.
The K timed steps are captured in one HIP graph, replayed once (upload),
then a 512 MB read evicts the caches and the graph is replayed between two
HIP events on its stream.

`roofline` is for the largest configuration shape, 13824 x 5120: algorithmic
bytes per launch (planes N*K/4 + scales N*K/64) over the kernel's average
launch duration, measured with HIP events on the launch stream around a
graph of back-to-back launches that visits every buffer of a 512 MB pool
once (the profiler's kernel-trace durations of the same launches agree).
Every shape of the five configurations also gets, in `ops.gemv`, its back-
to-back time, a plain read of the same bytes from the same pool (the read
ceiling, `bs_probe_read`) and the fraction of that ceiling reached.
`context` holds the empty-kernel launch floor.

`ops.f1` holds the activation-reuse sweep (N = 1 .. 8192 rows sharing one
activation vector, ternary GEMV and the three LNS8 paths, with the row counts
where popcount overtakes direct routing and matrix overtakes popcount), the
Phase B sweeps of the LNS8
GEMV (weight zero density, number of distinct activation codes) and the
fused four-launch layer step.  Other `ops` entries time the rest of the path:
Q1_0, LNS8 (with the VALU fraction), pure-LNS, the steps either side and the
lm_head.  `cpu_baseline` times the plain C oracle on the host: all cores
(OpenMP over rows) and single-threaded, medians of repeated samples.

Every measured block is preceded by a marker launch (an empty kernel whose
grid encodes the block) so that one `rocprofv3 --kernel-trace` run of this
script can be split per block and shape by `--trace-summary`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
                       [--no-cpu-baseline] [--cpu-seconds S]
       python bench.py --trace-summary <rocprofv3 kernel_trace.csv>
       python bench.py --traffic-run NxK       (workload of the --pmc runs)
       python bench.py --traffic-summary FETCH.csv WRITE.csv NxK
       python bench.py --lns8-counter-run      (workload of the LNS8 --pmc runs)
       python bench.py --flns-counter-run      (workload of the pure-LNS --pmc runs)
       python bench.py --counter-summary COUNTERS.csv
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
VALU_PEAK_OPS = 256 * 64 * 2.4e9   # 256 CUs x 64 int32 lane-ops per clock x 2.4 GHz
MFMA_I8_PEAK_OPS = 5.0e15      # MI355X published dense int8 matrix rate (ops/s)
IC_BYTES = 256 << 20           # MI355X Infinity Cache
METRIC = "ternary GEMV weight-stream GB/s & % HBM peak, batch-1, K=2560..5120"
# one step: the in-range per-configuration GEMVs, one launch each
STEP = [("q", 2560, 2560), ("k", 640, 2560), ("v", 640, 2560), ("o", 2560, 2560),
        ("gate", 6912, 2560), ("up", 6912, 2560), ("c3_11008x4096", 11008, 4096),
        ("c3_13824x5120", 13824, 5120)]
IN_RANGE = [(2560, 2560), (640, 2560), (6912, 2560), (11008, 4096), (13824, 5120)]
REPORTED = [(2560, 6912), (4096, 11008), (5120, 13824)]     # K outside 2560..5120
ROOF_SHAPE = (13824, 5120)
STEP_POOL_BYTES = int(1.1 * (1 << 30))
SHAPE_POOL_BYTES = 2 * IC_BYTES
# the BitNet-2B layer stored as four launches (f1: shared-activation fusion)
LAYER = [("q", 2560, 2560), ("k", 640, 2560), ("v", 640, 2560), ("o", 2560, 2560),
         ("gate", 6912, 2560), ("up", 6912, 2560), ("down", 2560, 6912)]
FUSED = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
         ("down", ("down",))]
RESIDUAL = ("o", "down")
# marker ids of the measured blocks (empty-kernel grid = (4096 + id) x 64)
MARKER_BASE = 4096
BLOCKS = ["step", "roofline_graph", "context_floor", "ceiling_scrub",
          "f1_fused_step", "lmhead", "lns8", "flns", "q1", "edges", "lmhead_ceiling",
          "context_stream"]
SHAPE_BLOCKS = ["gemv_%dx%d" % s for s in IN_RANGE + REPORTED]
SWEEP_BLOCKS = ["f1_reuse_%s_n%d" % (p, n) for p in ("ternary", "direct", "popcount", "matrix")
                for n in (1, 8, 32, 128, 512, 2048, 8192)]
PHASE_B_BLOCKS = (["f1_zero_%s_%s" % (p, z) for p in ("direct", "popcount", "matrix")
                   for z in ("0", "1/3", "0.6", "0.9")] +
                  ["f1_codes_%s_%d" % (p, m) for p in ("direct", "popcount", "matrix")
                   for m in (1, 8, 41, 127)] +
                  ["f1_k_%s_%d" % (p, k) for p in ("direct", "popcount", "matrix")
                   for k in (1024, 2048, 4096, 8192, 16384, 32768)])
ALL_BLOCKS = BLOCKS + SHAPE_BLOCKS + SWEEP_BLOCKS + PHASE_B_BLOCKS + ["concurrent_step"]
MARKER_ID = {name: i + 1 for i, name in enumerate(ALL_BLOCKS)}
# the LNS8 paths by their bs.h ids (DIRECT, POPCOUNT, MATRIX)
LNS8_PATHS_BY_ID = ((0, "direct"), (1, "popcount"), (2, "matrix"))
LNS8_PATHS = LNS8_PATHS_BY_ID


def weight_bytes(rows: int, k: int) -> int:
    """Algorithmic weight-stream bytes of one GEMV: planes (k/4 per row) plus
    int16 scales (2 bytes per 128 weights)."""
    return rows * k // 4 + rows * (k // 128) * 2


def log(msg: str):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Harness:
    """Graph-replay timing on one stream with HIP events, plus the
    measurement kernels (read ceiling, launch floor, markers)."""

    def __init__(self, torch, dev):
        from bit_decode_gemv_amd import probe
        self.torch = torch
        self.dev = dev
        self.stream = torch.cuda.Stream(device=dev)
        self.probe = probe
        probe.lib()
        self.scrub_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.scrub_sink = probe.sink_for(self.scrub_buf.numel(), 8, dev)

    def marker(self, block: str):
        with self.torch.cuda.stream(self.stream):
            self.probe.empty(MARKER_BASE + MARKER_ID[block], 64, self.stream)

    def scrub(self):
        """Read 512 MB of an unrelated buffer: afterwards no weight line is
        left in the L2s or the Infinity Cache."""
        self.probe.read(self.scrub_buf, self.scrub_buf.numel(), 8, self.scrub_sink, self.stream)

    def graph(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    fn(i)
        return g

    def replay_us(self, g, scrub=False):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            if scrub:
                self.scrub()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) * 1000.0, wall * 1e6

    def per_launch(self, fn, n, reps=3, block=None):
        """Median over `reps` replays of a graph of n back-to-back launches
        (each replay visits the whole pool once), in us per launch."""
        if block:
            self.marker(block)
        g = self.graph(fn, n)
        self.replay_us(g)                       # upload
        us = sorted(self.replay_us(g)[0] / n for _ in range(reps))
        del g
        return us[len(us) // 2]

    def ceiling(self, pool, nbytes, n, block=None):
        """Best back-to-back time of a plain read of `nbytes` from each pool
        buffer in turn: one pass with 2, 4 or 8 16-byte loads per thread, or
        a fixed grid of 512, 1024 or 2048 workgroups striding over it."""
        best = None
        for u in (2, 4, 8):
            sink = self.probe.sink_for(nbytes, u, self.dev)
            us = self.per_launch(lambda i: self.probe.read(pool[i % len(pool)], nbytes, u, sink,
                                                           self.stream), n, block=block)
            best = us if best is None else min(best, us)
        sink = self.torch.empty(2048 * 256, dtype=self.torch.int64, device=self.dev)
        for blocks in (512, 1024, 2048):
            us = self.per_launch(lambda i: self.probe.read_strided(
                pool[i % len(pool)], nbytes, blocks, sink, self.stream), n, block=block)
            best = min(best, us)
        return best


def packed_pool(torch, bs, synth, dev, rows, k, min_bytes, seed=0, max_copies=None):
    """Packed planes and scales of one seeded shape, copied into distinct
    device buffers (planes then scales in one allocation) totalling at least
    min_bytes.  Returns (buffers, views [(planes, scales)], x, bytes each)."""
    import numpy as np
    t, sc, x = synth.ternary(rows, k, seed)
    pl = bs.ternary_pack(t)
    ps = bs.ternary_pack_scales(sc)
    base = torch.from_numpy(np.concatenate([pl, ps.view(np.uint8)])).to(dev)
    n = max(2, -(-min_bytes // base.numel()))
    if max_copies:
        n = min(n, max_copies)
    bufs = carve_copies(torch, base, n, dev)
    views = [(b[:pl.size], b[pl.size:].view(torch.int16)) for b in bufs]
    return bufs, views, torch.from_numpy(x).to(dev), base.numel()


def carve_copies(torch, base, n, dev):
    """n copies of a uint8 device tensor, each 4 KiB-aligned inside one
    allocation (a model's weights sit in one allocation too; separate
    allocations per copy measured about 1 % slower on first touch)."""
    stride = -(-base.numel() // 4096) * 4096
    big = torch.empty(stride * n, dtype=torch.uint8, device=dev)
    out = []
    for i in range(n):
        b = big[i * stride:i * stride + base.numel()]
        b.copy_(base)
        out.append(b)
    return out


# ---------------------------------------------------------------- CPU side

def _cpu_model():
    """/proc/cpuinfo's model name, with the family and model numbers (a
    virtual machine may report only a generic name) and the logical CPUs."""
    vals = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                vals.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    name = vals.get("model name", "unknown")
    return "%s (family %s, model %s; %d logical CPUs, %d in this process's affinity)" % (
        name, vals.get("cpu family", "?"), vals.get("model", "?"), os.cpu_count() or 0,
        len(os.sched_getaffinity(0)))


def _baseline_threads():
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_baseline(seconds_target: float):
    """The oracle's definition-form GEMV over the headline step's eight
    shapes at full size (seed 0), on all host cores (rows shared out by
    OpenMP; identical results) and on one thread: the median of five
    samples, each as many steps as fill about seconds_target / 10 of wall
    time, in the metric's unit (weight-stream bytes of the packed format the
    GPU reads, per second).  Per-configuration oracle timings beside it."""
    import oracle
    from bit_decode_gemv_amd import synth
    cases = [synth.ternary(r, k, 0) for _, r, k in STEP]
    step_bytes = sum(weight_bytes(r, k) for _, r, k in STEP)
    cores = oracle.set_threads(_baseline_threads())

    def sample(fn, budget):
        done, t0 = 0, time.perf_counter()
        while True:
            for t, sc, x in cases:
                fn(t, sc, x)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done * step_bytes / el / 1e9, el / done

    mt = sorted(sample(oracle.ternary_gemv_def_mt, seconds_target / 10) for _ in range(5))
    st = sorted(sample(oracle.ternary_gemv_def, seconds_target / 10) for _ in range(5))
    out = {"value": round(mt[2][0], 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": "median of 5 samples of %.1f s wall each: full headline steps (the eight "
                     "per-configuration GEMVs, seed 0) through the definition-form oracle on "
                     "unpacked int8 trits, rows on %d OpenMP threads" % (seconds_target / 10,
                                                                         cores),
           "cpu_model": _cpu_model(), "ms_per_step": round(1000.0 * mt[2][1], 2),
           "single_thread": {"value": round(st[2][0], 4), "unit": "GB/s", "cores": 1,
                             "ms_per_step": round(1000.0 * st[2][1], 2)}}
    out["per_config"] = _oracle_per_config(cores)
    oracle.set_threads(1)
    return out


def _oracle_per_config(cores):
    """The oracle's other entry points on one seeded input each, median of
    three wall times, single thread and (row-parallel forms) all cores."""
    import oracle
    from bit_decode_gemv_amd import synth

    def med(fn, reps=3):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    out = {}
    t, sc, x = synth.tiny(0)
    oracle.set_threads(1)
    out["ternary_256x512_us"] = round(1e6 * med(lambda: oracle.ternary_gemv_def(t, sc, x)), 1)
    t, sc, x = synth.ternary(13824, 5120, 0)
    for tag, fn, n in (("1t", oracle.ternary_gemv_def, 1), ("mt", oracle.ternary_gemv_def_mt,
                                                             cores)):
        oracle.set_threads(n)
        sec = med(lambda: fn(t, sc, x))
        out["ternary_13824x5120_%s_us" % tag] = round(1e6 * sec, 1)
        out["ternary_13824x5120_%s_GBps" % tag] = round(weight_bytes(13824, 5120) / sec / 1e9, 4)
    t8, x8 = synth.lns8(4096, 4096, 0)
    oracle.set_threads(1)
    out["lns8_4096x4096_direct_1t_us"] = round(1e6 * med(lambda: oracle.lns8_direct(t8, x8)), 1)
    oracle.set_threads(cores)
    out["lns8_4096x4096_direct_mt_us"] = round(
        1e6 * med(lambda: oracle.lns8_direct_mt(t8, x8)), 1)
    oracle.set_threads(1)
    out["lns8_4096x4096_popcount_1t_us"] = round(
        1e6 * med(lambda: oracle.lns8_popcount(t8, x8), 1), 1)
    V = 16384
    trits, rs, h = synth.lmhead(V, 2560, 0)
    scale = synth.LMHEAD_SHAPE[0] / V
    out["lmhead_two_stage_1t_us_scaled_from_16384_rows"] = round(
        1e6 * scale * med(lambda: oracle.lmhead_two_stage(trits, rs, h, 40, 200), 1), 1)
    out["lmhead_brute_1t_us_scaled_from_16384_rows"] = round(
        1e6 * scale * med(lambda: oracle.lmhead_brute(trits, rs, h, 40), 1), 1)
    oracle.set_threads(cores)
    out["lmhead_brute_mt_us_scaled_from_16384_rows"] = round(
        1e6 * scale * med(lambda: oracle.lmhead_brute_mt(trits, rs, h, 40), 1), 1)
    oracle.set_threads(1)
    return out


# ------------------------------------------------------ records under profiles/

def _source_digest(kernel_file="ternary_gemv.hip"):
    """Digest of a kernel's source: its file, the headers it includes
    (shared device helpers, status codes, the ABI header) and the build
    script that holds the compiler flags."""
    h = hashlib.sha256()
    for rel in (("bit_decode_gemv_amd", "csrc", kernel_file),
                ("bit_decode_gemv_amd", "csrc", "kcommon.h"),
                ("bit_decode_gemv_amd", "csrc", "bs_internal.h"),
                ("include", "bs.h"),
                ("bit_decode_gemv_amd", "build.py")):
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


# ------------------------------------------------------------ GPU workloads

def run_step(torch, bs, synth, dev, H, steps, warmup):
    """The headline: K steps of the eight in-range per-configuration GEMVs."""
    import numpy as np
    step_bytes = sum(weight_bytes(r, k) for _, r, k in STEP)
    n_sets = -(-STEP_POOL_BYTES // step_bytes)
    log("building %d weight sets of the %d-launch step (%.1f MB each, %.2f GB in all)" % (
        n_sets, len(STEP), step_bytes / 1e6, n_sets * step_bytes / 1e9))
    bases, xs, ys = {}, {}, {}
    for name, rows, k in STEP:
        t, sc, x = synth.ternary(rows, k, 0)
        pl, ps = bs.ternary_pack(t), bs.ternary_pack_scales(sc)
        bases[name] = torch.from_numpy(np.concatenate([pl, ps.view(np.uint8)])).to(dev), pl.size
        xs[k] = torch.from_numpy(x).to(dev) if k not in xs else xs[k]
        ys[name] = torch.empty(rows, dtype=torch.int64, device=dev)
        del t
    # every weight set in one allocation, each buffer 4 KiB-aligned
    copies = {name: carve_copies(torch, bases[name][0], n_sets, dev) for name, _, _ in STEP}
    sets = [{name: (copies[name][i][:bases[name][1]],
                    copies[name][i][bases[name][1]:].view(torch.int16)) for name, _, _ in STEP}
            for i in range(n_sets)]

    def step(i):
        s = sets[i % n_sets]
        for name, rows, k in STEP:
            bs.ternary_gemv(s[name][0], s[name][1], xs[k], rows, k, out=ys[name],
                            stream=H.stream)

    with torch.cuda.stream(H.stream):
        for i in range(warmup):
            step(n_sets - 1 - (i % n_sets))
    torch.cuda.synchronize()
    H.marker("step")
    g = H.graph(step, steps)
    H.replay_us(g)                              # first replay uploads the graph
    us, wall_us = H.replay_us(g, scrub=True)
    del g
    distinct = min(steps, n_sets) * step_bytes
    value = step_bytes * steps / (us * 1e-6) / 1e9
    log("step (%d launches): %.2f us (events), %.2f us (host wall) -> %.1f GB/s" % (
        len(STEP), us / steps, wall_us / steps, value))
    cfg = {"workload": "per-configuration ternary GEMVs with K in [2560, 5120], batch 1, one "
                       "bs_ternary_gemv launch each: BitNet-b1.58-2B decode projections q, k, v, "
                       "o (2560/640/640/2560 x 2560), gate, up (6912 x 2560) and the larger-K "
                       "11008 x 4096 and 13824 x 5120; P(0) = 0.4, int16 scales U[1, 4096], "
                       "int8 activations rint(N(0, 32^2)), seed 0",
           "launches": {name: "%dx%d" % (r, k) for name, r, k in STEP},
           "weight_bytes_per_step": step_bytes, "weight_sets_in_pool": n_sets,
           "pool_bytes": step_bytes * n_sets, "parallelism": "single GPU",
           "frac_hbm_peak_whole_job": round(value / HBM_PEAK_GBS, 4),
           "host_wall_us_per_step": round(wall_us / steps, 3),
           "timed_region_distinct_bytes": distinct,
           "timed_region_reuse": ("none: %d steps on %d distinct weight sets" % (steps, n_sets)
                                  if steps <= n_sets else
                                  "each weight set re-read after %.2f GB of other sets (> the "
                                  "256 MB Infinity Cache)" % ((n_sets - 1) * step_bytes / 1e9)),
           "before_timed_region": "graph upload replay, then a 512 MB read of another buffer "
                                  "(evicts the L2s and the Infinity Cache)"}
    H.concurrent = concurrent_step(torch, bs, H, sets, xs, ys, step_bytes, steps)
    del sets, bases, copies
    torch.cuda.empty_cache()
    return value, us / steps / 1000.0, cfg


def concurrent_step(torch, bs, H, sets, xs, ys, step_bytes, steps, nstreams=4):
    """The headline's eight launches, unfused and unchanged, captured as
    independent graph branches: each step forks onto `nstreams` streams
    (default priority), the launches shared out by weight bytes, and joins
    before the next step.  Not the headline (which orders every launch)."""
    branches = [torch.cuda.Stream(device=H.dev) for _ in range(nstreams)]
    load = [0] * nstreams
    assign = {}
    for name, rows, k in sorted(STEP, key=lambda e: -weight_bytes(e[1], e[2])):
        j = load.index(min(load))
        assign[name] = j
        load[j] += weight_bytes(rows, k)
    n_sets = len(sets)

    def step(i):
        s = sets[i % n_sets]
        fork = torch.cuda.Event()
        fork.record(H.stream)
        joins = []
        for j, b in enumerate(branches):
            b.wait_event(fork)
            with torch.cuda.stream(b):
                for name, rows, k in STEP:
                    if assign[name] == j:
                        bs.ternary_gemv(s[name][0], s[name][1], xs[k], rows, k, out=ys[name],
                                        stream=b)
            e = torch.cuda.Event()
            e.record(b)
            joins.append(e)
        for e in joins:
            H.stream.wait_event(e)

    H.marker("concurrent_step")
    g = H.graph(step, steps)
    H.replay_us(g)                              # upload
    reps = sorted(H.replay_us(g, scrub=True)[0] / steps for _ in range(3))
    del g
    us = reps[1]
    log("concurrent step (%d branches): %.2f us (of %s)" % (nstreams, us, reps))
    return {"us_per_step": round(us, 3), "us_per_step_min_max": [round(reps[0], 3),
                                                                round(reps[2], 3)],
            "GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
            "branches": {name: assign[name] for name, _, _ in STEP},
            "note": "the headline's eight unfused bs_ternary_gemv launches as independent "
                    "graph branches on %d streams, joined after every step; median of three "
                    "replays; not the headline" % nstreams}


def run_shapes(torch, bs, synth, dev, H):
    """Every configuration shape: back-to-back launch time, its read ceiling
    and, for the roofline shape, the roofline entry."""
    out, roof = {}, None
    for rows, k in IN_RANGE + REPORTED:
        bufs, views, x, nb = packed_pool(torch, bs, synth, dev, rows, k, SHAPE_POOL_BYTES)
        n = len(bufs)
        y = torch.empty(rows, dtype=torch.int64, device=dev)
        wb = weight_bytes(rows, k)
        fn = lambda i: bs.ternary_gemv(views[i % n][0], views[i % n][1], x, rows, k, out=y,
                                       stream=H.stream)
        tag = "%dx%d" % (rows, k)
        us = H.per_launch(fn, n, block="gemv_" + tag)
        ceil_us = H.ceiling(bufs, wb, n)
        e = {"us_per_gemv": round(us, 3), "weight_bytes": wb, "GBps": round(wb / us / 1e3, 1),
             "frac_hbm_peak": round(wb / us / 1e3 / HBM_PEAK_GBS, 4),
             "ceiling_us": round(ceil_us, 3), "frac_of_ceiling": round(ceil_us / us, 3),
             "k_in_2560_5120": 2560 <= k <= 5120, "pool_bytes": n * nb}
        out["ternary_gemv_" + tag] = e
        log("ternary %s: %.3f us (read ceiling %.3f us, %.0f%%)" % (tag, us, ceil_us,
                                                                  100.0 * ceil_us / us))
        if (rows, k) == ROOF_SHAPE:
            us_r = H.per_launch(fn, n, block="roofline_graph")
            achieved = wb / us_r / 1e3
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": _recorded_traffic(tag),
                    "kernel": "bs_ternary_gemv %s (ternary_pipe_kernel)" % tag,
                    "bytes_per_launch": wb, "us_per_launch": round(us_r, 3),
                    "ceiling_us": round(ceil_us, 3), "frac_of_ceiling": round(ceil_us / us_r, 3),
                    "timing": "HIP events on the launch stream around a graph of %d back-to-"
                              "back launches, one per buffer of a %d MB pool; median of 3 "
                              "replays" % (n, n * nb >> 20)}
            log("roofline %s: %.3f us per launch" % (tag, us_r))
        del bufs, views
        torch.cuda.empty_cache()
    return out, roof


def run_f1(torch, bs, synth, dev, H):
    """f1: the activation-reuse sweep, the LNS8 Phase B sweeps and the
    fused four-launch layer step."""
    import numpy as np
    out = {}
    # reuse sweep at K = 4096 (the LNS8 workload's K): N rows share one x
    K = 4096
    sweep = {"ternary": {}, "direct": {}, "popcount": {}, "matrix": {}}
    for n_rows in (1, 8, 32, 128, 512, 2048, 8192):
        bufs, views, x, nb = packed_pool(torch, bs, synth, dev, n_rows, K, SHAPE_POOL_BYTES,
                                         max_copies=1024)
        y = torch.empty(n_rows, dtype=torch.int64, device=dev)
        n = len(bufs)
        us = H.per_launch(lambda i: bs.ternary_gemv(views[i % n][0], views[i % n][1], x, n_rows,
                                                    K, out=y, stream=H.stream), n,
                          block="f1_reuse_ternary_n%d" % n_rows)
        sweep["ternary"][str(n_rows)] = {"us": round(us, 3),
                                         "weights_per_ns": round(n_rows * K / us / 1e3, 2)}
        del bufs, views
        t8, x8 = synth.lns8(n_rows, K, 0)
        p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
        pool = [p8.clone() for _ in range(min(1024, max(2, -(-SHAPE_POOL_BYTES // p8.numel()))))]
        xd = torch.from_numpy(x8).to(dev)
        acc = torch.empty((n_rows, 8), dtype=torch.int32, device=dev)
        s8 = torch.empty(n_rows, dtype=torch.float64, device=dev)
        ws = torch.zeros(bs.lib().bs_lns8_workspace_bytes(n_rows, K), dtype=torch.uint8,
                         device=dev)
        for path, name in LNS8_PATHS:
            us = H.per_launch(lambda i: bs.lns8_phase_gemv(pool[i % len(pool)], xd, n_rows, K,
                                                           path, acc=acc, s=s8, workspace=ws,
                                                           stream=H.stream), len(pool),
                              block="f1_reuse_%s_n%d" % (name, n_rows))
            sweep[name][str(n_rows)] = {"us": round(us, 3),
                                        "weights_per_ns": round(n_rows * K / us / 1e3, 2)}
        del pool
        torch.cuda.empty_cache()
    def crossover(a, b):
        for n_rows in (1, 8, 32, 128, 512, 2048, 8192):
            if sweep[a][str(n_rows)]["us"] <= sweep[b][str(n_rows)]["us"]:
                return n_rows
        return None

    cross = crossover("popcount", "direct")
    out["reuse_sweep_k4096"] = {**sweep, "crossover_rows": cross,
                                "crossover_note": "smallest row count (of those swept) where the "
                                                  "popcount path is at least as fast as direct "
                                                  "routing; null if it never is",
                                "matrix_crossover_rows": crossover("matrix", "popcount"),
                                "matrix_crossover_note": "smallest row count where the matrix "
                                                         "path is at least as fast as popcount"}
    log("f1 reuse sweep: crossover at %s rows" % cross)
    # Phase B: weight zero density and the number of distinct codes, 4096 x 4096
    R = 4096
    phase_b = {"zero_density": {}, "distinct_codes": {}}
    for kind, values in (("zero_density", (0.0, 1.0 / 3.0, 0.6, 0.9)),
                         ("distinct_codes", (1, 8, 41, 127))):
        for v in values:
            if kind == "zero_density":
                t8, x8 = synth.lns8_sweep(R, K, 0, v, 41)
                label = {0.0: "0", 0.6: "0.6", 0.9: "0.9"}.get(v, "1/3")
            else:
                t8, x8 = synth.lns8_sweep(R, K, 0, 1.0 / 3.0, v)
                label = str(v)
            p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
            pool = [p8.clone() for _ in range(-(-SHAPE_POOL_BYTES // p8.numel()))]
            xd = torch.from_numpy(x8).to(dev)
            acc = torch.empty((R, 8), dtype=torch.int32, device=dev)
            ws = torch.zeros(bs.lib().bs_lns8_workspace_bytes(R, K), dtype=torch.uint8,
                             device=dev)
            ent = {}
            for path, name in LNS8_PATHS:
                blk = ("f1_zero_%s_%s" % (name, label) if kind == "zero_density"
                       else "f1_codes_%s_%d" % (name, v))
                us = H.per_launch(lambda i: bs.lns8_phase_gemv(pool[i % len(pool)], xd, R, K,
                                                               path, acc=acc, s=False,
                                                               workspace=ws, stream=H.stream),
                                  len(pool), block=blk)
                ent[name + "_us"] = round(us, 3)
            phase_b[kind][label] = ent
            del pool
            torch.cuda.empty_cache()
    # Phase B over K: 4096 rows, K from 1024 to 32768 (the C4 distributions)
    ksweep = {}
    for kk in (1024, 2048, 4096, 8192, 16384, 32768):
        t8, x8 = synth.lns8(R, kk, 0)
        p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
        pool = [p8.clone() for _ in range(-(-SHAPE_POOL_BYTES // p8.numel()))]
        xd = torch.from_numpy(x8).to(dev)
        acc = torch.empty((R, 8), dtype=torch.int32, device=dev)
        ws = torch.zeros(bs.lib().bs_lns8_workspace_bytes(R, kk), dtype=torch.uint8, device=dev)
        ent = {}
        for path, name in LNS8_PATHS:
            us = H.per_launch(lambda i: bs.lns8_phase_gemv(pool[i % len(pool)], xd, R, kk, path,
                                                           acc=acc, s=False, workspace=ws,
                                                           stream=H.stream),
                              len(pool), block="f1_k_%s_%d" % (name, kk))
            ent[name + "_us"] = round(us, 3)
            ent[name + "_weights_per_ns"] = round(R * kk / us / 1e3, 1)
        ksweep[str(kk)] = ent
        del pool
        torch.cuda.empty_cache()
    phase_b["k_rows4096"] = ksweep
    out["lns8_phase_b_4096x4096"] = phase_b
    # shared-activation fusion: the layer as four launches (q|k|v and gate|up
    # stored concatenated by rows; o and down add into the residual stream)
    shape = {name: (r, k) for name, r, k in LAYER}
    lbytes = sum(weight_bytes(r, k) for _, r, k in LAYER)
    n_layers = -(-STEP_POOL_BYTES // lbytes)
    base = {}
    for fname, members in FUSED:
        parts = [synth.ternary(*shape[m], li) for li, m in enumerate(members)]
        t = np.concatenate([pt[0] for pt in parts])
        sc = np.concatenate([pt[1] for pt in parts])
        k = shape[members[0]][1]
        base[fname] = (torch.from_numpy(bs.ternary_pack(t)).to(dev),
                       torch.from_numpy(bs.ternary_pack_scales(sc)).to(dev),
                       torch.from_numpy(parts[0][2]).to(dev), t.shape[0], k)
    layers = [{f: (base[f][0].clone(), base[f][1].clone()) for f, _ in FUSED}
              for _ in range(n_layers)]
    ys = {f: torch.zeros(base[f][3], dtype=torch.int64, device=dev) for f, _ in FUSED}

    def fused_step(i):
        for fname, _ in FUSED:
            p, s = layers[i % n_layers][fname]
            _, _, x, r, k = base[fname]
            if fname in RESIDUAL:
                bs.ternary_gemv_acc(p, s, x, r, k, ys[fname], stream=H.stream)
            else:
                bs.ternary_gemv(p, s, x, r, k, out=ys[fname], stream=H.stream)

    us = H.per_launch(fused_step, n_layers, block="f1_fused_step")
    out["fused_layer_step"] = {"us_per_step": round(us, 3), "weight_bytes_per_step": lbytes,
                               "GBps": round(lbytes / us / 1e3, 1),
                               "launches": {f: "%dx%d" % (base[f][3], base[f][4])
                                            for f, _ in FUSED},
                               "note": "q|k|v and gate|up stored concatenated (shared "
                                       "activation), o and down as y += W x; not the headline"}
    log("f1 fused layer step: %.2f us" % us)
    del layers, base
    torch.cuda.empty_cache()
    return out


def lns8_counter(key: str):
    """A per-call counter mean from the LNS8 counter record under profiles/
    (None if absent or taken on other source)."""
    fn = os.path.join(ROOT, "profiles", "lns8_4096x4096_valu.txt")
    if not os.path.exists(fn):
        return None
    vals = {}
    for line in open(fn):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            vals[a.strip()] = b.strip()
    if vals.get("kernel_source_sha256_16") != _source_digest("lns8_phase.hip"):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def lns8_valu_ops(path: int) -> float:
    """VALU instructions per launch of the LNS8 kernel at 4096 x 4096, from
    the SQ_INSTS_VALU counter runs recorded under profiles/ (None if absent
    or taken on other source)."""
    fn = os.path.join(ROOT, "profiles", "lns8_4096x4096_valu.txt")
    if not os.path.exists(fn):
        return None
    vals = {}
    for line in open(fn):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            vals[a.strip()] = b.strip()
    if vals.get("kernel_source_sha256_16") != _source_digest("lns8_phase.hip"):
        return None
    key = "valu_insts_per_call_" + dict(LNS8_PATHS_BY_ID)[path]
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def flns_valu_ops(small: bool) -> float:
    """VALU instructions per call of the pure fractional-LNS kernel at 4096 x
    4096 (LDS tables, f <= 8: the mean of the f = 0 and f = 8 calls; device
    tables: f = 12), from the SQ counter record under profiles/ (None if
    absent or taken on other source)."""
    fn = os.path.join(ROOT, "profiles", "flns_4096x4096_sq_counters.txt")
    if not os.path.exists(fn):
        return None
    want = "flns_rows_kernel<%s>" % ("true" if small else "false")
    digest, valu = None, None
    for line in open(fn):
        if line.startswith("kernel_source_sha256_16:"):
            digest = line.split(":", 1)[1].strip()
        elif want in line and " SQ_INSTS_VALU " in line and " mean " in line:
            valu = float(line.split(" mean ")[1].split()[0])
    if digest != _source_digest("flns_phase.hip"):
        return None
    return valu


def run_extras(torch, bs, synth, dev, H):
    import numpy as np
    ops = {}
    # Q1_0 (one sign bit per weight)
    q1_bytes = lambda r, k: r * k // 8 + r * (k // 128) * 2
    H.marker("q1")
    for rows, k in [(2560, 2560), (13824, 2560), (2560, 6912), (13824, 5120)]:
        sgn, sc, x = synth.q1(rows, k, 0)
        b = torch.from_numpy(bs.q1_pack(sgn)).to(dev)
        s = torch.from_numpy(bs.ternary_pack_scales(sc)).to(dev)
        n = max(2, -(-SHAPE_POOL_BYTES // q1_bytes(rows, k)))
        bp, sp = [b.clone() for _ in range(n)], [s.clone() for _ in range(n)]
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty(rows, dtype=torch.int64, device=dev)
        us = H.per_launch(lambda i: bs.q1_gemv(bp[i % n], sp[i % n], xd, rows, k, out=y,
                                               stream=H.stream), n)
        wb = q1_bytes(rows, k)
        ops["q1_gemv_%dx%d" % (rows, k)] = {
            "us_per_gemv": round(us, 3), "weight_bytes": wb, "GBps": round(wb / us / 1e3, 1),
            "frac_hbm_peak": round(wb / us / 1e3 / HBM_PEAK_GBS, 4)}
        del bp, sp
        log("q1 %dx%d: %.2f us" % (rows, k, us))
    # LNS8 eight-phase GEMV, 4096 x 4096
    t8, x8 = synth.lns8(4096, 4096, 0)
    p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
    pool8 = [p8.clone() for _ in range(-(-SHAPE_POOL_BYTES // p8.numel()))]
    xd8 = torch.from_numpy(x8).to(dev)
    acc = torch.empty((4096, 8), dtype=torch.int32, device=dev)
    s8 = torch.empty(4096, dtype=torch.float64, device=dev)
    ws8 = torch.zeros(bs.lib().bs_lns8_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    H.marker("lns8")
    for path, name in LNS8_PATHS:
        us = H.per_launch(lambda i: bs.lns8_phase_gemv(pool8[i % len(pool8)], xd8, 4096, 4096,
                                                       path, acc=acc, s=s8, workspace=ws8,
                                                       stream=H.stream), len(pool8))
        ent = {"us_per_gemv": round(us, 3), "weight_bytes": p8.numel(),
               "GBps": round(p8.numel() / us / 1e3, 1),
               "frac_hbm_peak": round(p8.numel() / us / 1e3 / HBM_PEAK_GBS, 4),
               "weights_per_s": round(4096 * 4096 / us * 1e6, 1)}
        valu = lns8_valu_ops(path)
        if valu is not None:
            ent["valu_insts_per_call"] = valu
            ent["valu_lane_ops_per_weight"] = round(valu * 64 / (4096 * 4096), 3)
            ent["frac_valu_peak"] = round(valu * 64 / (us * 1e-6) / VALU_PEAK_OPS, 4)
        if name == "matrix":
            # the contraction: 4096 rows x 4096 positions x 16 columns, a
            # multiply and an add each, on the int8 matrix instructions
            mops = 4096 * 4096 * 16 * 2
            ent["mfma_int8_ops_per_call"] = mops
            ent["frac_mfma_int8_peak"] = round(mops / (us * 1e-6) / MFMA_I8_PEAK_OPS, 4)
            for key, out in (("sq_insts_valu_mfma_i8_per_call_matrix", "mfma_i8_insts_per_call"),
                             ("sq_valu_mfma_busy_cycles_per_call_matrix",
                              "mfma_busy_simd_cycles_per_call")):
                v = lns8_counter(key)
                if v is not None:
                    ent[out] = v
            busy = lns8_counter("sq_valu_mfma_busy_cycles_per_call_matrix")
            if busy is not None:
                # MFMA-busy SIMD-cycles against every SIMD over the timed call
                # at 2.4 GHz (the profiler's own busy-cycle count per dispatch
                # includes its serialisation, so the event time is used)
                ent["frac_simd_cycles_mfma_busy"] = round(busy / (SIMDS * us * 1e-6 * 2.4e9), 4)
        ops["lns8_4096x4096_" + name] = ent
        log("lns8 %s: %.2f us" % (name, us))
    # pure fractional-LNS reduction of the same products, by internal
    # precision: time per call and the error of the decoded result against
    # the exact dyadic S of the linear path
    s_exact = s8.clone()
    bs.lns8_phase_gemv(p8, xd8, 4096, 4096, bs.LNS8_DIRECT, acc=acc, s=s_exact, workspace=ws8,
                       stream=H.stream)
    torch.cuda.synchronize()
    s_ref = s_exact.cpu().numpy()
    wsf = torch.zeros(bs.lib().bs_flns_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    outf = torch.empty((4096, 2), dtype=torch.int32, device=dev)
    flns = {}
    H.marker("flns")
    for f in (0, 2, 4, 8, 12):
        tb = torch.from_numpy(bs.flns_table(f)).to(dev)
        us = H.per_launch(lambda i: bs.flns_phase_gemv(pool8[i % len(pool8)], xd8, 4096, 4096, f,
                                                       tb, out=outf, workspace=wsf,
                                                       stream=H.stream), 50)
        bs.flns_phase_gemv(p8, xd8, 4096, 4096, f, tb, out=outf, workspace=wsf, stream=H.stream)
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
        valu = flns_valu_ops(f <= 8)
        if valu is not None:
            flns["f%d" % f]["valu_insts_per_call"] = valu
            flns["f%d" % f]["frac_valu_peak"] = round(valu * 64 / (us * 1e-6) / VALU_PEAK_OPS, 4)
        log("flns f=%d: %.2f us, median rel err %.3g" % (f, us, np.median(rel)))
    ops["flns_4096x4096"] = {"error_vs": "exact dyadic S of the linear eight-phase path "
                                         "(rows with |S| >= 1e-3 x median |S|)", **flns}
    del pool8
    # steps either side of the GEMVs
    rng = np.random.default_rng(0)
    H.marker("edges")
    for k in (2560, 6912):
        xq = torch.from_numpy(rng.integers(-(1 << 40), 1 << 40, k).astype(np.int64)).to(dev)
        qo = torch.empty(k, dtype=torch.int8, device=dev)
        am = torch.empty(1, dtype=torch.int64, device=dev)
        stq = torch.empty(1, dtype=torch.int32, device=dev)
        us = H.per_launch(lambda i: bs.act_quant_i8(xq, q=qo, absmax=am, status=stq,
                                                    stream=H.stream), 100)
        ops["act_quant_i8_k%d" % k] = {"us_per_call": round(us, 3)}
    xe = torch.from_numpy((rng.standard_normal(4096) * 2.0 ** 20).astype(np.int64)).to(dev)
    eo = torch.empty(4096, dtype=torch.uint8, device=dev)
    ops["lns8_encode_k4096"] = {"us_per_call": round(H.per_launch(
        lambda i: bs.lns8_encode(xe, 16, out=eo, stream=H.stream), 100), 3)}
    ci = torch.from_numpy(rng.permutation(128256)[:40].astype(np.int32)).to(dev)
    cs = torch.from_numpy(np.sort(rng.integers(0, 1 << 30, 40))[::-1].copy()).to(dev)
    res = torch.empty(6, dtype=torch.int64, device=dev)
    ops["sample_candidates_n40"] = {"us_per_call": round(H.per_launch(
        lambda i: bs.sample_candidates(ci, cs, bs.SAMPLE_DRAW, beta_q16=1 << 10, seed=1,
                                       position=i, result=res, stream=H.stream), 100), 3)}
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
    info = torch.empty(3, dtype=torch.int32, device=dev)
    wsl = torch.zeros(bs.lib().bs_lmhead_workspace_bytes(V, K, 40, 200), dtype=torch.uint8,
                      device=dev)
    us = H.per_launch(lambda i: bs.lmhead_planes_topk(
        pool03[i % 4], d47, drs, dh, V, K, 40, 200, top_idx=idx, top_score=sc, info=info,
        workspace=wsl, stream=H.stream), 20, block="lmhead")
    stage1_bytes = p03.size + rs.nbytes
    torch.cuda.synchronize()
    # the read ceiling of stage 1's planes 0-3 bytes over the same pool
    ceil_us = H.ceiling(pool03, p03.size, 4, block="lmhead_ceiling")
    ops["lmhead_planes_topk_128256x2560"] = {
        "us_per_call": round(us, 3), "stage1_bytes": stage1_bytes,
        "GBps_stage1_bytes": round(stage1_bytes / us / 1e3, 1),
        "frac_hbm_peak": round(stage1_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
        "planes03_read_ceiling_us": round(ceil_us, 3),
        "n_candidates": int(info[0].item()), "capped": int(info[1].item()),
        "certified_exact": int(info[2].item())}
    log("lm_head: %.2f us" % us)
    del pool03
    torch.cuda.empty_cache()
    return ops


def context(torch, H):
    """The empty-kernel floor (back-to-back launches of a kernel that does
    nothing, at two grid sizes) and the streaming-read ceiling of the GPU: a
    plain read of 1 GiB (four times the Infinity Cache) by a fixed grid."""
    out = {}
    for blocks, threads in ((256, 256), (1024, 1024)):
        out["launch_floor_us_%dx%d" % (blocks, threads)] = round(H.per_launch(
            lambda i: H.probe.empty(blocks, threads, H.stream), 200, block="context_floor"), 3)
    nbytes = 1 << 30
    big = torch.empty(nbytes, dtype=torch.uint8, device=H.dev)
    sink = torch.empty(8192 * 256, dtype=torch.int64, device=H.dev)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        us = H.per_launch(lambda i: H.probe.read_strided(big, nbytes, blocks, sink, H.stream), 4,
                          block="context_stream")
        best = us if best is None else min(best, us)
    out["stream_read_1GiB_us"] = round(best, 2)
    out["stream_read_1GiB_GBps"] = round(nbytes / best / 1e3, 1)
    out["stream_read_1GiB_frac_hbm_peak"] = round(nbytes / best / 1e3 / HBM_PEAK_GBS, 4)
    del big, sink
    return out


# ------------------------------------------------------- profile summaries

def trace_summary(path: str):
    """Per-block kernel durations from a rocprofv3 --kernel-trace CSV of this
    script: dispatches are assigned to the block named by the last marker
    launch before them (an empty kernel of (4096 + id) x 64 threads)."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by_id = {v: k for k, v in MARKER_ID.items()}
    block = "setup"
    groups = {}
    for r in rows:
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
        grid, wg = int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"])
        if "empty_kernel" in name and wg == 64 and grid % 64 == 0 and grid // 64 > MARKER_BASE:
            block = by_id.get(grid // 64 - MARKER_BASE, "marker?")
            continue
        key = (block, name, grid, wg)
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = []
    for (block, name, grid, wg), d in groups.items():
        out.append("%-28s %-58s grid %8d wg %4d calls %6d avg %8.3f us median %8.3f us "
                   "min %8.3f us" % (block[:28], name[:58], grid, wg, len(d),
                                     statistics.mean(d) / 1e3, statistics.median(d) / 1e3,
                                     min(d) / 1e3))
    return "\n".join(out)


CALIB_BYTES = 256 << 20         # the calibration kernel reads and writes this many bytes


def traffic_run(shape: str, launches: int = 20):
    """Workload for the rocprofv3 --pmc runs behind roofline.traffic: three
    launches of a plain elementwise kernel of known size (int32 negation,
    CALIB_BYTES read and CALIB_BYTES written: the counter calibration), then
    `launches` launches of the ternary GEMV of `shape` on distinct weight
    buffers (> 1 GiB in total, so they stream from HBM), then as many plain
    reads of the same bytes from other buffers of the pool (the read-ceiling
    kernel, four 16-byte loads per thread), for counters side by side."""
    import torch
    import bit_decode_gemv_amd as bs
    from bit_decode_gemv_amd import synth
    rows, k = (int(v) for v in shape.split("x"))
    dev = torch.device("cuda:0")
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    from bit_decode_gemv_amd import probe
    bufs, views, x, _ = packed_pool(torch, bs, synth, dev, rows, k, 1 << 30)
    y = torch.empty(rows, dtype=torch.int64, device=dev)
    wb = weight_bytes(rows, k)
    sink = probe.sink_for(wb, 4, dev)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    for i in range(launches):
        bs.ternary_gemv(views[i % len(views)][0], views[i % len(views)][1], x, rows, k, out=y)
    torch.cuda.synchronize()
    for i in range(launches):
        probe.read(bufs[(launches + i) % len(bufs)], wb, 4, sink, torch.cuda.current_stream())
    torch.cuda.synchronize()
    log("traffic run done: 3 calibration launches, %d GEMV launches of %s, %d reads of its "
        "weight bytes" % (launches, shape, launches))


def lns8_counter_run(launches: int = 10):
    """Workload for the rocprofv3 --pmc runs behind the LNS8 VALU fraction:
    `launches` calls of each LNS8 path (direct, popcount, matrix) at 4096 x
    4096 on distinct weight buffers."""
    import torch
    import bit_decode_gemv_amd as bs
    from bit_decode_gemv_amd import synth
    dev = torch.device("cuda:0")
    t8, x8 = synth.lns8(4096, 4096, 0)
    p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
    pool = [p8.clone() for _ in range(launches)]
    xd = torch.from_numpy(x8).to(dev)
    for path, _ in LNS8_PATHS:
        for i in range(launches):
            bs.lns8_phase_gemv(pool[i], xd, 4096, 4096, path)
        torch.cuda.synchronize()
    log("LNS8 counter run done: %d calls per path" % launches)


def flns_counter_run(launches: int = 10):
    """Workload for the rocprofv3 --pmc runs of the pure fractional-LNS
    kernel: `launches` calls at 4096 x 4096 for each of f = 0 and f = 8 (LDS
    tables) and f = 12 (device tables), on distinct weight buffers."""
    import torch
    import bit_decode_gemv_amd as bs
    from bit_decode_gemv_amd import synth
    dev = torch.device("cuda:0")
    t8, x8 = synth.lns8(4096, 4096, 0)
    p8 = torch.from_numpy(bs.ternary_pack(t8)).to(dev)
    pool = [p8.clone() for _ in range(launches)]
    xd = torch.from_numpy(x8).to(dev)
    ws = torch.zeros(bs.lib().bs_flns_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    out = torch.empty((4096, 2), dtype=torch.int32, device=dev)
    for f in (0, 8, 12):
        tb = torch.from_numpy(bs.flns_table(f)).to(dev)
        for i in range(launches):
            bs.flns_phase_gemv(pool[i], xd, 4096, 4096, f, tb, out=out, workspace=ws)
        torch.cuda.synchronize()
    log("pure-LNS counter run done: %d calls at each of f = 0, 8, 12" % launches)


SIMDS = 1024                    # 256 CUs x 4 SIMDs


def counter_summary(*paths: str):
    """Mean of every counter per kernel name (template arguments kept) over
    one or more rocprofv3 --pmc counter_collection.csv files: one line per
    (kernel, counter), then per kernel the ratios these counters give."""
    vals = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            vals.setdefault((name, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    out = ["%-60s %-28s dispatches %4d mean %.6g" % (n[:60], c, len(v), statistics.mean(v))
           for (n, c), v in sorted(vals.items())]
    means = {}
    for (n, c), v in vals.items():
        means.setdefault(n, {})[c] = statistics.mean(v)
    for n, m in sorted(means.items()):
        d = []
        if "SQ_WAVES" in m:
            d.append("waves_per_simd %.3f" % (m["SQ_WAVES"] / SIMDS))
            if "SQ_INSTS_VALU" in m:
                d.append("valu_insts_per_wave %.1f" % (m["SQ_INSTS_VALU"] / m["SQ_WAVES"]))
            if "SQ_INSTS_VMEM_RD" in m:
                d.append("vmem_rd_insts_per_wave %.1f" % (m["SQ_INSTS_VMEM_RD"] / m["SQ_WAVES"]))
        if m.get("SQ_WAVE_CYCLES"):
            for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU"):
                if c in m:
                    d.append("%s_per_wave_cycle %.3f" % (c.lower(), m[c] / m["SQ_WAVE_CYCLES"]))
        if m.get("TCP_TCC_READ_REQ_sum"):
            if "TCP_TCC_READ_REQ_LATENCY_sum" in m:
                d.append("l2_read_latency_cycles %.1f" % (m["TCP_TCC_READ_REQ_LATENCY_sum"] /
                                                         m["TCP_TCC_READ_REQ_sum"]))
        if d:
            out.append("%-60s derived: %s" % (n[:60], ", ".join(d)))
    return "\n".join(out)


def lns8_valu_summary(*paths: str):
    """The LNS8 counter record: every counter's mean per call of each path
    (lns8_kernel = direct routing, lns8_pc_kernel = popcount histogram,
    lns8_mx_kernel = the matrix contraction) from one or more --pmc CSVs of
    --lns8-counter-run, keyed to the kernel source it was taken on."""
    vals = {}
    rows = [r for path in paths for r in csv.DictReader(open(path))]
    for r in rows:
        name = r["Kernel_Name"]
        if "lns8_pc_kernel" in name:
            p = "popcount"
        elif "lns8_mx_kernel" in name:
            p = "matrix"
        elif "lns8_kernel" in name:
            p = "direct"
        else:
            continue
        vals.setdefault((r["Counter_Name"], p), []).append(float(r["Counter_Value"]))
    lines = ["kernel_source_sha256_16: %s" % _source_digest("lns8_phase.hip")]
    for (c, p), v in sorted(vals.items()):
        key = "valu_insts" if c == "SQ_INSTS_VALU" else c.lower()
        lines.append("%s_per_call_%s: %.1f" % (key, p, statistics.mean(v)))
        lines.append("%s_calls_%s: %d" % (key, p, len(v)))
    return "\n".join(lines)


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
            if "ternary_" in name and "_kernel" in name:
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true", help="skip the non-headline workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time of each of the two all-step baseline legs")
    ap.add_argument("--trace-summary", help="summarise a rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--traffic-run", metavar="NxK",
                    help="run the workload of the --pmc traffic measurement and exit")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "NxK"),
                    help="HBM bytes per launch from the two counter CSVs and exit")
    ap.add_argument("--lns8-counter-run", action="store_true",
                    help="run the workload of the LNS8 --pmc runs and exit")
    ap.add_argument("--flns-counter-run", action="store_true",
                    help="run the workload of the pure-LNS --pmc runs and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="mean counters per kernel of --pmc CSVs, with their ratios, and exit")
    ap.add_argument("--lns8-valu-summary", metavar="CSV", nargs="+",
                    help="the LNS8 counter record from a --pmc CSV of --lns8-counter-run, and exit")
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
    if args.lns8_counter_run:
        lns8_counter_run()
        return 0
    if args.flns_counter_run:
        flns_counter_run()
        return 0
    if args.counter_summary:
        print(counter_summary(*args.counter_summary))
        return 0
    if args.lns8_valu_summary:
        print(lns8_valu_summary(*args.lns8_valu_summary))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the GEMVs would "
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
    H = Harness(torch, dev)
    value, ms_per_step, cfg = run_step(torch, bs, synth, dev, H, args.steps, args.warmup)
    gemv, roofline = run_shapes(torch, bs, synth, dev, H)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int64",
        "data": "synthetic", "config": cfg, "roofline": roofline,
        "ops": {"gemv": gemv},
    }
    out["context"] = context(torch, H)
    if not args.no_extras:
        out["ops"]["f1"] = run_f1(torch, bs, synth, dev, H)
        out["ops"]["f1"]["concurrent_step"] = H.concurrent
        out["ops"].update(run_extras(torch, bs, synth, dev, H))
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (~%.0f s)" % (2.5 * args.cpu_seconds))
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
