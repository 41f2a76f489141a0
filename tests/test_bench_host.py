"""Host-side checks of bench.py's contract paths that need no GPU: the
one-GPU rule, and the parsers behind the profiles/ summaries (kernel trace
and --pmc traffic), fed small synthetic CSV files."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_summary(tmp_path):
    """Dispatches are split per measured block by the marker launches (empty
    kernels of (4096 + block id) x 64 threads) that precede them."""
    p = tmp_path / "kernel_trace.csv"
    fields = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    gemv = "void bs::(anonymous namespace)::ternary_pipe_kernel<16, 3, 2, 2>(x)"

    def marker(block, t):
        mid = bench.MARKER_ID[block]
        return {"Kernel_Name": "(anonymous namespace)::empty_kernel()",
                "Grid_Size_X": (bench.MARKER_BASE + mid) * 64, "Workgroup_Size_X": 64,
                "Start_Timestamp": t, "End_Timestamp": t + 100}

    rows = [marker("gemv_2560x2560", 0)]
    rows += [{"Kernel_Name": gemv, "Grid_Size_X": 30720, "Workgroup_Size_X": 192,
              "Start_Timestamp": 1000 * (i + 1), "End_Timestamp": 1000 * (i + 1) + d}
             for i, d in enumerate([3000, 4000, 5000])]
    rows += [marker("gemv_640x2560", 10000)]
    rows += [{"Kernel_Name": gemv, "Grid_Size_X": 30720, "Workgroup_Size_X": 192,
              "Start_Timestamp": 20000, "End_Timestamp": 22000}]
    _write(p, fields, list(reversed(rows)))            # order restored by start time
    out = bench.trace_summary(str(p)).splitlines()
    assert len(out) == 2
    a = [line for line in out if line.startswith("gemv_2560x2560")][0]
    b = [line for line in out if line.startswith("gemv_640x2560")][0]
    assert "void bs::ternary_pipe_kernel<16, 3, 2, 2>" in a
    assert "calls      3" in a and "avg    4.000 us" in a and "min    3.000 us" in a
    assert "calls      1" in b and "avg    2.000 us" in b


def test_marker_ids_are_distinct_and_small():
    ids = list(bench.MARKER_ID.values())
    assert len(set(ids)) == len(ids) and min(ids) >= 1 and max(ids) < 1024


def test_traffic_summary(tmp_path):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    calib = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    gemv = "void bs::(anonymous namespace)::ternary_pipe_kernel<16, 3, 2, 2>(args)"
    half = bench.CALIB_BYTES / 1024 / 2          # FETCH_SIZE reads half the known bytes
    _write(tmp_path / "f.csv", fields,
           [{"Kernel_Name": calib, "Counter_Name": "FETCH_SIZE", "Counter_Value": half}] * 3 +
           [{"Kernel_Name": gemv, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0}] * 4)
    _write(tmp_path / "w.csv", fields,
           [{"Kernel_Name": calib, "Counter_Name": "WRITE_SIZE",
             "Counter_Value": bench.CALIB_BYTES / 1024}] * 3 +
           [{"Kernel_Name": gemv, "Counter_Name": "WRITE_SIZE", "Counter_Value": 20.0}] * 4)
    out = bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "640x2560")
    vals = dict(line.split(": ", 1) for line in out.splitlines())
    assert float(vals["fetch_bytes_per_launch"]) == pytest.approx(2 * 1000 * 1024)
    assert float(vals["write_bytes_per_launch"]) == pytest.approx(20 * 1024)
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx(2 * 1000 * 1024 + 20 * 1024)
    assert vals["kernel_source_sha256_16"] == bench._source_digest()


def test_source_digest_covers_included_headers(tmp_path, monkeypatch):
    """The recorded HBM traffic is dropped once the GEMV kernel changes; a
    change to a header the kernel includes is such a change."""
    import shutil
    for rel in (("bit_decode_gemv_amd", "csrc", "ternary_gemv.hip"),
                ("bit_decode_gemv_amd", "csrc", "kcommon.h"),
                ("bit_decode_gemv_amd", "csrc", "bs_internal.h"),
                ("include", "bs.h"),
                ("bit_decode_gemv_amd", "build.py")):
        dst = tmp_path.joinpath(*rel)
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, *rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = bench._source_digest()
    with open(tmp_path / "bit_decode_gemv_amd" / "csrc" / "kcommon.h", "a") as f:
        f.write("\n// edit\n")
    assert bench._source_digest() != before
    # so is a change of the compiler flags
    after_header = bench._source_digest()
    with open(tmp_path / "bit_decode_gemv_amd" / "build.py", "a") as f:
        f.write("\n# edit\n")
    assert bench._source_digest() != after_header


def test_lns8_valu_record_round_trip(tmp_path, monkeypatch):
    """The LNS8 counter record written by --lns8-valu-summary is read back by
    the bench, and ignored once the LNS8 kernel source changes."""
    import shutil
    for rel in (("bit_decode_gemv_amd", "csrc", "lns8_phase.hip"),
                ("bit_decode_gemv_amd", "csrc", "kcommon.h"),
                ("bit_decode_gemv_amd", "csrc", "bs_internal.h"),
                ("include", "bs.h"),
                ("bit_decode_gemv_amd", "build.py")):
        dst = tmp_path.joinpath(*rel)
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, *rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for name, v in (("lns8_kernel", 1000.0), ("lns8_pc_kernel", 700.0), ("lns8_mx_kernel", 400.0)):
        for i in range(3):
            rows.append({"Kernel_Name": "void bs::(anonymous namespace)::%s(args)" % name,
                         "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": v + i})
            rows.append({"Kernel_Name": "void bs::(anonymous namespace)::%s(args)" % name,
                         "Counter_Name": "SQ_WAVES", "Counter_Value": 4096})
    rows.append({"Kernel_Name": "void at::native::other", "Counter_Name": "SQ_INSTS_VALU",
                 "Counter_Value": 5.0})
    _write(tmp_path / "c.csv", fields, rows)
    # a second pass (the MFMA counters) merges into the same record
    mfma = [{"Kernel_Name": "void bs::(anonymous namespace)::lns8_mx_kernel(args)",
             "Counter_Name": c, "Counter_Value": v}
            for c, v in (("SQ_INSTS_VALU_MFMA_I8", 16384), ("SQ_VALU_MFMA_BUSY_CYCLES", 262144))]
    _write(tmp_path / "m.csv", fields, mfma)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "lns8_4096x4096_valu.txt").write_text(
        "# header\n" + bench.lns8_valu_summary(str(tmp_path / "c.csv"), str(tmp_path / "m.csv"))
        + "\n")
    assert bench.lns8_valu_ops(0) == pytest.approx(1001.0)
    assert bench.lns8_valu_ops(1) == pytest.approx(701.0)
    assert bench.lns8_valu_ops(2) == pytest.approx(401.0)
    assert bench.lns8_counter("sq_insts_valu_mfma_i8_per_call_matrix") == 16384
    assert bench.lns8_counter("sq_valu_mfma_busy_cycles_per_call_matrix") == 262144
    assert bench.lns8_counter("sq_valu_mfma_busy_cycles_per_call_direct") is None
    with open(tmp_path / "bit_decode_gemv_amd" / "csrc" / "lns8_phase.hip", "a") as f:
        f.write("\n// edit\n")
    assert bench.lns8_valu_ops(0) is None
    assert bench.lns8_counter("sq_insts_valu_mfma_i8_per_call_matrix") is None


def test_marker_blocks_cover_the_sweeps():
    """Every block the benchmark marks has an id: the K sweep of Phase B and
    the concurrent step included."""
    for p in ("direct", "popcount", "matrix"):
        for k in (1024, 2048, 4096, 8192, 16384, 32768):
            assert "f1_k_%s_%d" % (p, k) in bench.MARKER_ID
    assert "concurrent_step" in bench.MARKER_ID


def test_flns_valu_record_round_trip(tmp_path, monkeypatch):
    """The pure-LNS counter record (a --counter-summary of --flns-counter-run
    under a header with the source digest) is read back per table placement
    and ignored once the kernel source changes."""
    import shutil
    for rel in (("bit_decode_gemv_amd", "csrc", "flns_phase.hip"),
                ("bit_decode_gemv_amd", "csrc", "kcommon.h"),
                ("bit_decode_gemv_amd", "csrc", "bs_internal.h"),
                ("include", "bs.h"),
                ("bit_decode_gemv_amd", "build.py")):
        dst = tmp_path.joinpath(*rel)
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, *rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for small, v in (("true", 4000.0), ("false", 5000.0)):
        for i in range(2):
            rows.append({"Kernel_Name": "void bs::(anonymous namespace)::flns_rows_kernel<%s>(a)"
                                        % small,
                         "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": v + 2 * i})
    _write(tmp_path / "c.csv", fields, rows)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "flns_4096x4096_sq_counters.txt").write_text(
        "# header\nkernel_source_sha256_16: %s\n%s\n" % (
            bench._source_digest("flns_phase.hip"), bench.counter_summary(str(tmp_path / "c.csv"))))
    assert bench.flns_valu_ops(True) == pytest.approx(4001.0)
    assert bench.flns_valu_ops(False) == pytest.approx(5001.0)
    with open(tmp_path / "bit_decode_gemv_amd" / "csrc" / "flns_phase.hip", "a") as f:
        f.write("\n// edit\n")
    assert bench.flns_valu_ops(True) is None


def test_counter_summary_ratios(tmp_path):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void bs::(anonymous namespace)::ternary_pipe_kernel<8, 3, 1, 1>(args)"
    _write(tmp_path / "a.csv", fields,
           [{"Kernel_Name": k, "Counter_Name": "SQ_WAVES", "Counter_Value": 2048},
            {"Kernel_Name": k, "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": 204800},
            {"Kernel_Name": k, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": 1000},
            {"Kernel_Name": k, "Counter_Name": "SQ_WAIT_INST_ANY", "Counter_Value": 250}])
    _write(tmp_path / "b.csv", fields,
           [{"Kernel_Name": k, "Counter_Name": "TCP_TCC_READ_REQ_sum", "Counter_Value": 10},
            {"Kernel_Name": k, "Counter_Name": "TCP_TCC_READ_REQ_LATENCY_sum",
             "Counter_Value": 7000}])
    out = bench.counter_summary(str(tmp_path / "a.csv"), str(tmp_path / "b.csv"))
    d = [line for line in out.splitlines() if "derived" in line][0]
    assert "waves_per_simd 2.000" in d and "valu_insts_per_wave 100.0" in d
    assert "sq_wait_inst_any_per_wave_cycle 0.250" in d and "l2_read_latency_cycles 700.0" in d
