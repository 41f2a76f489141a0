"""CPU sanitizer leg: the C oracle (bs_oracle.c, flns_oracle.c) and the
host-only sources of the library (codec.cpp, flns_tables.cpp) are rebuilt by
gcc/g++ with AddressSanitizer and UndefinedBehaviorSanitizer (every UB report
fatal), and a child pytest with libasan preloaded runs every oracle pin and
the host codec / table tests against those builds (tests/conftest.py swaps
them in).  A report from either sanitizer fails the child, hence this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
HOST_TESTS = ("test_ternary_codec_matches_oracle_layout or test_ternary_codec_rejects_invalid "
              "or test_planes_codec_matches_oracle_layout or test_q1_codec_matches_oracle_layout "
              "or test_status_strings or test_table_blob_equals_oracle_tables "
              "or test_table_bytes_and_build_errors")


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc/g++ not found")
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    d = tmp_path_factory.mktemp("san")
    orc = str(d / "liboracle_san.so")
    host = str(d / "libbshost_san.so")
    subprocess.check_call(["gcc", "-std=gnu11", "-fopenmp", "-shared", "-fPIC", *SAN,
                           os.path.join(ROOT, "oracle", "bs_oracle.c"),
                           os.path.join(ROOT, "oracle", "flns_oracle.c"),
                           "-o", orc, "-lquadmath", "-lm"])
    csrc = os.path.join(ROOT, "bit_decode_gemv_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", "-shared", "-fPIC", *SAN,
                           "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           os.path.join(csrc, "codec.cpp"), os.path.join(csrc, "flns_tables.cpp"),
                           "-o", host])
    return asan, orc, host, d


def _child(sanitized, args, tag):
    """Run pytest on `args` over the sanitized builds; the sanitizers write
    their reports to files (pytest's output capture would swallow them when
    a report ends the process)."""
    asan, orc, host, d = sanitized
    logs = d / ("logs_" + tag)
    logs.mkdir()
    env = dict(os.environ)
    # ASan's runtime must come first; whatever the environment preloads stays
    preload = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env.update({"LD_PRELOAD": preload, "BS_SANITIZED_ORACLE": orc, "BS_SANITIZED_HOST": host,
                # the interpreter and its extension modules are not built with
                # ASan: leak reports at exit would be theirs
                "ASAN_OPTIONS": "detect_leaks=0:exitcode=86:log_path=%s/asan" % logs,
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=87:"
                                 "log_path=%s/ubsan" % logs,
                "OMP_NUM_THREADS": "4"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *args], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=1500)
    out = r.stdout + r.stderr
    reports = "".join(open(p).read() for p in sorted(logs.iterdir()))
    assert reports == "", reports[:6000]
    assert r.returncode == 0, "exit %d\n%s" % (r.returncode, out[-6000:])
    return out


def test_oracle_pins_under_asan_ubsan(sanitized):
    out = _child(sanitized, sorted(os.path.join("tests", f) for f in os.listdir(
        os.path.join(ROOT, "tests")) if f.startswith("test_oracle_") and f.endswith(".py")), "oracle")
    assert " passed" in out


def test_host_codec_under_asan_ubsan(sanitized):
    out = _child(sanitized, ["tests/test_abi_host.py", "tests/test_flns_host.py",
                             "-k", HOST_TESTS], "host")
    assert " passed" in out and " deselected" in out
