"""The oracle and the library's host-only code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Two drivers in tests/sanitize/ call every oracle function and every host-only
entry point (layout, loss-scale decision, accounting, sharded checkpoints) on
heap buffers of exactly the sizes the calls may touch; a third runs the
launchers' plan that cuts a long shard into consecutive launches (launch.h).  They are built with
gcc/g++ and the sanitizers, so a read or write past an end, a use after free,
a leak or undefined arithmetic aborts the run; the drivers also check the
documented results and error codes.  The kernels' host wrappers (api.cpp)
link the HIP runtime and are exercised through the library instead.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "zero_sharded_mixed_shard_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _build(compiler, args, exe):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    r = subprocess.run([compiler, *SAN, *args, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]


def _run(cmd):
    r = subprocess.run([str(c) for c in cmd], capture_output=True, text=True, timeout=600,
                       env=ENV)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), \
        (r.returncode, r.stdout[-2000:], r.stderr[-6000:])


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    _build("gcc", ["-std=c11", "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
                   os.path.join(HERE, "oracle_driver.c"), "-lm"], exe)
    _run([exe])


def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_driver"
    srcs = [os.path.join(CSRC, f) for f in ("layout.cpp", "scaler.cpp", "accounting.cpp",
                                            "checkpoint.cpp")]
    _build("g++", ["-std=c++17", "-I", os.path.join(ROOT, "include"), *srcs,
                   os.path.join(HERE, "host_driver.cpp")], exe)
    scratch = tmp_path / "files"
    scratch.mkdir()
    _run([exe, scratch])


def test_launch_plan_under_sanitizers(tmp_path):
    # by_pieces / piece_tiles from launch.h, host-only code that needs the HIP
    # headers for its types but no GPU and no HIP runtime
    inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(inc, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not found")
    exe = tmp_path / "launch_plan_driver"
    _build("g++", ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I",
                   os.path.join(ROOT, "include"), "-I", CSRC,
                   os.path.join(HERE, "launch_plan_driver.cpp")], exe)
    _run([exe])
