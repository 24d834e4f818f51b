"""Build libzero_shard.so (the C-ABI library and its gfx950 kernels) in tree.

    python zero_sharded_mixed_shard_amd/build.py

(Run it by path: importing the package would load the library it rebuilds.)

Flags that carry the numerics:
  -ffp-contract=off                 no FMA contraction: one rounding per op
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed FP32 VALU ops are generated
  (default)                         correctly rounded FP32 '/' and sqrt,
                                    denormals preserved; never -ffast-math
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzero_shard.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["layout.cpp", "scaler.cpp", "accounting.cpp", "checkpoint.cpp", "api.cpp",
           "shard_kernels.hip",
           "exchange_kernels.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-ffp-contract=off",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library."""
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            # every source goes through the HIP driver (host files include the runtime API)
            cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            _run(cmd)
            objs.append(obj)
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, *DEVICE, "-shared", "-fPIC", "-o", out_tmp, *objs]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        os.replace(out_tmp, LIB)
    return LIB


def device_assembly(src: str = "shard_kernels.hip") -> str:
    """gfx950 assembly of one source, built with the library's flags."""
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        _run([HIPCC, "-x", "hip", *DEVICE, *COMMON, "--cuda-device-only", "-S",
              os.path.join(CSRC, src), "-o", out])
        with open(out) as f:
            return f.read()


if __name__ == "__main__":
    print(build(verbose=True))
