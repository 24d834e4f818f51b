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

import hashlib
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzero_shard.so")
# SHA-256 of each kernel's machine code, written beside the library by build()
ISA_HASHES = os.path.join(PKG, "kernel_isa.sha256")
KERNEL_SOURCES = ["shard_kernels.hip", "exchange_kernels.hip"]

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
        hashes = {}
        for src in KERNEL_SOURCES:
            hashes.update(kernel_isa_hashes(device_assembly(src)))
        with open(ISA_HASHES + ".tmp", "w") as f:
            for name in sorted(hashes):
                f.write(f"{hashes[name]}  {name}\n")
        os.replace(ISA_HASHES + ".tmp", ISA_HASHES)
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


def kernel_isa_hashes(asm: str) -> dict:
    """SHA-256 of each kernel's gfx950 code and kernel descriptor, by symbol.

    Comments, debug-line directives and the file-wide numbering of local labels
    are left out, so a kernel's hash changes when its own instructions or launch
    resources do, and not when another kernel in the same file changes."""
    lines = asm.splitlines()
    names = re.findall(r"^\s*\.amdhsa_kernel (\S+)", asm, re.M)
    out = {}
    for name in names:
        body = []
        start = next(i for i, ln in enumerate(lines) if ln.startswith(name + ":"))
        for ln in lines[start:]:
            body.append(ln)
            if ln.startswith(".Lfunc_end"):
                break
        desc_start = next(i for i, ln in enumerate(lines)
                          if ln.strip() == f".amdhsa_kernel {name}")
        for ln in lines[desc_start:]:
            body.append(ln)
            if ln.strip() == ".end_amdhsa_kernel":
                break
        norm = []
        for ln in body:
            ln = ln.split(";", 1)[0].strip()
            if not ln or ln.startswith((".loc", ".file", ".cfi_")):
                continue
            ln = re.sub(r"\.LBB\d+_(\d+)", r".LBB_\1", ln)
            ln = re.sub(r"\.Lfunc_end\d+", ".Lfunc_end", ln)
            norm.append(ln)
        out[name] = hashlib.sha256("\n".join(norm).encode()).hexdigest()
    return out


def read_isa_hashes(path: str = ISA_HASHES) -> dict:
    """The per-kernel hashes that the last build() wrote (empty if none)."""
    if not os.path.exists(path):
        return {}
    out = {}
    with open(path) as f:
        for ln in f:
            h, name = ln.split()
            out[name] = h
    return out


if __name__ == "__main__":
    print(build(verbose=True))
