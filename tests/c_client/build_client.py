"""Compile tests/c_client/step_client.c, a C99 caller of libzero_shard.so and
the HIP runtime with no Python in between, into tests/c_client/step_client.

The GPU test that runs it lives beside the other GPU tests; the program is
built here, on the host, like the library (gcc against the HIP runtime's C
API; no device code).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "step_client.c")
EXE = os.path.join(HERE, "step_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    lib_dir = os.path.join(ROOT, "zero_sharded_mixed_shard_amd")
    tmp = EXE + ".tmp"
    subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROCM, "include"), SRC, "-o", tmp,
                    "-L", lib_dir, "-lzero_shard", "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../zero_sharded_mixed_shard_amd",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
