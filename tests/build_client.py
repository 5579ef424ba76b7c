"""Compile tests/c_abi_client.c, a plain C program that drives libs2attn.so
through include/s2attn.h with device memory from the HIP runtime.

    python tests/build_client.py

The binary goes to tests/_bin/c_abi_client and finds libs2attn.so next to the
package sources at run time (rpath relative to the binary), so the tree can be
moved.  Needs libs2attn.so built first.
"""

import os
import subprocess

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
PKG = os.path.join(ROOT, "shifted_sparse_attention_s2attn_amd")
SRC = os.path.join(TESTS, "c_abi_client.c")
BIN = os.path.join(TESTS, "_bin", "c_abi_client")
ROCM = "/opt/rocm"


def build_client(out=BIN):
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", out + ".tmp",
           "-L", PKG, "-ls2attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../shifted_sparse_attention_s2attn_amd", "-Wl,-rpath," + PKG,
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"client build failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_client())
