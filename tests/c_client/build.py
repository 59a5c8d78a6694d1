"""Builds rra_c_client, the plain C11 caller of the library's C ABI that
tests/test_gpu_c_client.py runs beside the Python binding.  Host code only: gcc
compiles it against include/rra.h and the HIP runtime API and links the
in-tree librra.so (found at run time through an $ORIGIN-relative run path)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BINARY = os.path.join(HERE, "rra_c_client")


def build() -> str:
    """Compiles the client (the library must be built first); returns its path."""
    lib_dir = os.path.join(ROOT, "rope_residual_add_amd")
    if not os.path.exists(os.path.join(lib_dir, "librra.so")):
        raise RuntimeError("librra.so is not built: build the library first")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(HERE, "rra_c_client.c"),
           "-L", lib_dir, "-lrra", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../rope_residual_add_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", BINARY + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY


if __name__ == "__main__":
    print(build())
