"""Build librra.so, the HIP C-ABI library, for gfx950 with hipcc.

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into rope_residual_add_amd/librra.so (in-tree, next to the
Python binding that loads it)."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SO = os.path.join(PKG, "librra.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from forming v_pk_{add,mul,fma}_f32.
# Code object v5 loads under both the ROCm 7.2 toolchain's runtime and the
# ROCm 7.0 HIP runtime bundled with PyTorch.  Kernel-argument preloading puts
# the first 14 dwords of each kernel's arguments in scalar registers at wave
# start (with a fallback prologue that loads them where the firmware does
# not), so a short wave's first loads need not wait for its arguments; the
# kernels lead with the arguments those loads need.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-I", INCLUDE, "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="rra_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(pair):
            src, obj = pair
            cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            if verbose and r.stderr.strip():
                print(r.stderr)

        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            list(ex.map(compile_one, zip(srcs, objs)))
        tmp_so = SO + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_so]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_so, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
