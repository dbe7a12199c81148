"""Build libhci.so (HIP, gfx950) in-tree with hipcc.

    python -m hybrid_conv_iir_amd.build

Compiles every ``csrc/*.hip`` to an object in parallel and links the shared
library next to this file.  Always rebuilds (the build is the "does it
compile" check); takes a few tens of seconds.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libhci.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # compiler-formed packed fp32 ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in vector registers where they fit: otherwise the attention
    # kernels' score accumulators land in accumulation registers and are copied out for the
    # softmax on every tile (several hundred extra moves per KV tile with four query tiles)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr}")


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found under csrc/")
    with tempfile.TemporaryDirectory(prefix="hci_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s)[:-4] + ".o") for s in srcs]
        workers = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), 16)
        with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
            list(ex.map(_compile, srcs, objs))
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        shutil.move(out_tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
