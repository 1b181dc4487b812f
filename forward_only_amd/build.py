"""Build libzo.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m forward_only_amd.build        # or forward_only_amd.build.build()

Every .hip file under csrc/ is compiled to an object in _build/ and linked into
forward_only_amd/libzo.so.  Flags:
  * -ffp-contract=off: no implicit FMA; the kernels spell out every fused multiply-add
    they want, so each rounding is the one the code names.
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU instructions.
  * no fast-math and no denormal flushing.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libzo.so")
CEILING_SRC = os.path.join(HERE, "ceiling", "hbm_ceiling.hip")
CEILING_BIN = os.path.join(HERE, "hbm_ceiling")
PHILOX_SRC = os.path.join(HERE, "ceiling", "philox_ceiling.hip")
PHILOX_BIN = os.path.join(HERE, "philox_ceiling")
ARCH = os.environ.get("ZO_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_ceiling(verbose)
    return LIB


def build_ceiling(verbose: bool = False) -> str:
    """The standalone ceiling microbenchmarks: HBM (read, write, copy, in-place RMW) and
    Philox4x32-10 calls per second."""
    for src, out in ((CEILING_SRC, CEILING_BIN), (PHILOX_SRC, PHILOX_BIN)):
        tmp = out + f".tmp{os.getpid()}"
        cmd = [HIPCC, *CFLAGS, "-o", tmp, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, out)
    return CEILING_BIN


if __name__ == "__main__":
    print(build(verbose=True))
