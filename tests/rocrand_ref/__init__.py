"""rocRAND's Philox4x32-10 engine as a second, independent check of the probe bits.

Test-only: ``rocrand_ref.cpp`` is compiled for the host with g++ against the open-source
header shipped in the ROCm include tree and loaded with ctypes; nothing in the library or
the oracle uses it.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rocrand_ref.cpp")
LIB = os.path.join(HERE, "librocrand_ref.so")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
HEADER = os.path.join(ROCM_INCLUDE, "rocrand", "rocrand_philox4x32_10.h")

_lib = None


def available() -> bool:
    return os.path.exists(LIB) or os.path.exists(HEADER)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", ROCM_INCLUDE, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        u64, u32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
        L.rr_philox_words.argtypes = [u64, u32, u32, u64, u64, vp]
        L.rr_philox_words.restype = None
        L.rr_plane.argtypes = [u64, u32, u32, u64, u64, vp]
        L.rr_plane.restype = None
        _lib = L
    return _lib


def philox_words(seed: int, step: int, probe: int, blk0: int, nblk: int) -> np.ndarray:
    """Words of blocks blk0 .. blk0+nblk-1 as a uint32 array of shape (nblk, 4)."""
    out = np.zeros((nblk, 4), dtype=np.uint32)
    lib().rr_philox_words(seed, step, probe, blk0, nblk, out.ctypes.data)
    return out


def plane(seed: int, step: int, probe: int, offset: int, n: int) -> np.ndarray:
    """Packed sign plane of one probe over [offset, offset + n) (offset % 128 == 0)."""
    assert offset % 128 == 0
    out = np.zeros(((n + 127) // 128) * 16, dtype=np.uint8)
    lib().rr_plane(seed, step, probe, offset, n, out.ctypes.data)
    return out
