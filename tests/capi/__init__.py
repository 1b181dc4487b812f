"""Build of the plain-C check of the library's ABI (``capi_check.c``).

Test-only: the program links ``forward_only_amd/libzo.so`` and the C oracle
``oracle/liboracle.so`` side by side and is run by ``tests/test_gpu_capi.py``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "capi_check.c")
BIN = os.path.join(HERE, "capi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ZO_DIR = os.path.join(ROOT, "forward_only_amd")
ORA_DIR = os.path.join(ROOT, "oracle")


def build(verbose: bool = False) -> str:
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O1", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-o", tmp, SRC,
           "-L", ZO_DIR, "-lzo", "-Wl,-rpath,$ORIGIN/../../forward_only_amd",
           "-L", ORA_DIR, "-loracle", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN
