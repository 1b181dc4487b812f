"""The library's C ABI driven from a plain C program (no torch, no Python): planes, passes,
weights and the update against the C oracle, and the documented argument errors.  The
program is built by ``__graft_entry__.build()`` from ``tests/capi/capi_check.c``."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "capi", "capi_check")


@pytest.mark.gpu
def test_c_program_through_the_abi_matches_the_oracle():
    if not os.path.exists(BIN):
        import capi
        capi.build()
    print(f"running {BIN}", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi ok" in r.stdout
