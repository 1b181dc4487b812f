"""Host-only checks of libzo.so: it loads without a GPU, exports every entry point that
include/*.h declares, and rejects bad arguments before touching the device."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import forward_only_amd as zo
from forward_only_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(zo_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("zo_init", "zo_gen_probes", "zo_perturb", "zo_probe_weights", "zo_update",
                 "zo_tune_placement"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    # and the binding covers every one of them
    assert set(declared_functions()) <= set(_lib.SIGNATURES)


def test_pure_host_calls():
    L = _lib.lib()
    assert L.zo_bits_stride(0) == 0
    assert L.zo_bits_stride(1) == 16
    assert L.zo_bits_stride(128) == 16
    assert L.zo_bits_stride(129) == 32
    assert L.zo_bits_stride(125_000_000) == 15_625_008
    for s in range(6):
        assert L.zo_strerror(s)
    assert L.zo_get_seed(None) == 0


def test_null_context_and_arguments_are_rejected():
    L = _lib.lib()
    assert L.zo_init(0, None) == _lib.ZO_EINVAL
    assert L.zo_destroy(None) == _lib.ZO_OK
    assert L.zo_perturb(None, None, 0, 0, 16, 0, 0, 1.0, None, None) == _lib.ZO_EINVAL
    assert L.zo_update(None, None, 0, 0, 16, 0, None, 1, 1.0, None, None) == _lib.ZO_EINVAL
    assert L.zo_gen_probes(None, 0, 0, 1, 0, 16, None, None) == _lib.ZO_EINVAL
    assert L.zo_probe_weights(None, None, None, None, 1, 1e-3, 0.0, None, None) == _lib.ZO_EINVAL
    v = ctypes.c_uint32()
    assert L.zo_nonfinite_count(None, None, ctypes.byref(v)) == _lib.ZO_EINVAL
    assert L.zo_stream_rmw(None, None, 16, 0, None) == _lib.ZO_EINVAL
    assert L.zo_restore_update(None, None, 0, 0, 16, 0, 0, 1.0, None, 1, 1.0, None,
                               None) == _lib.ZO_EINVAL
    assert L.zo_set_slice_bytes(None, 0) == _lib.ZO_EINVAL
    assert L.zo_get_slice_bytes(None) == 0
    assert L.zo_tune_placement(None, None, 16, None, None, None, None) == _lib.ZO_EINVAL
    assert L.zo_mlp_loss_pair(None, None, 0, 0, 0, 1.0, None, None, None, 16, 16, 16, 2, None,
                              0, None, None, None) == _lib.ZO_EINVAL
    assert L.zo_quad_loss_probes(None, None, 0, None, 0, 16, 0, 0, 1, 1.0, None, None, None,
                                 None, None) == _lib.ZO_EINVAL
    assert L.zo_mlp_loss_probes(None, None, 0, 0, 0, 1, 1.0, None, None, None, 16, 16, 16, 2,
                                None, 0, None, None, None, None) == _lib.ZO_EINVAL


def test_init_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    st = _lib.lib().zo_init(1, ctypes.byref(h))
    assert st in (_lib.ZO_EHIP, _lib.ZO_ENOMEM)
    assert h.value is None
    with pytest.raises(zo.ZOError):
        zo.zo_init(1)


def test_fused_step_needs_a_clean_loss_source():
    """spsa_step_fused without loss_at must get the clean loss from loss_probes_at; the check
    comes before any device call."""
    import pytest
    import torch
    from forward_only_amd.step import spsa_step_fused
    theta = torch.zeros(8)
    with pytest.raises(ValueError):
        spsa_step_fused(None, theta, step=0, npert=2, eps=1e-3, eta=1e-3, delta=1e-6)
    with pytest.raises(ValueError):
        spsa_step_fused(None, theta, step=0, npert=2, eps=1e-3, eta=1e-3, delta=1e-6,
                        loss_probes_at=lambda *a: None)
