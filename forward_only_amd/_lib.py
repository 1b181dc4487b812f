"""ctypes loader of libzo.so: symbol signatures and status codes of include/zo.h and
include/zo_placement.h.

Loading builds the library in-tree with hipcc only when no built library is present, and
fails loudly otherwise: there is no fallback implementation of any call.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzo.so")

ZO_OK, ZO_EINVAL, ZO_EHIP, ZO_ENOMEM, ZO_EUNSUPPORTED = 0, 1, 2, 3, 4
ZO_FP32, ZO_BF16 = 0, 1
ZO_WEIGHTS_PRECOND, ZO_WEIGHTS_POWER, ZO_WEIGHTS_SPSA_MEAN = 0, 1, 2
ZO_MAX_NPERT = 512
ZO_NOALLOC_SCRATCH_BYTES = 1 << 20

_vp = ctypes.c_void_p
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u32, _u64, _f32, _f64, _int = (ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float,
                                ctypes.c_double, ctypes.c_int)

# name -> (restype, argtypes), in the order of include/zo.h, then include/zo_placement.h
SIGNATURES = {
    "zo_init": (_int, [_u64, ctypes.POINTER(_vp)]),
    "zo_destroy": (_int, [_vp]),
    "zo_get_seed": (_u64, [_vp]),
    "zo_strerror": (ctypes.c_char_p, [_int]),
    "zo_bits_stride": (ctypes.c_size_t, [_u64]),
    "zo_gen_probes": (_int, [_vp, _u32, _u32, _u32, _u64, _u64, _vp, _vp]),
    "zo_perturb": (_int, [_vp, _vp, _int, _u64, _u64, _u32, _u32, _f32, _vp, _vp]),
    "zo_perturb2": (_int, [_vp, _vp, _int, _u64, _u64, _u32, _u32, _f32, _u32, _f32, _vp, _vp,
                           _vp]),
    "zo_probe_weights": (_int, [_vp, _vp, _vp, _vp, _u32, _f64, _f64, _vp, _vp]),
    "zo_probe_weights_ex": (_int, [_vp, _vp, _vp, _vp, _u32, _f64, _f64, _int, _f64, _vp, _vp]),
    "zo_update": (_int, [_vp, _vp, _int, _u64, _u64, _u32, _vp, _u32, _f32, _vp, _vp]),
    "zo_nonfinite_count": (_int, [_vp, _vp, ctypes.POINTER(_u32)]),
    "zo_reset_nonfinite": (_int, [_vp, _vp]),
    "zo_quad_loss": (_int, [_vp, _vp, _int, _vp, _u64, _vp, _vp]),
    "zo_quad_loss_probes": (_int, [_vp, _vp, _int, _vp, _u64, _u64, _u32, _u32, _u32, _f32, _vp,
                                   _vp, _vp, _vp, _vp]),
    "zo_lowrank_quad_loss": (_int, [_vp, _vp, _int, _vp, _vp, _u32, _u64, _vp, _vp]),
    "zo_mlp_workspace_bytes": (_u64, [_u32, _u32, _u32, _u32]),
    "zo_mlp_loss": (_int, [_vp, _vp, _vp, _vp, _u32, _u32, _u32, _u32, _vp, _u64, _vp, _vp]),
    "zo_mlp_loss_perturbed": (_int, [_vp, _vp, _u64, _u32, _u32, _f32, _vp, _vp, _vp, _u32,
                                     _u32, _u32, _u32, _vp, _u64, _vp, _vp]),
    "zo_mlp_loss_pair": (_int, [_vp, _vp, _u64, _u32, _u32, _f32, _vp, _vp, _vp, _u32,
                                _u32, _u32, _u32, _vp, _u64, _vp, _vp, _vp]),
    "zo_mlp_probes_workspace_bytes": (_u64, [_u32, _u32, _u32, _u32, _u32]),
    "zo_mlp_loss_probes": (_int, [_vp, _vp, _u64, _u32, _u32, _u32, _f32, _vp, _vp, _vp, _u32,
                                  _u32, _u32, _u32, _vp, _u64, _vp, _vp, _vp, _vp]),
    "zo_mlp_loss_pair_noalloc": (_int, [_vp, _vp, _u64, _u32, _u32, _f32, _vp, _vp, _vp, _u32,
                                        _u32, _u32, _u32, _vp, _vp, _vp]),
    "zo_stream_rmw": (_int, [_vp, _vp, _u64, _u32, _vp]),
    "zo_tune_placement": (_int, [_vp, _vp, _u64, _vp, _vp, _vp, _vp]),
    "zo_set_slice_bytes": (_int, [_vp, _u64]),
    "zo_get_slice_bytes": (_u64, [_vp]),
    "zo_restore_update": (_int, [_vp, _vp, _int, _u64, _u64, _u32, _u32, _f32, _vp, _u32,
                                 _f32, _vp, _vp]),
}

_lock = threading.Lock()
_lib = None


class ZOError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().zo_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from . import build as _build
                _build.build()
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def check(status: int, what: str) -> None:
    if status != ZO_OK:
        raise ZOError(status, what)
