"""Plain CPU oracle for the 1.5-SPSA perturb / probe-weight / update path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  It never imports the HIP library
(``forward_only_amd``) and shares no code with it; the two meet only through the seeded
input generators in ``workloads``.

The arithmetic lives in ``zo_oracle.c`` (compiled by ``oracle/build.py`` with gcc, no
FMA contraction); this module marshals numpy arrays into it and adds the parts that are
plain library calls in fp64 (the MLP loss) and the step driver that strings the
primitives together in the order the pages give.

Sources (page titles and sections, see the header of ``zo_oracle.c`` for details):
  * "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation" -- "How 1.5-SPSA Works"
    (probes, central difference) and "Probe-Space Preconditioning" (clean pass, per-probe
    curvature weight).
  * "Pretraining Transformers Without Backprop: What Two Zero-Order Papers Actually
    Measure" -- the ZOO training-loop flowchart (perturb, forward, estimate, update).

bf16 arrays are numpy ``uint16`` holding the bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))

_lib = None


def lib() -> ctypes.CDLL:
    """Load ``liboracle.so``, compiling it with gcc first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    u64, u32, f32, f64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_double
    sig = {
        "ora_philox4x32_10": (None, [u32p, u32p, u32p]),
        "ora_sign": (ctypes.c_int, [u64, u32, u32, u64]),
        "ora_plane_bytes": (u64, [u64]),
        "ora_gen_plane": (None, [u64, u32, u32, u64, u64, u8p]),
        "ora_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "ora_f64_to_bf16": (ctypes.c_uint16, [f64]),
        "ora_f32_to_bf16": (ctypes.c_uint16, [f32]),
        "ora_f64_to_bf16_array": (None, [f64p, u16p, u64]),
        "ora_f32_to_bf16_array": (None, [f32p, u16p, u64]),
        "ora_perturb_f32": (None, [f32p, u64, u64, u64, u32, u32, f32, u8p]),
        "ora_perturb_bf16": (None, [u16p, u64, u64, u64, u32, u32, f32, u8p]),
        "ora_perturb2_f32": (None, [f32p, u64, u64, u64, u32, u32, f32, u32, f32, u8p, u8p]),
        "ora_perturb2_bf16": (None, [u16p, u64, u64, u64, u32, u32, f32, u32, f32, u8p, u8p]),
        "ora_probe_weights": (u32, [f64p, f64p, f64, u32, f64, f64, f32p]),
        "ora_probe_weights_ex": (u32, [f64p, f64p, f64, u32, f64, f64, ctypes.c_int, f64, f32p]),
        "ora_update_f32": (None, [f32p, u64, u64, u64, u32, f32p, u32, f32, u8p]),
        "ora_update_bf16": (None, [u16p, u64, u64, u64, u32, f32p, u32, f32, u8p]),
        "ora_probe_sums": (None, [f64p, u64, u64, u64, u32, f32p, u32, u8p]),
        "ora_quad_loss_f32": (f64, [f32p, f32p, u64]),
        "ora_quad_loss_bf16": (f64, [u16p, f32p, u64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bits_ptr(bits):
    if bits is None:
        return ctypes.POINTER(ctypes.c_uint8)()
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    return _ptr(bits, ctypes.c_uint8)


# ------------------------------------------------------------------------------------
# Philox4x32-10 and the probe signs
# ------------------------------------------------------------------------------------
def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of a 4-word counter and a 2-word key (Salmon et al., SC'11)."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().ora_philox4x32_10(_ptr(c, ctypes.c_uint32), _ptr(k, ctypes.c_uint32),
                            _ptr(out, ctypes.c_uint32))
    return out


def sign(seed: int, step: int, probe: int, j: int) -> int:
    """Rademacher sign of global parameter j for (seed, step, probe)."""
    return int(lib().ora_sign(seed, step, probe, j))


def plane_bytes(n: int) -> int:
    return int(lib().ora_plane_bytes(n))


def gen_plane(seed: int, step: int, probe: int, offset: int, n: int) -> np.ndarray:
    """Packed signs of one probe over global params [offset, offset+n); offset % 128 == 0."""
    assert offset % 128 == 0
    out = np.zeros(plane_bytes(n), dtype=np.uint8)
    lib().ora_gen_plane(seed, step, probe, offset, n, _ptr(out, ctypes.c_uint8))
    return out


def gen_planes(seed: int, step: int, probe0: int, n_probes: int, offset: int,
               n: int) -> np.ndarray:
    """n_probes consecutive packed rows, shape (n_probes, plane_bytes(n))."""
    return np.stack([gen_plane(seed, step, probe0 + p, offset, n) for p in range(n_probes)]) \
        if n_probes else np.zeros((0, plane_bytes(n)), dtype=np.uint8)


def signs_from_plane(row: np.ndarray, n: int) -> np.ndarray:
    """Expand a packed row into n values in {-1, +1} (float64)."""
    bits = np.unpackbits(np.asarray(row, dtype=np.uint8), bitorder="little")[:n]
    return bits.astype(np.float64) * 2.0 - 1.0


# ------------------------------------------------------------------------------------
# bf16 helpers
# ------------------------------------------------------------------------------------
def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    lib().ora_f64_to_bf16_array(_ptr(x, ctypes.c_double), _ptr(out, ctypes.c_uint16), x.size)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, dtype=np.uint16)
    lib().ora_f32_to_bf16_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


# ------------------------------------------------------------------------------------
# The path's primitives
# ------------------------------------------------------------------------------------
def perturb(theta: np.ndarray, offset: int, seed: int, step: int, probe: int, alpha: float,
            bits=None) -> None:
    """theta <- theta + alpha * z_probe, in place.  theta: float32, or uint16 (bf16 bits)."""
    assert offset % 128 == 0
    a = float(np.float32(alpha))
    if theta.dtype == np.float32:
        lib().ora_perturb_f32(_ptr(theta, ctypes.c_float), theta.size, offset, seed, step,
                              probe, a, _bits_ptr(bits))
    elif theta.dtype == np.uint16:
        lib().ora_perturb_bf16(_ptr(theta, ctypes.c_uint16), theta.size, offset, seed, step,
                               probe, a, _bits_ptr(bits))
    else:
        raise TypeError(theta.dtype)


def perturb2(theta: np.ndarray, offset: int, seed: int, step: int, probe_a: int,
             alpha_a: float, probe_b: int, alpha_b: float, bits_a=None, bits_b=None) -> None:
    """theta <- round(theta + ((+/-alpha_a) + (+/-alpha_b))) in one pass, in place."""
    assert offset % 128 == 0
    aa, ab = float(np.float32(alpha_a)), float(np.float32(alpha_b))
    if theta.dtype == np.float32:
        lib().ora_perturb2_f32(_ptr(theta, ctypes.c_float), theta.size, offset, seed, step,
                               probe_a, aa, probe_b, ab, _bits_ptr(bits_a), _bits_ptr(bits_b))
    elif theta.dtype == np.uint16:
        lib().ora_perturb2_bf16(_ptr(theta, ctypes.c_uint16), theta.size, offset, seed, step,
                                probe_a, aa, probe_b, ab, _bits_ptr(bits_a), _bits_ptr(bits_b))
    else:
        raise TypeError(theta.dtype)


def probe_weights(Lp, Lm, L0: float, eps: float, delta: float):
    """c_i = g_i / max(|h_i|, delta) as fp32, and the count of dropped (non-finite) probes."""
    Lp = np.ascontiguousarray(Lp, dtype=np.float64)
    Lm = np.ascontiguousarray(Lm, dtype=np.float64)
    n = Lp.size
    assert Lm.size == n
    c = np.zeros(n, dtype=np.float32)
    bad = lib().ora_probe_weights(_ptr(Lp, ctypes.c_double), _ptr(Lm, ctypes.c_double),
                                  float(L0), n, float(eps), float(delta),
                                  _ptr(c, ctypes.c_float))
    return c, int(bad)


WEIGHTS_PRECOND, WEIGHTS_POWER, WEIGHTS_SPSA_MEAN = 0, 1, 2


def probe_weights_ex(Lp, Lm, L0: float, eps: float, delta: float, mode: int,
                     power: float = 1.0):
    """The weight forms of the pages: preconditioned, curvature power, plain SPSA mean."""
    Lp = np.ascontiguousarray(Lp, dtype=np.float64)
    Lm = np.ascontiguousarray(Lm, dtype=np.float64)
    n = Lp.size
    c = np.zeros(n, dtype=np.float32)
    bad = lib().ora_probe_weights_ex(_ptr(Lp, ctypes.c_double), _ptr(Lm, ctypes.c_double),
                                     float(L0), n, float(eps), float(delta), int(mode),
                                     float(power), _ptr(c, ctypes.c_float))
    return c, int(bad)


def update(theta: np.ndarray, offset: int, seed: int, step: int, c, eta: float,
           bits=None) -> None:
    """theta <- theta - eta * sum_i c_i z_i, in place; fp64 sum, one final rounding."""
    assert offset % 128 == 0
    c = np.ascontiguousarray(c, dtype=np.float32)
    e = float(np.float32(eta))
    if bits is not None:
        bits = np.ascontiguousarray(bits, dtype=np.uint8)
        assert bits.shape == (c.size, plane_bytes(theta.size))
    if theta.dtype == np.float32:
        lib().ora_update_f32(_ptr(theta, ctypes.c_float), theta.size, offset, seed, step,
                             _ptr(c, ctypes.c_float), c.size, e, _bits_ptr(bits))
    elif theta.dtype == np.uint16:
        lib().ora_update_bf16(_ptr(theta, ctypes.c_uint16), theta.size, offset, seed, step,
                              _ptr(c, ctypes.c_float), c.size, e, _bits_ptr(bits))
    else:
        raise TypeError(theta.dtype)


def probe_sums(n: int, offset: int, seed: int, step: int, c, bits=None) -> np.ndarray:
    """s_j = sum_i c_i z_ij in fp64 (i ascending), j in [offset, offset+n)."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    s = np.zeros(n, dtype=np.float64)
    lib().ora_probe_sums(_ptr(s, ctypes.c_double), n, offset, seed, step,
                         _ptr(c, ctypes.c_float), c.size, _bits_ptr(bits))
    return s


def quad_loss(theta: np.ndarray, a: np.ndarray) -> float:
    """L = 1/2 sum_j a_j theta_j^2 in fp64 (j ascending)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    assert a.size == theta.size
    if theta.dtype == np.float32:
        return float(lib().ora_quad_loss_f32(_ptr(theta, ctypes.c_float),
                                             _ptr(a, ctypes.c_float), theta.size))
    if theta.dtype == np.uint16:
        return float(lib().ora_quad_loss_bf16(_ptr(theta, ctypes.c_uint16),
                                              _ptr(a, ctypes.c_float), theta.size))
    raise TypeError(theta.dtype)


from .lowrank import lowrank_quad_loss  # noqa: E402  (plain fp64 numpy)
from .mlp import mlp_loss, mlp_unflatten  # noqa: E402  (plain fp64 numpy)
from .step import spsa_step  # noqa: E402
