"""Helpers shared by the GPU tests: host<->device conversions and the tolerances.

Tolerances (written here, used by every GPU parity test):
  * integer / bit work (packed planes, perturb, probe weights): bit-exact;
  * fp32 update: |theta_gpu - theta_ora| <= 1e-5 * max(|theta_ora|, eta * sum_i |c_i|);
  * bf16 update: at most one bf16 ulp apart.  Both sides form theta - eta * s in fp64 and
    round that double once to bf16 (the GPU through a round-to-odd fp32 and the hardware
    nearest-even convert, which together round the double correctly; the oracle directly),
    but they sum the probes in different orders (per-8-probe tables against one running
    sum), so s -- and with it a result next to a rounding boundary -- may differ by one.
"""
from __future__ import annotations

import numpy as np
import torch


def to_dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_dev_bf16(h: np.ndarray) -> torch.Tensor:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 at |x| (2^(e-7) for normals, 2^-133 below 2^-126)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.maximum(2.0 ** (e - 7), 2.0 ** -133)


def assert_f32_update_close(got: np.ndarray, ref: np.ndarray, eta: float, c: np.ndarray):
    scale = np.maximum(np.abs(ref.astype(np.float64)),
                       float(np.float32(eta)) * float(np.sum(np.abs(c.astype(np.float64)))))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bad = err > 1e-5 * scale
    assert not bad.any(), (f"{bad.sum()} of {bad.size} elements out of tolerance; worst "
                           f"{(err / scale).max():.3e} relative")


def assert_bf16_within_ulp(got: np.ndarray, ref: np.ndarray):
    g, r = bf16_values(got), bf16_values(ref)
    both_nan = np.isnan(g) & np.isnan(r)
    ok = both_nan | (g == r) | (np.abs(g - r) <= bf16_ulp(np.maximum(np.abs(g), np.abs(r))))
    assert ok.all(), f"{(~ok).sum()} bf16 elements more than 1 ulp apart"
    return int((g != r).sum() - both_nan.sum())


def assert_same_bits_or_nan(got: np.ndarray, ref: np.ndarray, kind: str):
    if kind == "f32":
        gv, rv = got.view(np.uint32), ref.view(np.uint32)
        nan = np.isnan(got) & np.isnan(ref)
    else:
        gv, rv = got, ref
        nan = np.isnan(bf16_values(got)) & np.isnan(bf16_values(ref))
    diff = (gv != rv) & ~nan
    assert not diff.any(), f"{diff.sum()} elements differ; first at {np.argmax(diff)}"


def weight_bound(Lp, Lm, L0, dL, eps, delta, c):
    """Largest |c_gpu - c_oracle| the loss differences |dL| (per loss, a bound) can cause.

    c = g / max(|h|, delta), g = (L+ - L-)/(2 eps), h = (L+ + L- - 2 L0)/eps^2.  With every
    loss off by at most dL: |dg| <= dL / eps, |dh| <= 4 dL / eps^2, and
    c' - c = dg / (d + dd) - g dd / (d (d + dd)) with d = max(|h|, delta) and |dd| <= |dh|
    (the max is 1-Lipschitz), so |dc| <= (|dg| + |g| |dh| / d) / (d - |dh|), plus one fp32
    rounding of c on each side.  Returns inf where d <= 2 |dh|.
    """
    Lp, Lm = np.asarray(Lp, np.float64), np.asarray(Lm, np.float64)
    g = (Lp - Lm) / (2 * eps)
    h = (Lp + Lm - 2 * L0) / eps ** 2
    dg = dL / eps
    dh = 4 * dL / eps ** 2
    d = np.maximum(np.abs(h), delta)
    with np.errstate(divide="ignore", invalid="ignore"):
        b = (dg + np.abs(g) * dh / d) / (d - dh)
    b = np.where(d > 2 * dh, b, np.inf)
    ulp = np.spacing(np.abs(np.asarray(c, np.float32))).astype(np.float64)
    return b + 2 * ulp
