"""fp64 loss of the low-rank-plus-diagonal quadratic, a synthetic stand-in for a model
forward whose curvature differs from probe to probe.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

    L(theta) = 1/2 sum_j a_j theta_j^2 + 1/2 ||U theta||^2,   A = diag(a) + U^T U,

with U of shape (r, M).  Along a Rademacher probe the curvature is
z^T A z = sum_j a_j + ||U z||^2, which varies with z when U is not zero -- the situation in
which the clean-pass preconditioner of "Stanford's 1.5-SPSA Trains OPT-30B Without
Backpropagation" ("Probe-Space Preconditioning") is said to pay off in proportion to the
condition number, and to coincide with plain SPSA when the condition number is near 1.
Plain numpy in float64 (the matrix-vector product is a library call).
"""
from __future__ import annotations

import numpy as np


def _as_f64(theta: np.ndarray) -> np.ndarray:
    if theta.dtype == np.uint16:
        return (theta.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(theta, dtype=np.float64)


def lowrank_quad_loss(theta: np.ndarray, a: np.ndarray, U: np.ndarray) -> float:
    t = _as_f64(theta)
    a64 = np.asarray(a, dtype=np.float64)
    u = np.asarray(U, dtype=np.float64).reshape(-1, t.size)
    return float(0.5 * np.sum(a64 * t * t) + 0.5 * np.sum((u @ t) ** 2))
