"""fp64 loss of the two-layer MLP classifier used as a small real forward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The loss is the model's forward pass that the ZOO loop evaluates at the clean and the
perturbed weights (flowchart of "Pretraining Transformers Without Backprop: What Two
Zero-Order Papers Actually Measure", the forward-pass box).  Layout of the flat
parameter vector: W1 [hidden x in] row-major, b1 [hidden], W2 [out x hidden] row-major,
b2 [out].  Hidden activation: GELU in its exact form x * Phi(x) with the normal CDF Phi
written through erf.  Loss: batch mean of logsumexp(logits) - logits[label].
Every step is a plain numpy/scipy call in float64.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def mlp_unflatten(params: np.ndarray, d_in: int, d_hid: int, d_out: int):
    p = np.asarray(params, dtype=np.float64).ravel()
    sizes = [d_hid * d_in, d_hid, d_out * d_hid, d_out]
    assert p.size == sum(sizes), (p.size, sum(sizes))
    o = np.cumsum([0] + sizes)
    W1 = p[o[0]:o[1]].reshape(d_hid, d_in)
    b1 = p[o[1]:o[2]]
    W2 = p[o[2]:o[3]].reshape(d_out, d_hid)
    b2 = p[o[3]:o[4]]
    return W1, b1, W2, b2


def gelu_exact(x: np.ndarray) -> np.ndarray:
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def mlp_logits(params, X, d_hid: int, d_out: int) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    W1, b1, W2, b2 = mlp_unflatten(params, X.shape[1], d_hid, d_out)
    h = gelu_exact(X @ W1.T + b1)
    return h @ W2.T + b2


def mlp_loss(params, X, labels, d_hid: int, d_out: int) -> float:
    """Mean cross-entropy of the MLP at `params` (fp32 or fp64 values, computed in fp64)."""
    z = mlp_logits(params, X, d_hid, d_out)
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))).ravel()
    lab = np.asarray(labels, dtype=np.int64)
    return float(np.mean(lse - z[np.arange(z.shape[0]), lab]))
