"""Seeded input generators.

* theta and the quadratic's coefficients: numpy PCG64 seeded with the workload's seed;
  theta first, then a_j = 10^U(lo, hi) (log-uniform), both stored as float32.
* synthetic per-probe losses of the OPT-shaped workloads, redrawn every step from
  PCG64(SeedSequence([seed, step])) in the order L0, u[n], v+[n], v-[n]:
  L0 ~ N(2.0, 0.05); L+_i = L0 + u_i + v+_i; L-_i = L0 - u_i + v-_i, with
  u_i ~ N(0, 0.01) shared by the pair and v+/-_i ~ N(0.002, 0.001) independent.
* MLP data: teacher weights N(0, 0.02) from the teacher seed, inputs N(0, 1) from the
  input seed, labels = argmax of the teacher's logits (teacher evaluated in float64).
* OPT-shaped bf16 parameter sets are too large for the host: they are drawn on the
  device with torch's own seeded generator (device_normal_), chunk by chunk.

Nothing here implements any step of the method itself.
"""
from __future__ import annotations

import numpy as np

from .configs import Config


def theta_and_a(cfg: Config):
    """(theta float32 [M], a float32 [M] or None) for the host-sized workloads."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    theta = rng.standard_normal(cfg.M, dtype=np.float64)
    theta = (theta * cfg.theta_std).astype(np.float32)
    a = None
    if cfg.loss == "quad":
        lo, hi = cfg.a_range
        a = np.power(10.0, rng.uniform(lo, hi, cfg.M)).astype(np.float32)
    return theta, a


def lowrank_problem(cfg: Config, M: int | None = None, rank: int | None = None,
                    spike: float | None = None):
    """(theta float32 [M], a float32 [M], U float32 [rank, M]) for the low-rank-plus-
    diagonal quadratic: theta ~ N(0, theta_std), a_j = diag, and U's rows orthogonal
    directions scaled so that the curvature along row k is `spike` (times 1, 2, ...)."""
    e = cfg.extra
    M = M or cfg.M
    rank = rank if rank is not None else e["rank"]
    spike = spike if spike is not None else e["spike"]
    rng = np.random.Generator(np.random.PCG64(cfg.seed + 101))
    theta = (rng.standard_normal(M) * cfg.theta_std).astype(np.float32)
    a = np.full(M, e["diag"], dtype=np.float32)
    G = rng.standard_normal((rank, M))
    Q, _ = np.linalg.qr(G.T)                              # orthonormal columns
    scales = np.sqrt(spike * (np.arange(rank) + 1.0))
    U = np.ascontiguousarray((Q.T * scales[:, None]).astype(np.float32))
    return theta, a, U


def synthetic_losses(seed: int, step: int, n: int):
    """(L0, Lp[n], Lm[n]) float64 for the synthetic-loss workloads."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, step])))
    L0 = rng.normal(2.0, 0.05)
    u = rng.normal(0.0, 0.01, n)
    vp = rng.normal(0.002, 0.001, n)
    vm = rng.normal(0.002, 0.001, n)
    return float(L0), L0 + u + vp, L0 - u + vm


def _gelu_exact_f64(x):
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def mlp_data(cfg: Config):
    """(X float32 [batch, d_in], labels int64 [batch]) for the MLP workload."""
    e = cfg.extra
    d_in, d_hid, d_out, B = e["d_in"], e["d_hid"], e["d_out"], e["batch"]
    rt = np.random.Generator(np.random.PCG64(e["teacher_seed"]))
    W1 = rt.standard_normal((d_hid, d_in)) * 0.02
    b1 = rt.standard_normal(d_hid) * 0.02
    W2 = rt.standard_normal((d_out, d_hid)) * 0.02
    b2 = rt.standard_normal(d_out) * 0.02
    rx = np.random.Generator(np.random.PCG64(e["input_seed"]))
    X = rx.standard_normal((B, d_in)).astype(np.float32)
    logits = _gelu_exact_f64(X.astype(np.float64) @ W1.T + b1) @ W2.T + b2
    labels = np.argmax(logits, axis=1).astype(np.int64)
    return X, labels


def dyadic_theta(n: int, seed: int, frac_bits: int = 12, max_abs_log2: int = 4):
    """float32 values k * 2^-frac_bits with |value| < 2^max_abs_log2 (exact in fp32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lim = 2 ** (max_abs_log2 + frac_bits) - 1
    k = rng.integers(-lim, lim + 1, n)
    return (k.astype(np.float64) * 2.0 ** -frac_bits).astype(np.float32)


def device_normal_(t, std: float, seed: int, chunk: int = 1 << 28):
    """Fill a device tensor in place with N(0, std) from torch's seeded generator."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    for s in range(0, flat.numel(), chunk):
        flat[s:s + chunk].normal_(0.0, std, generator=g)
    return t
