"""Pins of the oracle's probe weights, multi-probe update, losses and whole step.

Independent anchors (closed forms of the estimator on a quadratic, brute force over every
sign pattern, exact rational arithmetic, the Rademacher variance law, and library/autograd
evaluations of the MLP):
  * "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation", section "How 1.5-SPSA
    Works" -- central difference per probe, relative variance growing like M / n_pert;
    section "Probe-Space Preconditioning" -- curvature from the clean pass, and that with
    a condition number near 1 the preconditioned and plain estimators coincide.
  * "Pretraining Transformers Without Backprop: What Two Zero-Order Papers Actually
    Measure", ZOO training-loop flowchart -- W <- W - eta * g_hat.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, gen


# ------------------------------------------------------------------------------------
# helpers
# ------------------------------------------------------------------------------------
def _nearest_f32(F: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (ties to even), by exact comparison."""
    f = np.float32(float(F))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        key = (abs(Fraction(float(cand)) - F), int(np.array([cand]).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def _dyadic_quadratic(M, seed):
    """theta = k/2^8, |theta| < 16; a = k/16 in [1/16, 16): small exact binary values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    th = (rng.integers(-4095, 4096, M) / 256.0).astype(np.float32)
    a = (rng.integers(1, 256, M) / 16.0).astype(np.float32)
    return th, a


# ------------------------------------------------------------------------------------
# probe weights
# ------------------------------------------------------------------------------------
def test_weights_quadratic_closed_forms_exact():
    # With exact binary inputs every loss is exact in fp64, so the central difference is
    # exactly g_i = z_i^T A theta and the second difference exactly h_i = z_i^T A z_i,
    # which for a diagonal A and z_j^2 = 1 is tr(A) for every probe.
    M, n, seed, step = 4096, 16, 7, 2
    th0, a = _dyadic_quadratic(M, 11)
    eps = 2.0 ** -8
    th = th0.copy()
    out = oracle.spsa_step(th, seed=seed, step=step, npert=n, eps=eps, eta=0.0, delta=1e-6,
                           loss_fn=lambda t: oracle.quad_loss(t, a))
    trA = float(np.sum(a.astype(np.float64)))
    Z = np.stack([oracle.signs_from_plane(oracle.gen_plane(seed, step, i, 0, M), M)
                  for i in range(n)])
    g_exact = Z @ (a.astype(np.float64) * th0.astype(np.float64))
    g = (out["Lp"] - out["Lm"]) / (2 * eps)
    h = (out["Lp"] + out["Lm"] - 2 * out["L0"]) / eps ** 2
    assert np.array_equal(g, g_exact)
    assert np.all(h == trA)
    for i in range(n):
        assert out["c"][i] == _nearest_f32(Fraction(g_exact[i]) / Fraction(trA))
    assert np.array_equal(th, th0)          # eta = 0 and exact restores: unchanged


def test_weights_floor_sign_and_nonfinite():
    L0 = 1.0
    eps = 1e-3
    # h = 0 -> divided by delta; negative curvature -> divided by |h|
    Lp = np.array([1.0 + 1e-4, 1.0 + 1e-4, 1.0 - 3e-4, np.nan, 1.0])
    Lm = np.array([1.0 - 1e-4, 1.0 - 5e-4, 1.0 - 1e-4, 1.0, np.inf])
    c, bad = oracle.probe_weights(Lp, Lm, L0, eps, 1e-6)
    g = (Lp[:3] - Lm[:3]) / (2 * eps)
    h = ((Lp[:3] + Lm[:3]) - 2 * L0) / eps ** 2
    assert abs(h[0]) < 1e-6 and c[0] == np.float32(g[0] / 1e-6)
    assert h[1] < 0 and c[1] == np.float32(g[1] / abs(h[1]))
    assert np.sign(c[2]) == np.sign(g[2])
    assert c[3] == 0 and c[4] == 0 and bad == 2
    # a non-finite clean loss drops every probe
    c, bad = oracle.probe_weights(Lp[:3], Lm[:3], np.inf, eps, 1e-6)
    assert bad == 3 and np.all(c == 0)


def test_weights_isotropic_reduce_to_plain_spsa():
    # A = a I (condition number 1): h_i = a M for every probe, so the preconditioned
    # weights are the plain central differences times the single constant 1/(a M).
    M, n, step = 512, 8, 0
    rng = np.random.Generator(np.random.PCG64(3))
    th = (rng.integers(-1000, 1000, M) / 64.0).astype(np.float32)
    a = np.full(M, 0.25, dtype=np.float32)
    eps = 2.0 ** -6
    out = oracle.spsa_step(th, seed=1, step=step, npert=n, eps=eps, eta=0.0, delta=1e-6,
                           loss_fn=lambda t: oracle.quad_loss(t, a))
    h = (out["Lp"] + out["Lm"] - 2 * out["L0"]) / eps ** 2
    g = (out["Lp"] - out["Lm"]) / (2 * eps)
    assert np.all(h == 0.25 * M)
    for i in range(n):
        assert out["c"][i] == _nearest_f32(Fraction(g[i]) / Fraction(0.25 * M))


# ------------------------------------------------------------------------------------
# update
# ------------------------------------------------------------------------------------
def _all_patterns_bits(M=8):
    rows = np.zeros((256, oracle.plane_bytes(M)), dtype=np.uint8)
    rows[:, 0] = np.arange(256, dtype=np.uint8)
    Z = np.array([[1.0 if (p >> j) & 1 else -1.0 for j in range(M)] for p in range(256)])
    return rows, Z


def test_update_brute_force_all_sign_patterns():
    # Over all 2^8 patterns sum_z z z^T = 256 I, so with c_z = z^T A theta (plain SPSA
    # weights, no 1/n) the update subtracts exactly eta * 256 * A theta.  A is a
    # non-diagonal symmetric matrix of small binary fractions; everything is exact.
    rng = np.random.Generator(np.random.PCG64(5))
    B = rng.integers(-8, 9, (8, 8)) / 16.0
    A = (B + B.T) / 2
    th0 = (rng.integers(-64, 65, 8) / 16.0).astype(np.float32)
    rows, Z = _all_patterns_bits()
    v = A @ th0.astype(np.float64)
    c = (Z @ v).astype(np.float32)
    assert np.array_equal(c.astype(np.float64), Z @ v)
    eta = 2.0 ** -10
    th = th0.copy()
    oracle.update(th, 0, 0, 0, c, eta, bits=rows)
    assert np.array_equal(th.astype(np.float64), th0 - eta * 256 * v)


def test_update_brute_force_preconditioned():
    # 1.5-SPSA weights on a quadratic with SPD A: c_z = (z^T A theta) / (z^T A z).  The
    # reference sum over all 256 patterns is done in exact rationals on the fp32 weights.
    rng = np.random.Generator(np.random.PCG64(6))
    B = rng.standard_normal((8, 8))
    A = B @ B.T + 8 * np.eye(8)
    th0 = rng.standard_normal(8).astype(np.float32)
    rows, Z = _all_patterns_bits()
    c = np.array([(z @ A @ th0) / (z @ A @ z) for z in Z], dtype=np.float32)
    eta = 1e-2
    th = th0.copy()
    oracle.update(th, 0, 0, 0, c, eta, bits=rows)
    e = Fraction(float(np.float32(eta)))
    for j in range(8):
        s = sum(Fraction(float(c[k])) * int(Z[k, j]) for k in range(256))
        exact = Fraction(float(th0[j])) - e * s
        assert th[j] == _nearest_f32(exact)


def test_update_single_probe_is_a_perturb():
    n = 1000
    rng = np.random.default_rng(8)
    eta = 2.0 ** -9
    for kind in ("f32", "bf16"):
        base = (rng.standard_normal(n) * 0.02).astype(np.float32)
        t0 = base if kind == "f32" else oracle.f32_to_bf16(base)
        a, b = t0.copy(), t0.copy()
        oracle.update(a, 384, 4, 6, [1.0], eta)
        oracle.perturb(b, 384, 4, 6, 0, -eta)
        assert np.array_equal(a, b), kind


def test_update_identity_cases():
    n = 777
    rng = np.random.default_rng(9)
    th0 = rng.standard_normal(n).astype(np.float32)
    c = rng.standard_normal(16).astype(np.float32)
    th = th0.copy()
    oracle.update(th, 0, 1, 1, c, 0.0)
    assert np.array_equal(th, th0)
    oracle.update(th, 0, 1, 1, np.zeros(16, np.float32), 0.5)
    assert np.array_equal(th, th0)


def test_update_bits_mode_equals_regenerate_ragged():
    n, npert = 1000, 13
    rng = np.random.default_rng(10)
    th0 = rng.standard_normal(n).astype(np.float32)
    c = rng.standard_normal(npert).astype(np.float32)
    a, b = th0.copy(), th0.copy()
    oracle.update(a, 128, 2, 3, c, 1e-2)
    oracle.update(b, 128, 2, 3, c, 1e-2, bits=oracle.gen_planes(2, 3, 0, npert, 128, n))
    assert np.array_equal(a, b)


def test_estimator_unbiased_and_variance_law():
    # c_i = (z_i^T v) / n: E[sum_i c_i z_i] = v and
    # E ||sum_i c_i z_i - v||^2 / ||v||^2 = (M - 1) / n for Rademacher probes -- the
    # exact form of the M / n_pert variance scaling.
    M, n, R = 64, 16, 600
    rng = np.random.Generator(np.random.PCG64(12))
    v = rng.standard_normal(M)
    ests, ratios = [], []
    for step in range(R):
        Z = np.stack([oracle.signs_from_plane(oracle.gen_plane(77, step, i, 0, M), M)
                      for i in range(n)])
        c = (Z @ v / n).astype(np.float32)
        s = oracle.probe_sums(M, 0, 77, step, c)
        ests.append(s)
        ratios.append(np.sum((s - v) ** 2) / np.sum(v ** 2))
    ratio = np.mean(ratios)
    assert abs(ratio / ((M - 1) / n) - 1) < 0.1, ratio
    bias = np.sum((np.mean(ests, axis=0) - v) ** 2) / np.sum(v ** 2)
    assert bias < 3 * (M - 1) / (n * R), bias


# ------------------------------------------------------------------------------------
# losses
# ------------------------------------------------------------------------------------
def test_quad_loss_exact_on_dyadic():
    th, a = _dyadic_quadratic(300, 13)
    exact = sum(Fraction(float(ai)) * Fraction(float(t)) ** 2 for ai, t in zip(a, th)) / 2
    assert oracle.quad_loss(th, a) == float(exact)
    hb = oracle.f32_to_bf16(th)
    exact_b = sum(Fraction(float(ai)) * Fraction(float(t)) ** 2
                  for ai, t in zip(a, oracle.bf16_to_f32(hb))) / 2
    assert oracle.quad_loss(hb, a) == float(exact_b)


def _torch_mlp_loss(p, X, y, d_hid, d_out):
    import torch.nn.functional as F
    d_in = X.shape[1]
    o = np.cumsum([0, d_hid * d_in, d_hid, d_out * d_hid, d_out])
    W1 = p[o[0]:o[1]].view(d_hid, d_in)
    b1 = p[o[1]:o[2]]
    W2 = p[o[2]:o[3]].view(d_out, d_hid)
    b2 = p[o[3]:o[4]]
    h = F.gelu(F.linear(X, W1, b1), approximate="none")
    return F.cross_entropy(F.linear(h, W2, b2), y)


def test_mlp_loss_matches_torch_fp64():
    cfg = CONFIGS["mlp"]
    e = cfg.extra
    X, y = gen.mlp_data(cfg)
    theta, _ = gen.theta_and_a(cfg)
    ref = _torch_mlp_loss(torch.from_numpy(theta.astype(np.float64)),
                          torch.from_numpy(X.astype(np.float64)), torch.from_numpy(y),
                          e["d_hid"], e["d_out"]).item()
    got = oracle.mlp_loss(theta, X, y, e["d_hid"], e["d_out"])
    assert abs(got - ref) <= 1e-12 * abs(ref)
    assert 0.2 < got < 2.0 and 0 < y.sum() < y.size  # both classes present


def test_mlp_central_difference_matches_directional_derivative():
    # g_i = (L(theta + eps z) - L(theta - eps z)) / (2 eps) = z^T grad L + O(eps^2).
    d_in, d_hid, d_out, B = 16, 32, 2, 8
    rng = np.random.Generator(np.random.PCG64(14))
    M = d_hid * d_in + d_hid + d_out * d_hid + d_out
    theta = rng.standard_normal(M) * 0.3
    X = rng.standard_normal((B, d_in))
    y = rng.integers(0, d_out, B)
    p = torch.tensor(theta, requires_grad=True)
    _torch_mlp_loss(p, torch.from_numpy(X), torch.from_numpy(y), d_hid, d_out).backward()
    grad = p.grad.numpy()
    for i in range(4):
        z = oracle.signs_from_plane(oracle.gen_plane(0, 0, i, 0, M), M)
        errs = []
        for eps in (2e-3, 1e-3):
            g = (oracle.mlp_loss(theta + eps * z, X, y, d_hid, d_out)
                 - oracle.mlp_loss(theta - eps * z, X, y, d_hid, d_out)) / (2 * eps)
            errs.append(abs(g - z @ grad))
        # second-order convergence: halving eps cuts the error ~4x
        assert errs[1] < errs[0] / 3 + 1e-12
        assert errs[1] < 1e-4 * (1 + abs(z @ grad))


# ------------------------------------------------------------------------------------
# whole step
# ------------------------------------------------------------------------------------
def test_tiny_config_closed_forms_and_descent():
    # On theta ~ N(0, 1) the perturbed values are exact except where theta +/- eps*z
    # rounds (binade crossings).  With L+/- = 1/2 sum a (theta +/- eps z + e+/-)^2 and
    # |e| <= u = ulp(|theta| + eps) on that set S only, expanding the squares gives
    #   |g - z^T A theta| <= sum_S a ((|theta| + eps) 2u + u^2) / (2 eps),
    #   |h - tr(A)|       <= sum_S a (2 (|theta| + eps) u + u^2) / eps^2,
    # plus the fp64 rounding of the three losses.  S is found with numpy's fp32 add.
    cfg = CONFIGS["tiny"]
    th0, a = gen.theta_and_a(cfg)
    th = th0.copy()
    a64 = a.astype(np.float64)
    trA = float(np.sum(a64))
    eps = float(np.float32(cfg.eps))
    lossf = lambda t: oracle.quad_loss(t, a)  # noqa: E731
    losses = [lossf(th)]
    for step in range(cfg.steps):
        thb = th.copy()
        t64 = thb.astype(np.float64)
        out = oracle.spsa_step(th, seed=cfg.seed, step=step, npert=cfg.npert, eps=cfg.eps,
                               eta=cfg.eta, delta=cfg.delta, loss_fn=lossf)
        h = (out["Lp"] + out["Lm"] - 2 * out["L0"]) / eps ** 2
        g = (out["Lp"] - out["Lm"]) / (2 * eps)
        u = np.spacing((np.abs(thb) + np.float32(eps)).astype(np.float32)).astype(np.float64)
        for i in range(cfg.npert):
            z = oracle.signs_from_plane(oracle.gen_plane(cfg.seed, step, i, 0, cfg.M), cfg.M)
            z32 = z.astype(np.float32)
            S = ((thb + np.float32(eps) * z32).astype(np.float64) != t64 + eps * z) | \
                ((thb - np.float32(eps) * z32).astype(np.float64) != t64 - eps * z)
            rnd = 4 * cfg.M * 2.0 ** -53 * (abs(out["Lp"][i]) + abs(out["Lm"][i]) + 2 * out["L0"])
            bg = np.sum(a64[S] * ((np.abs(t64[S]) + eps) * 2 * u[S] + u[S] ** 2)) / (2 * eps) \
                + rnd / (2 * eps)
            bh = np.sum(a64[S] * (2 * (np.abs(t64[S]) + eps) * u[S] + u[S] ** 2)) / eps ** 2 \
                + rnd / eps ** 2
            assert abs(g[i] - z @ (a64 * t64)) <= bg
            assert abs(h[i] - trA) <= bh
            assert bh < 1e-2 * trA          # the bound itself is tight enough to mean something
        losses.append(lossf(th))
    assert losses[-1] < losses[0]


def test_step_bits_mode_equals_regenerate_mode():
    cfg = CONFIGS["tiny"]
    th0, a = gen.theta_and_a(cfg)
    lossf = lambda t: oracle.quad_loss(t, a)  # noqa: E731
    x, y = th0.copy(), th0.copy()
    for step in range(2):
        oracle.spsa_step(x, seed=0, step=step, npert=cfg.npert, eps=cfg.eps, eta=cfg.eta,
                         delta=cfg.delta, loss_fn=lossf)
        bits = oracle.gen_planes(0, step, 0, cfg.npert, 0, cfg.M)
        oracle.spsa_step(y, seed=0, step=step, npert=cfg.npert, eps=cfg.eps, eta=cfg.eta,
                         delta=cfg.delta, loss_fn=lossf, bits=bits)
        assert np.array_equal(x, y)


def test_bf16_s4_drift_is_bounded():
    # In bf16 each +eps / -eps move rounds, so a restore need not land back on theta.  The
    # four-pass schedule (+eps, -eps, -eps, +eps) keeps every element within one bf16 ulp
    # of |theta| + eps of its start however many probes run (no random walk); the
    # three-pass schedule (+eps, -2 eps, +eps) does random-walk, which is why the path
    # uses four passes.
    n = 20000
    rng = np.random.Generator(np.random.PCG64(0))
    h0 = oracle.f32_to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    x0 = oracle.bf16_to_f32(h0).astype(np.float64)
    ulp = np.spacing((np.abs(x0) + 1e-3).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    h4, h3 = h0.copy(), h0.copy()
    for i in range(64):
        for s in (+1e-3, -1e-3, -1e-3, +1e-3):
            oracle.perturb(h4, 0, 0, 0, i, s)
        for s in (+1e-3, -2e-3, +1e-3):
            oracle.perturb(h3, 0, 0, 0, i, s)
    assert np.all(np.abs(oracle.bf16_to_f32(h4) - x0) <= ulp)
    assert np.max(np.abs(oracle.bf16_to_f32(h3) - x0) / ulp) > 4


# ------------------------------------------------------------------------------------
# the other weight forms of the pages
# ------------------------------------------------------------------------------------
def _losses(n, seed):
    L0, Lp, Lm = gen.synthetic_losses(seed, 0, n)
    return L0, Lp, Lm


def test_weights_power_one_is_the_preconditioned_form():
    L0, Lp, Lm = _losses(64, 1)
    a, _ = oracle.probe_weights(Lp, Lm, L0, 1e-3, 1e-6)
    b, _ = oracle.probe_weights_ex(Lp, Lm, L0, 1e-3, 1e-6, oracle.WEIGHTS_POWER, 1.0)
    c, _ = oracle.probe_weights_ex(Lp, Lm, L0, 1e-3, 1e-6, oracle.WEIGHTS_PRECOND)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_weights_power_special_exponents():
    L0, Lp, Lm = _losses(64, 2)
    eps = 1e-3
    g = (Lp - Lm) / (2 * eps)
    h = (Lp + Lm - 2 * L0) / eps ** 2
    d = np.maximum(np.abs(h), 1e-6)
    c0, _ = oracle.probe_weights_ex(Lp, Lm, L0, eps, 1e-6, oracle.WEIGHTS_POWER, 0.0)
    assert np.array_equal(c0, g.astype(np.float32))            # d^0 = 1: plain central difference
    c5, _ = oracle.probe_weights_ex(Lp, Lm, L0, eps, 1e-6, oracle.WEIGHTS_POWER, 0.5)
    ref = g / np.sqrt(d)                                        # library square root
    assert np.all(np.abs(c5 - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
    c01, _ = oracle.probe_weights_ex(Lp, Lm, L0, eps, 1e-6, oracle.WEIGHTS_POWER, 0.1)
    # shrinks high-curvature probes less than the full preconditioner does
    ratio = np.abs(c01 / g)
    assert np.all(np.abs(ratio - d ** -0.1) <= 1e-6 * d ** -0.1)


def test_weights_spsa_mean_on_quadratic_is_exact():
    # c_i = g_i / n with exact binary losses: (z_i^T A theta) / n, no clean pass read
    M, n = 4096, 16
    th0, a = _dyadic_quadratic(M, 17)
    th = th0.copy()
    out = oracle.spsa_step(th, seed=4, step=0, npert=n, eps=2.0 ** -8, eta=0.0, delta=1e-6,
                           loss_fn=lambda t: oracle.quad_loss(t, a))
    c, bad = oracle.probe_weights_ex(out["Lp"], out["Lm"], np.nan, 2.0 ** -8, 1e-6,
                                     oracle.WEIGHTS_SPSA_MEAN)
    assert bad == 0                                             # L0 is not read
    Z = np.stack([oracle.signs_from_plane(oracle.gen_plane(4, 0, i, 0, M), M) for i in range(n)])
    g = Z @ (a.astype(np.float64) * th0.astype(np.float64))
    for i in range(n):
        assert c[i] == _nearest_f32(Fraction(g[i]) / n)
