"""The low-rank-plus-diagonal quadratic on the GPU: the loss kernel against the fp64
oracle, and one full workload step each side on its own."""
import numpy as np
import pytest
import torch

import forward_only_amd as zo
import oracle
from forward_only_amd.step import spsa_step
from gpu_util import to_dev_bf16, to_dev_f32, weight_bound
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = zo.zo_init(0)
    yield c
    c.close()


def _bound(theta, a, U):
    """|L_gpu - L_oracle| bound: fp64 sums of n terms on both sides (recursive-summation
    bound), the dot products' errors amplified by squaring (2 |d| dd)."""
    t = oracle.bf16_to_f32(theta).astype(np.float64) if theta.dtype == np.uint16 else theta.astype(np.float64)
    n = t.size
    u = 2 * (n + 4) * 2.0 ** -53
    diag = 0.5 * np.sum(np.abs(a.astype(np.float64) * t * t))
    dots = U.astype(np.float64) @ t
    absd = np.abs(U.astype(np.float64)) @ np.abs(t)
    return 1.01 * (u * diag + np.sum(np.abs(dots) * u * absd) + u * 0.5 * np.sum(dots ** 2))


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("n,r", [(1, 1), (4096, 0), (4096, 3), (1_000_003, 4), (1 << 20, 16)])
def test_lowrank_loss(ctx, kind, n, r):
    rng = np.random.default_rng(n + r)
    x = (rng.standard_normal(n) * 0.5).astype(np.float32)
    theta = x if kind == "f32" else oracle.f32_to_bf16(x)
    a = np.power(10.0, rng.uniform(-2, 2, n)).astype(np.float32)
    U = (rng.standard_normal((r, n)) * 0.1).astype(np.float32)
    t = to_dev_f32(theta) if kind == "f32" else to_dev_bf16(theta)
    got = zo.zo_lowrank_quad_loss(ctx, t, to_dev_f32(a), to_dev_f32(U)).item()
    ref = oracle.lowrank_quad_loss(theta, a, U)
    assert abs(got - ref) <= _bound(theta, a, U), (got, ref)
    assert zo.zo_lowrank_quad_loss(ctx, t, to_dev_f32(a), to_dev_f32(U)).item() == got


def test_lowrank_rank_limit(ctx):
    t = torch.zeros(256, device="cuda")
    with pytest.raises(zo.ZOError) as e:
        zo.zo_lowrank_quad_loss(ctx, t, torch.ones(256, device="cuda"),
                                torch.zeros((17, 256), device="cuda"))
    assert e.value.status == zo.ZO_EUNSUPPORTED


@pytest.mark.parametrize("mode", [zo.ZO_WEIGHTS_PRECOND, zo.ZO_WEIGHTS_SPSA_MEAN])
def test_lowrank_workload_step(ctx, mode):
    """One step of the low-rank workload (two-pass schedule), each side on its own from the
    seeded problem: losses within the fp64 bound, weights within the bound those loss
    differences imply, theta within the update tolerance plus eta * sum of the bounds."""
    cfg = CONFIGS["lowrank"]
    theta, a, U = gen.lowrank_problem(cfg)
    local = zo.zo_init(cfg.seed)
    t, ad, Ud = to_dev_f32(theta), to_dev_f32(a), to_dev_f32(U)
    lossf = lambda x, o: zo.zo_lowrank_quad_loss(local, x, ad, Ud, out=o)  # noqa: E731
    out = spsa_step(local, t, step=0, npert=cfg.npert, eps=cfg.eps, eta=0.0, delta=cfg.delta,
                    loss=lossf, schedule="S2f")
    eps = float(np.float32(cfg.eps))
    eta = 1e-6 if mode == zo.ZO_WEIGHTS_SPSA_MEAN else 1e-2
    c = zo.zo_probe_weights_ex(local, out["Lp"], out["Lm"], out["L0"], eps, cfg.delta, mode)
    zo.zo_update(local, t, 0, 0, c, eta)
    h = theta.copy()
    res = oracle.spsa_step(h, seed=cfg.seed, step=0, npert=cfg.npert, eps=cfg.eps, eta=0.0,
                           delta=cfg.delta, loss_fn=lambda x: oracle.lowrank_quad_loss(x, a, U),
                           schedule="S2f")
    cref, _ = oracle.probe_weights_ex(res["Lp"], res["Lm"], res["L0"], eps, cfg.delta, mode)
    oracle.update(h, 0, cfg.seed, 0, cref, eta)
    dL = max(abs(out["L0"].item() - res["L0"]),
             np.max(np.abs(out["Lp"].cpu().numpy() - res["Lp"])),
             np.max(np.abs(out["Lm"].cpu().numpy() - res["Lm"])))
    assert dL <= _bound(theta, a, U) * 4
    cg = c.cpu().numpy().astype(np.float64)
    if mode == zo.ZO_WEIGHTS_SPSA_MEAN:
        bound = dL / eps / cfg.npert + 2 * np.spacing(np.abs(cref))
    else:
        bound = weight_bound(res["Lp"], res["Lm"], res["L0"], dL * (1 + 1e-12), eps,
                             cfg.delta, cref)
    assert np.all(np.abs(cg - cref) <= bound)
    got = t.cpu().numpy().astype(np.float64)
    scale = np.maximum(np.abs(h.astype(np.float64)), eta * float(np.sum(np.abs(cref))))
    assert np.all(np.abs(got - h) <= 1e-5 * scale + eta * float(np.sum(bound)))
    local.close()
