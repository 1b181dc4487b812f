"""The MLP loss on MFMA and its perturbation-fused variant, against the fp64 oracle.

Tolerance for the loss: 1e-5 relative.  The GEMM accumulates K = d_in fp32 products per
hidden unit (typical error ~ sqrt(K) * 2^-24 * |h|, ~1e-6 relative at K = 768) and the
loss averages ~batch * d_hid such terms, so the observed error is far below this; a
dropped bias, a wrong activation or a transposed operand moves the loss by >= 1e-3.
The fused variant is held to bit-equality with perturb-in-place-then-forward.
"""
import numpy as np
import pytest
import torch

import forward_only_amd as zo
import oracle
from forward_only_amd.step import spsa_step_fused
from gpu_util import to_dev_f32, weight_bound
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu

# 16 x 16 tiles where the batch or the hidden width is not a multiple of 32 (the batch, the
# width, or both), 32 x 32 tiles otherwise; K below one 16-k group's multiple of the staging,
# with a ragged group count, and the workload's shape
SHAPES = [(16, 16, 16, 2), (32, 48, 64, 3), (48, 32, 128, 16), (64, 208, 96, 16),
          (64, 32, 48, 5), (128, 768, 3072, 2)]


@pytest.fixture(scope="module")
def ctx():
    c = zo.zo_init(11)
    yield c
    c.close()


def _problem(batch, d_in, d_hid, d_out, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    M = d_hid * d_in + d_hid + d_out * d_hid + d_out
    theta = (rng.standard_normal(M) * 0.02).astype(np.float32)
    X = rng.standard_normal((batch, d_in)).astype(np.float32)
    y = rng.integers(0, d_out, batch).astype(np.int64)
    return theta, X, y


def _dev(theta, X, y):
    return to_dev_f32(theta), to_dev_f32(X), torch.from_numpy(y).cuda()


@pytest.mark.parametrize("shape", SHAPES)
def test_mlp_loss_matches_oracle(ctx, shape):
    batch, d_in, d_hid, d_out = shape
    theta, X, y = _problem(*shape, seed=sum(shape))
    t, x, yl = _dev(theta, X, y)
    got = zo.zo_mlp_loss(ctx, t, x, yl, d_hid, d_out).item()
    ref = oracle.mlp_loss(theta, X, y, d_hid, d_out)
    assert abs(got - ref) <= 1e-5 * abs(ref), (got, ref)
    again = zo.zo_mlp_loss(ctx, t, x, yl, d_hid, d_out).item()
    assert again == got                                   # deterministic


def test_mlp_config_loss(ctx):
    cfg = CONFIGS["mlp"]
    e = cfg.extra
    theta, _ = gen.theta_and_a(cfg)
    X, y = gen.mlp_data(cfg)
    got = zo.zo_mlp_loss(ctx, to_dev_f32(theta), to_dev_f32(X), torch.from_numpy(y).cuda(),
                         e["d_hid"], e["d_out"]).item()
    ref = oracle.mlp_loss(theta, X, y, e["d_hid"], e["d_out"])
    assert abs(got - ref) <= 1e-5 * abs(ref), (got, ref)


@pytest.mark.parametrize("shape", [(16, 16, 16, 2), (32, 48, 64, 3), (64, 208, 96, 16),
                                   (128, 768, 3072, 2)])
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_fused_perturbation_equals_perturb_then_forward(ctx, shape, mode):
    batch, d_in, d_hid, d_out = shape
    theta, X, y = _problem(*shape, seed=7 + sum(shape))
    t, x, yl = _dev(theta, X, y)
    M = theta.size
    for probe, alpha in ((0, 1e-3), (3, -1e-3), (5, 2.0 ** -7)):
        bits = zo.zo_gen_probes(ctx, 2, probe, 1, 0, M)[0] if mode == "bits" else None
        fused = zo.zo_mlp_loss_perturbed(ctx, t, 0, 2, probe, alpha, x, yl, d_hid, d_out,
                                         bits=bits).item()
        moved = t.clone()
        zo.zo_perturb(ctx, moved, 0, 2, probe, alpha, bits)
        direct = zo.zo_mlp_loss(ctx, moved, x, yl, d_hid, d_out).item()
        assert fused == direct, (probe, alpha, fused, direct)
        # and the oracle at the perturbed point
        h = theta.copy()
        oracle.perturb(h, 0, 11, 2, probe, alpha)
        ref = oracle.mlp_loss(h, X, y, d_hid, d_out)
        assert abs(fused - ref) <= 1e-5 * abs(ref)
    assert np.array_equal(t.cpu().numpy(), theta)          # parameters untouched


@pytest.mark.parametrize("shape", [(16, 16, 16, 2), (32, 48, 64, 3), (48, 144, 128, 16),
                                   (64, 208, 96, 16), (64, 32, 48, 5), (128, 768, 3072, 2)])
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_pair_equals_two_fused_calls(ctx, shape, mode):
    """zo_mlp_loss_pair gives exactly the two single fused losses (+alpha, -alpha), in
    both bit modes and with K not a multiple of the kernel's 128-wide stages; the
    parameters stay untouched."""
    batch, d_in, d_hid, d_out = shape
    theta, X, y = _problem(*shape, seed=31 + sum(shape))
    t, x, yl = _dev(theta, X, y)
    M = theta.size
    for probe, alpha in ((0, 1e-3), (6, 2.0 ** -7), (9, -3e-3)):
        bits = zo.zo_gen_probes(ctx, 4, probe, 1, 0, M)[0] if mode == "bits" else None
        lp, lm = zo.zo_mlp_loss_pair(ctx, t, 0, 4, probe, alpha, x, yl, d_hid, d_out,
                                     bits=bits)
        sp = zo.zo_mlp_loss_perturbed(ctx, t, 0, 4, probe, alpha, x, yl, d_hid, d_out,
                                      bits=bits).item()
        sm = zo.zo_mlp_loss_perturbed(ctx, t, 0, 4, probe, -alpha, x, yl, d_hid, d_out,
                                      bits=bits).item()
        assert (lp.item(), lm.item()) == (sp, sm), (probe, alpha, lp.item(), lm.item(), sp, sm)
    assert np.array_equal(t.cpu().numpy(), theta)


@pytest.mark.parametrize("shape", [(16, 16, 16, 2), (32, 48, 64, 3), (48, 144, 128, 16),
                                   (64, 208, 96, 16), (64, 32, 48, 5), (128, 768, 3072, 2)])
@pytest.mark.parametrize("mode", ["regen", "bits"])
@pytest.mark.parametrize("nprobes", [1, 3, 8, 13, 21, 70])
def test_probes_equal_pairs(ctx, shape, mode, nprobes):
    """zo_mlp_loss_probes gives, for every probe of the batch, exactly the losses of
    zo_mlp_loss_pair (70 probes run as launch sequences of 64, 4 and 2 probes, 21 as 16, 4
    and 1, 13 as 8, 4 and 1, each with several probes per wave), and with out_clean exactly
    zo_mlp_loss from the first sequence's extra wave group; parameters untouched."""
    batch, d_in, d_hid, d_out = shape
    theta, X, y = _problem(*shape, seed=57 + sum(shape) + nprobes)
    t, x, yl = _dev(theta, X, y)
    M = theta.size
    probe0, step, alpha = 5, 6, 1e-3
    rows = zo.zo_gen_probes(ctx, step, probe0, nprobes, 0, M) if mode == "bits" else None
    clean = torch.full((1,), np.nan, dtype=torch.float64, device="cuda")
    lp, lm = zo.zo_mlp_loss_probes(ctx, t, 0, step, probe0, nprobes, alpha, x, yl, d_hid, d_out,
                                   bits=rows, out_clean=clean)
    gp, gm = lp.cpu().numpy(), lm.cpu().numpy()
    assert clean.item() == zo.zo_mlp_loss(ctx, t, x, yl, d_hid, d_out).item()
    for i in range(nprobes):
        sp, sm = zo.zo_mlp_loss_pair(ctx, t, 0, step, probe0 + i, alpha, x, yl, d_hid, d_out,
                                     bits=None if rows is None else rows[i])
        assert (gp[i], gm[i]) == (sp.item(), sm.item()), (i, gp[i], gm[i], sp.item(), sm.item())
    assert len(set(gp.tolist())) == nprobes                 # every probe its own loss
    assert np.array_equal(t.cpu().numpy(), theta)


def test_probes_argument_checks(ctx):
    theta, X, y = _problem(16, 16, 16, 2, seed=1)
    t, x, yl = _dev(theta, X, y)
    L = zo._lib.lib()
    # one slot (partial logits and row losses of one loss) per sign and probe of the first
    # launch sequence (64 probes), plus one for the clean loss; the pair call holds two
    unit = zo.zo_mlp_workspace_bytes(16, 16, 16, 2) // 2
    need = zo.zo_mlp_probes_workspace_bytes(16, 16, 16, 2, 5)
    assert need == 11 * unit
    assert zo.zo_mlp_probes_workspace_bytes(16, 16, 16, 2, 64) == 129 * unit
    assert zo.zo_mlp_probes_workspace_bytes(16, 16, 16, 2, 100) == 129 * unit   # 64 per launch
    assert zo.zo_mlp_probes_workspace_bytes(16, 16, 16, 2, 0) == unit
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.full((12,), np.nan, dtype=torch.float64, device="cuda")
    args = lambda n, minus, wbytes=need, probe0=0, clean=None: L.zo_mlp_loss_probes(  # noqa: E731
        ctx.handle, t.data_ptr(), 0, 0, probe0, n, 1e-3, None, x.data_ptr(), yl.data_ptr(), 16,
        16, 16, 2, ws.data_ptr(), wbytes, out.data_ptr(), minus, clean, None)
    assert args(5, None) == zo.ZO_EINVAL                                  # no -alpha outputs
    assert args(5, out.data_ptr() + 40, wbytes=need - 8) == zo.ZO_EINVAL  # workspace
    assert args(5, out.data_ptr() + 40, probe0=2 ** 32 - 3) == zo.ZO_EINVAL  # probe wraps
    assert args(0, None) == zo.ZO_OK                                      # empty
    assert args(5, out.data_ptr() + 40) == zo.ZO_OK
    assert args(0, None, wbytes=unit, clean=out.data_ptr() + 80) == zo.ZO_OK   # clean only
    assert args(0, None, wbytes=unit - 8, clean=out.data_ptr() + 80) == zo.ZO_EINVAL
    torch.cuda.synchronize()
    assert out[10].item() == zo.zo_mlp_loss(ctx, t, x, yl, 16, 2).item()
    with pytest.raises(ValueError):
        zo.zo_mlp_loss_probes(ctx, t, 0, 0, 0, 5, 1e-3, x, yl, 16, 2,
                              bits=zo.zo_gen_probes(ctx, 0, 0, 4, 0, theta.size))  # 4 rows for 5


def test_pair_argument_checks(ctx):
    theta, X, y = _problem(16, 16, 16, 2, seed=1)
    t, x, yl = _dev(theta, X, y)
    M = theta.size
    L = zo._lib.lib()
    ws = torch.empty(zo.zo_mlp_workspace_bytes(16, 16, 16, 2), dtype=torch.uint8, device="cuda")
    out = torch.empty(2, dtype=torch.float64, device="cuda")
    args = lambda minus, offset=0, wbytes=ws.numel(): L.zo_mlp_loss_pair(  # noqa: E731
        ctx.handle, t.data_ptr(), offset, 0, 0, 1e-3, None, x.data_ptr(), yl.data_ptr(), 16, 16,
        16, 2, ws.data_ptr(), wbytes, out.data_ptr(), minus, None)
    assert args(None) == zo.ZO_EINVAL                                    # no -alpha output
    assert args(out.data_ptr() + 8, offset=64) == zo.ZO_EINVAL           # offset % 128 != 0
    assert args(out.data_ptr() + 8, wbytes=ws.numel() // 2 - 8) == zo.ZO_EINVAL  # workspace
    assert args(out.data_ptr() + 8) == zo.ZO_OK
    torch.cuda.synchronize()
    assert M == t.numel()


def test_mlp_argument_checks(ctx):
    theta8, X8, y8 = _problem(16, 8, 16, 2, seed=2)
    with pytest.raises(zo.ZOError) as e:
        zo.zo_mlp_loss(ctx, *_dev(theta8, X8, y8), 16, 2)              # d_in not a multiple of 16
    assert e.value.status == zo.ZO_EINVAL
    theta17, X17, y17 = _problem(16, 16, 16, 17, seed=3)
    with pytest.raises(zo.ZOError):
        zo.zo_mlp_loss(ctx, *_dev(theta17, X17, y17), 16, 17)          # more than 16 classes
    theta, X, y = _problem(16, 16, 16, 2, seed=1)
    t, x, yl = _dev(theta, X, y)
    ws = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(zo.ZOError):
        zo.zo_mlp_loss(ctx, t, x, yl, 16, 2, workspace=ws)             # workspace too small


def test_pair_step_equals_single_call_step():
    """A whole MLP-workload step with paired forwards, one with all probes in one batched
    call, and one whose batched call also gives the clean loss, equal the step with single
    fused forwards bit for bit: losses, weights and the updated parameters."""
    cfg = CONFIGS["mlp"]
    e = cfg.extra
    npert, step = 32, 3
    theta, _ = gen.theta_and_a(cfg)
    X, y = gen.mlp_data(cfg)
    x, yl = to_dev_f32(X), torch.from_numpy(y).cuda()
    results = []
    for form in ("single", "paired", "batched", "batched+clean"):
        local = zo.zo_init(cfg.seed)
        t = to_dev_f32(theta)
        ws = torch.empty(zo.zo_mlp_probes_workspace_bytes(e["batch"], e["d_in"], e["d_hid"],
                                                          e["d_out"], npert), dtype=torch.uint8,
                         device="cuda")

        def loss_at(probe, alpha, row, out):
            if probe is None:
                zo.zo_mlp_loss(local, t, x, yl, e["d_hid"], e["d_out"], workspace=ws, out=out)
            else:
                zo.zo_mlp_loss_perturbed(local, t, 0, step, probe, alpha, x, yl, e["d_hid"],
                                         e["d_out"], bits=row, workspace=ws, out=out)

        def pair_at(probe, alpha, row, op, om):
            zo.zo_mlp_loss_pair(local, t, 0, step, probe, alpha, x, yl, e["d_hid"], e["d_out"],
                                bits=row, workspace=ws, out_plus=op, out_minus=om)

        def probes_at(probe0, n, alpha, rows, op, om, oc=None):
            zo.zo_mlp_loss_probes(local, t, 0, step, probe0, n, alpha, x, yl, e["d_hid"],
                                  e["d_out"], bits=rows, workspace=ws, out_plus=op, out_minus=om,
                                  out_clean=oc)

        out = spsa_step_fused(local, t, step=step, npert=npert, eps=cfg.eps, eta=cfg.eta,
                              delta=cfg.delta, loss_at=loss_at,
                              loss_pair_at=pair_at if form == "paired" else None,
                              loss_probes_at=probes_at if form.startswith("batched") else None,
                              probes_give_clean=form == "batched+clean")
        results.append((out["L0"].cpu().numpy(), out["Lp"].cpu().numpy(), out["Lm"].cpu().numpy(),
                        out["c"].cpu().numpy(), t.cpu().numpy()))
        local.close()
    for other in results[1:]:
        for a, b in zip(results[0], other):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["bits", "regen"])
def test_mlp_config_fused_step(ctx, mode):
    """One step of the MLP workload at its probe count (n_pert = 64) with the fused forward,
    each side on its own from the seeded parameters: the oracle evaluates L(theta +/- eps
    z_i) by its own perturb and fp64 forward.  Losses agree within the loss tolerance; since
    the weight arithmetic is identical on both sides, the weights must lie within the bound
    implied by the measured loss differences, which must be finite for every probe (the
    smallest curvature |h_i| of this workload's 64 probes is ~10 against a loss-difference
    term of ~0.3); theta within the update tolerance plus eta * sum of those bounds; the
    GPU's parameters are untouched by the 64 x 2 perturbed forwards (only the update moves
    them).  The GPU side runs the benchmark's call: one batched call for all 64 probes'
    losses and the clean loss."""
    cfg = CONFIGS["mlp"]
    e = cfg.extra
    npert, step = cfg.npert, 0
    local = zo.zo_init(cfg.seed)
    theta, _ = gen.theta_and_a(cfg)
    X, y = gen.mlp_data(cfg)
    t, x, yl = to_dev_f32(theta), to_dev_f32(X), torch.from_numpy(y).cuda()
    ws = torch.empty(zo.zo_mlp_probes_workspace_bytes(e["batch"], e["d_in"], e["d_hid"],
                                                      e["d_out"], npert),
                     dtype=torch.uint8, device="cuda")

    def probes_at(probe0, n, alpha, rows, op, om, oc):
        zo.zo_mlp_loss_probes(local, t, 0, step, probe0, n, alpha, x, yl, e["d_hid"],
                              e["d_out"], bits=rows, workspace=ws, out_plus=op, out_minus=om,
                              out_clean=oc)

    bits = zo.zo_gen_probes(local, step, 0, npert, 0, cfg.M) if mode == "bits" else None
    out = spsa_step_fused(local, t, step=step, npert=npert, eps=cfg.eps, eta=cfg.eta,
                          delta=cfg.delta, bits=bits, loss_probes_at=probes_at,
                          probes_give_clean=True)
    a = float(np.float32(cfg.eps))
    lossf = lambda p: oracle.mlp_loss(p, X, y, e["d_hid"], e["d_out"])  # noqa: E731
    L0 = lossf(theta)
    Lp, Lm = np.zeros(npert), np.zeros(npert)
    for i in range(npert):
        for sgn, dst in ((+1, Lp), (-1, Lm)):
            p = theta.copy()
            oracle.perturb(p, 0, cfg.seed, step, i, sgn * a)
            dst[i] = lossf(p)
    h = theta.copy()
    res = oracle.spsa_step(h, seed=cfg.seed, step=step, npert=npert, eps=cfg.eps, eta=cfg.eta,
                           delta=cfg.delta, losses=(L0, Lp, Lm), schedule="none")
    gL0, gLp, gLm = out["L0"].item(), out["Lp"].cpu().numpy(), out["Lm"].cpu().numpy()
    dL = max(abs(gL0 - L0), np.max(np.abs(gLp - Lp)), np.max(np.abs(gLm - Lm)))
    assert dL <= 1e-5 * L0, dL
    bound = weight_bound(Lp, Lm, L0, dL * (1 + 1e-12), a, cfg.delta, res["c"])
    c = out["c"].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(bound)), (dL, bound)
    assert np.all(np.abs(c - res["c"]) <= bound), (c, res["c"], bound)
    got = t.cpu().numpy()
    scale = np.maximum(np.abs(h.astype(np.float64)),
                       float(np.float32(cfg.eta)) * float(np.sum(np.abs(res["c"]))))
    extra = float(np.float32(cfg.eta)) * float(np.sum(bound))
    assert np.all(np.abs(got.astype(np.float64) - h) <= 1e-5 * scale + extra)
    local.close()
