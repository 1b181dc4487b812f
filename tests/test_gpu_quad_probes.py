"""zo_quad_loss_probes: both losses of several probes of the quadratic workload with each
probe applied while theta is read.  Each loss must equal zo_perturb followed by zo_quad_loss
bit for bit (the library's own chain, itself pinned to the oracle by test_gpu_parity), theta
must come back untouched, and the values must sit within the fp64 summation bound of the
oracle's perturb followed by its loss."""
import numpy as np
import pytest
import torch

import forward_only_amd as zo
import oracle
from gpu_util import bf16_bits, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

SEED = 0x5EED0F0A


@pytest.fixture(scope="module")
def ctx():
    c = zo.zo_init(SEED)
    yield c
    c.close()


def _problem(kind, n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 0.5).astype(np.float32)
    a = np.power(10.0, rng.uniform(-2, 2, n)).astype(np.float32)
    h = x if kind == "f32" else oracle.f32_to_bf16(x)
    return h, a


def _dev(kind, h):
    return to_dev_f32(h) if kind == "f32" else to_dev_bf16(h)


def _host(kind, t):
    return t.cpu().numpy() if kind == "f32" else bf16_bits(t)


# The fused pass takes four probes at a time and 2048-param chunks per wave: probe counts
# below, at and above one pass and several passes; sizes below, at and above one chunk, a
# ragged tail, more chunks than waves; a non-zero global offset.
CASES = [("f32", 1, 0, 1), ("f32", 2047, 0, 4), ("bf16", 2049, 128, 5), ("f32", 4096 + 77, 0, 3),
         ("bf16", 1_000_003, 128 * 9, 9), ("f32", 8_388_608 + 4096 * 2 + 13, 0, 4),
         ("bf16", 16_777_293, 0, 2)]


@pytest.mark.parametrize("kind,n,offset,nprobes", CASES)
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_fused_losses_equal_perturb_then_loss(ctx, kind, n, offset, nprobes, mode):
    h, a = _problem(kind, n, seed=n + nprobes)
    t, ad = _dev(kind, h), to_dev_f32(a)
    step, probe0, alpha = 7, 11, 1e-3
    rows = zo.zo_gen_probes(ctx, step, probe0, nprobes, offset, n) if mode == "bits" else None
    clean = torch.full((1,), np.nan, dtype=torch.float64, device="cuda")
    lp, lm = zo.zo_quad_loss_probes(ctx, t, ad, offset, step, probe0, nprobes, alpha, bits=rows,
                                    out_clean=clean)
    gp, gm = lp.cpu().numpy(), lm.cpu().numpy()
    assert np.array_equal(_host(kind, t), h)                 # theta is not written
    assert clean.item() == zo.zo_quad_loss(ctx, t, ad).item()   # the clean loss, same bits
    for i in range(nprobes):
        row = None if rows is None else rows[i]
        for sign, got in ((+1.0, gp[i]), (-1.0, gm[i])):
            w = t.clone()
            zo.zo_perturb(ctx, w, offset, step, probe0 + i, sign * alpha, bits=row)
            ref = zo.zo_quad_loss(ctx, w, ad).item()
            assert got == ref, (i, sign, got, ref)
    if n > 1:
        assert len(set(gp.tolist()) | set(gm.tolist())) == 2 * nprobes   # all distinct


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_fused_losses_against_the_oracle(ctx, kind):
    n, offset, nprobes, step, probe0, alpha = 50_001, 128 * 3, 5, 2, 4, 2.0 ** -10
    h, a = _problem(kind, n, seed=3)
    lp, lm = zo.zo_quad_loss_probes(ctx, _dev(kind, h), to_dev_f32(a), offset, step, probe0,
                                    nprobes, alpha)
    for i in range(nprobes):
        for sign, got in ((+1.0, lp[i].item()), (-1.0, lm[i].item())):
            w = h.copy()
            oracle.perturb(w, offset, SEED, step, probe0 + i, sign * alpha)
            ref = oracle.quad_loss(w, a)
            # fp64 recursive-summation bound on n positive terms, with margin
            assert abs(got - ref) <= 4 * n * 2.0 ** -53 * abs(ref), (i, sign, got, ref)


def test_fused_losses_argument_checks(ctx):
    t = torch.zeros(1024, dtype=torch.float32, device="cuda")
    a = torch.ones(1024, dtype=torch.float32, device="cuda")
    op = torch.empty(4, dtype=torch.float64, device="cuda")
    om = torch.empty(4, dtype=torch.float64, device="cuda")
    L = zo._lib.lib()
    oc = torch.full((1,), np.nan, dtype=torch.float64, device="cuda")
    args = lambda off=0, bits=None, plus=op.data_ptr(), minus=om.data_ptr(), p0=0, k=4, clean=None: (  # noqa: E731
        L.zo_quad_loss_probes(ctx.handle, t.data_ptr(), zo.ZO_FP32, a.data_ptr(), off, 1024, 1,
                              p0, k, 1e-3, bits, plus, minus, clean, None))
    assert args() == zo.ZO_OK
    assert args(off=64) == zo.ZO_EINVAL                       # offset not a block multiple
    assert args(bits=t.data_ptr() + 4) == zo.ZO_EINVAL        # misaligned rows
    assert args(plus=None) == zo.ZO_EINVAL
    assert args(minus=None) == zo.ZO_EINVAL
    assert args(p0=0xFFFFFFFE, k=4) == zo.ZO_EINVAL           # probe indices wrap
    assert args(plus=None, minus=None, k=0) == zo.ZO_OK       # no probes: nothing to do
    assert args(plus=None, minus=None, k=0, clean=oc.data_ptr()) == zo.ZO_OK   # clean only
    torch.cuda.synchronize()
    assert oc.item() == zo.zo_quad_loss(ctx, t, a).item() == 0.0     # theta is zero
    with pytest.raises(ValueError):
        zo.zo_quad_loss_probes(ctx, t, a[:10], 0, 1, 0, 2, 1e-3)
    with pytest.raises(ValueError):
        zo.zo_quad_loss_probes(ctx, t, a, 0, 1, 0, 5, 1e-3, out_plus=op)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_fused_step_equals_s4_step_on_exact_inputs(ctx, kind):
    """Where every move is exact (dyadic theta and eps), the fused step (losses at theta +/-
    eps z_i from the clean theta, no passes; the clean loss from the first fused pass) and
    the four-pass S4 step visit the same points: equal losses, weights and updated theta,
    bit for bit."""
    from forward_only_amd.step import spsa_step, spsa_step_fused
    from workloads import gen
    n, npert, step = 70_001, 9, 4
    if kind == "f32":
        x, eps = gen.dyadic_theta(n, seed=5, frac_bits=12, max_abs_log2=4), 2.0 ** -10
    else:
        x, eps = gen.dyadic_theta(n, seed=5, frac_bits=4, max_abs_log2=3), 2.0 ** -4
    h = x if kind == "f32" else oracle.f32_to_bf16(x)
    a = np.power(10.0, np.random.default_rng(6).uniform(-1, 1, n)).astype(np.float32)
    ad = to_dev_f32(a)
    t4, tf = _dev(kind, h), _dev(kind, h)
    quad = lambda th, out: zo.zo_quad_loss(ctx, th, ad, out=out)   # noqa: E731
    r4 = spsa_step(ctx, t4, step=step, npert=npert, eps=eps, eta=1e-2, delta=1e-6, loss=quad,
                   schedule="S4")
    rf = spsa_step_fused(
        ctx, tf, step=step, npert=npert, eps=eps, eta=1e-2, delta=1e-6,
        loss_at=lambda probe, alpha, row, out: zo.zo_quad_loss(ctx, tf, ad, out=out),
        loss_probes_at=lambda p0, k, alpha, rows, op, om, oc: zo.zo_quad_loss_probes(
            ctx, tf, ad, 0, step, p0, k, alpha, bits=rows, out_plus=op, out_minus=om,
            out_clean=oc), probes_give_clean=True)
    for key in ("L0", "Lp", "Lm", "c"):
        assert np.array_equal(r4[key].cpu().numpy(), rf[key].cpu().numpy()), key
    assert np.array_equal(_host(kind, t4), _host(kind, tf))
    assert not np.array_equal(_host(kind, tf), h)            # the update moved theta
