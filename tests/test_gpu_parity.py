"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by element.

Sizes span several 8192-param chunks plus ragged tails; offsets, both sign modes (probes
regenerated from the counter, or read from stored rows), special values and the argument
checks are covered.  Tolerances: see tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import forward_only_amd as zo
from forward_only_amd import placement
import oracle
from forward_only_amd.step import spsa_step
from gpu_util import (assert_bf16_within_ulp, assert_f32_update_close, assert_same_bits_or_nan,
                      bf16_bits, to_dev_bf16, to_dev_f32, weight_bound)
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu

SEED = 0x0123456789ABCDEF


@pytest.fixture(scope="module")
def ctx():
    c = zo.zo_init(SEED)
    yield c
    c.close()


def _theta(kind, n, seed, scale=1.0, specials=False):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    if specials and n >= 12:
        x[:12] = [np.nan, np.inf, -np.inf, 1e-40, -1e-40, 0.0, -0.0, 3e38, -3e38,
                  1.17549435e-38, 2.0 ** -130, 1e-3]
    if kind == "f32":
        return x
    return oracle.f32_to_bf16(x)


def _dev(kind, h):
    return to_dev_f32(h) if kind == "f32" else to_dev_bf16(h)


def _host(kind, t):
    return t.cpu().numpy() if kind == "f32" else bf16_bits(t)


# ------------------------------------------------------------------------------------
# probe planes
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("n,offset,step,probe0,nprobes", [
    (4096, 0, 0, 0, 16), (1, 0, 3, 5, 2), (129, 128, 1, 0, 3), (1000, 128 * 77, 9, 100, 7),
    (8192 * 3 + 1000, 0, 0xFFFFFFFF, 0xFFFFFFF0, 4), (77777, (1 << 40) * 128, 2, 1, 2)])
def test_gen_probes_bit_exact(ctx, n, offset, step, probe0, nprobes):
    got = zo.zo_gen_probes(ctx, step, probe0, nprobes, offset, n).cpu().numpy()
    ref = oracle.gen_planes(SEED, step, probe0, nprobes, offset, n)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_gen_probes_plane_125m(ctx):
    n = 125_000_000
    got = zo.zo_gen_probes(ctx, 4, 17, 1, 0, n).cpu().numpy()[0]
    ref = oracle.gen_plane(SEED, 4, 17, 0, n)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------------------------
# perturb
# ------------------------------------------------------------------------------------
# 8192 params form one chunk of the streaming kernel, and the chunks are split into eight
# per-XCD ranges: the cases cover no whole chunk, 1, 3, 7, 9 and 13 chunks (ranges left
# empty, a grid rounded up to a multiple of 8), 512, and 8205 chunks (more than the 8192
# waves of the grid, not a multiple of 8), each with and without a ragged tail.
PERTURB_CASES = [(4096, 0), (8192, 128), (8192 * 3 + 1000, 0), (1, 256), (127, 0),
                 (8192 * 7, 128 * 3), (8192 * 9 + 8191, 128 * 5), (8192 * 13 + 5, 0),
                 (1 << 22, 0), (8192 * 8205 + 77, 128)]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("n,offset", PERTURB_CASES)
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_perturb_bit_exact(ctx, kind, n, offset, mode):
    step, probe, alpha = 5, 11, (2.0 ** -10 if kind == "f32" else 1e-3)
    h = _theta(kind, n, seed=n + offset, scale=1.0 if kind == "f32" else 0.02, specials=True)
    t = _dev(kind, h)
    bits_h = oracle.gen_plane(SEED, step, probe, offset, n) if mode == "bits" else None
    bits_d = zo.zo_gen_probes(ctx, step, probe, 1, offset, n)[0] if mode == "bits" else None
    for a in (alpha, -alpha, -3.0 * alpha):
        zo.zo_perturb(ctx, t, offset, step, probe, a, bits_d)
        oracle.perturb(h, offset, SEED, step, probe, a, bits_h)
        assert_same_bits_or_nan(_host(kind, t), h, kind)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_perturb_restore_schedule_matches(ctx, kind):
    n = 8192 * 5 + 333
    h = _theta(kind, n, seed=3, scale=0.02)
    t = _dev(kind, h)
    for i in range(8):
        for s in (+1e-3, -1e-3, -1e-3, +1e-3):
            zo.zo_perturb(ctx, t, 0, 0, i, s)
            oracle.perturb(h, 0, SEED, 0, i, s)
    assert_same_bits_or_nan(_host(kind, t), h, kind)


def test_perturb_restore_exact_on_dyadic_grid(ctx):
    th0 = gen.dyadic_theta(8192 * 4 + 17, seed=9, frac_bits=12, max_abs_log2=11)
    t = to_dev_f32(th0)
    zo.zo_perturb(ctx, t, 0, 1, 2, 2.0 ** -10)
    zo.zo_perturb(ctx, t, 0, 1, 2, -(2.0 ** -10))
    assert np.array_equal(t.cpu().numpy().view(np.uint32), th0.view(np.uint32))


def test_perturb_keeps_denormals(ctx):
    # Subnormal inputs and steps must not be flushed: fp32 k * 2^-149 +/- 2^-147 and bf16
    # subnormals +/- 2^-133 are exact, so flushing anything would show.
    n = 8192 + 100
    k = np.random.default_rng(3).integers(-2 ** 20, 2 ** 20, n)
    x = (k.astype(np.float64) * 2.0 ** -149).astype(np.float32)
    t = to_dev_f32(x)
    zo.zo_perturb(ctx, t, 0, 0, 1, 2.0 ** -147)
    oracle.perturb(x, 0, SEED, 0, 1, 2.0 ** -147)
    assert_same_bits_or_nan(t.cpu().numpy(), x, "f32")
    assert np.count_nonzero(np.abs(x) < 2.0 ** -126) > n // 2
    hb = np.random.default_rng(4).integers(0, 0x7F, n).astype(np.uint16) | \
        (np.random.default_rng(5).integers(0, 2, n).astype(np.uint16) << 15)
    tb = to_dev_bf16(hb)
    zo.zo_perturb(ctx, tb, 0, 0, 2, 2.0 ** -133)
    oracle.perturb(hb, 0, SEED, 0, 2, 2.0 ** -133)
    assert_same_bits_or_nan(bf16_bits(tb), hb, "bf16")


# ------------------------------------------------------------------------------------
# probe weights
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 16, 160, 300, 1024])
def test_probe_weights_bit_exact(ctx, n):
    rng = np.random.default_rng(n)
    L0 = 2.0 + rng.normal(0, 0.05)
    u = rng.normal(0, 0.01, n)
    Lp = L0 + u + rng.normal(0.002, 0.001, n)
    Lm = L0 - u + rng.normal(0.002, 0.001, n)
    if n >= 16:
        Lp[3] = np.nan
        Lm[5] = np.inf
        Lp[7] = Lm[7] = L0            # h = 0: floored by delta
        Lp[8], Lm[8] = L0 - 1e-6, L0 - 3e-6   # negative curvature
    eps = float(np.float32(1e-3))
    zo.zo_reset_nonfinite(ctx)
    c = zo.zo_probe_weights(ctx, torch.from_numpy(Lp).cuda(), torch.from_numpy(Lm).cuda(),
                            torch.tensor([L0], dtype=torch.float64).cuda(), eps, 1e-6)
    ref, bad = oracle.probe_weights(Lp, Lm, L0, eps, 1e-6)
    assert np.array_equal(c.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert zo.zo_nonfinite_count(ctx) == bad


def test_probe_weights_nonfinite_clean_loss(ctx):
    n = 40
    Lp = torch.ones(n, dtype=torch.float64).cuda()
    Lm = torch.ones(n, dtype=torch.float64).cuda()
    zo.zo_reset_nonfinite(ctx)
    c = zo.zo_probe_weights(ctx, Lp, Lm, torch.tensor([np.nan], dtype=torch.float64).cuda(),
                            1e-3, 1e-6)
    assert torch.all(c == 0)
    assert zo.zo_nonfinite_count(ctx) == n
    zo.zo_reset_nonfinite(ctx)
    assert zo.zo_nonfinite_count(ctx) == 0


# ------------------------------------------------------------------------------------
# update
# ------------------------------------------------------------------------------------
# n_pert 16, 29-32, 64 and 153-160 take the unrolled kernel (group counts 2, 4, 8, 20; 153
# and 29 with zero-weight padding probes), the others the general one.
UPDATE_CASES = [(4096, 0, 16), (1000, 128, 7), (8192 * 3 + 1000, 0, 160), (1, 0, 1),
                (2_368_514, 0, 64), (33333, 128 * 3, 512), (8192, 0, 9),
                (8192 * 2 + 77, 128, 153), (50000, 0, 32), (3000, 128 * 2, 29)]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("n,offset,npert", UPDATE_CASES)
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_update_parity(ctx, kind, n, offset, npert, mode):
    step = 3
    rng = np.random.default_rng(n + npert)
    h = _theta(kind, n, seed=n, scale=0.02)
    c = (rng.standard_normal(npert) * 2.5e-3).astype(np.float32)
    eta = 1.0 if kind == "bf16" else 1e-2      # large enough that bf16 updates do move
    t = _dev(kind, h)
    bits_h = oracle.gen_planes(SEED, step, 0, npert, offset, n) if mode == "bits" else None
    bits_d = zo.zo_gen_probes(ctx, step, 0, npert, offset, n) if mode == "bits" else None
    zo.zo_update(ctx, t, offset, step, to_dev_f32(c), eta, bits_d)
    oracle.update(h, offset, SEED, step, c, eta, bits_h)
    got = _host(kind, t)
    if kind == "f32":
        assert_f32_update_close(got, h, eta, c)
        same = np.mean(got.view(np.uint32) == h.view(np.uint32))
    else:
        assert_bf16_within_ulp(got, h)
        same = np.mean(got == h)
    # fp64 sums: all but (measure-zero) rounding ties agree bit for bit
    assert same >= 0.9999, same


RESTORE_CASES = [(4096, 0, 16, 15), (1000, 128, 7, 3), (8192 * 3 + 1000, 0, 160, 159),
                 (1, 0, 1, 0), (33333, 128 * 3, 512, 300), (8192 * 13 + 5, 128, 160, 8),
                 (8192 * 2 + 77, 128, 153, 152), (50000, 0, 32, 20)]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("n,offset,npert,rprobe", RESTORE_CASES)
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_restore_update_equals_perturb_then_update(ctx, kind, n, offset, npert, rprobe, mode):
    """zo_restore_update is zo_perturb followed by zo_update, bit for bit, on the GPU; and
    within the update bar of the oracle's perturb followed by its update.  Restore probes
    sit in the first, a middle and the last sign group, with ragged sizes and offsets."""
    step = 6
    rng = np.random.default_rng(n + npert + rprobe)
    h = _theta(kind, n, seed=n + 3, scale=0.02, specials=True)
    c = (rng.standard_normal(npert) * 2.5e-3).astype(np.float32)
    eta = 1.0 if kind == "bf16" else 1e-2
    alpha = 1e-3 if kind == "bf16" else 2.0 ** -10
    bits_h = oracle.gen_planes(SEED, step, 0, npert, offset, n) if mode == "bits" else None
    bits_d = zo.zo_gen_probes(ctx, step, 0, npert, offset, n) if mode == "bits" else None
    cd = to_dev_f32(c)
    fused, seq = _dev(kind, h), _dev(kind, h)
    zo.zo_restore_update(ctx, fused, offset, step, rprobe, alpha, cd, eta, bits_d)
    zo.zo_perturb(ctx, seq, offset, step, rprobe, alpha, None if bits_d is None else bits_d[rprobe])
    zo.zo_update(ctx, seq, offset, step, cd, eta, bits_d)
    got, want = _host(kind, fused), _host(kind, seq)
    assert_same_bits_or_nan(got, want, kind)
    oracle.perturb(h, offset, SEED, step, rprobe, alpha,
                   None if bits_h is None else bits_h[rprobe])
    oracle.update(h, offset, SEED, step, c, eta, bits_h)
    fin = np.isfinite(h.astype(np.float32) if kind == "f32" else
                      (h.astype(np.uint32) << 16).view(np.float32))
    if kind == "f32":
        assert_f32_update_close(got[fin], h[fin], eta, c)
    else:
        assert_bf16_within_ulp(got[fin], h[fin])


def test_restore_update_argument_checks(ctx):
    L = zo._lib.lib()
    t = torch.zeros(256, dtype=torch.float32, device="cuda")
    c = torch.zeros(8, dtype=torch.float32, device="cuda")
    args = lambda rp, npert=8: L.zo_restore_update(  # noqa: E731
        ctx.handle, t.data_ptr(), zo.ZO_FP32, 0, 256, 0, rp, 1e-3, c.data_ptr(), npert, 1e-2,
        None, None)
    assert args(8) == zo.ZO_EINVAL                 # restore probe outside the step's probes
    assert args(0, npert=0) == zo.ZO_EINVAL
    assert args(0, npert=513) == zo.ZO_EUNSUPPORTED
    assert args(7) == zo.ZO_OK
    torch.cuda.synchronize()


def test_update_sum_error_within_recursive_summation_bound(ctx):
    # s_j from the GPU (recovered with eta = 1 on theta = 0 in fp32: theta' = -s rounded
    # once to fp32) vs the oracle's fp64 sums: |s_gpu - s| <= half an fp32 ulp of s plus
    # gamma_(n/8 + 8) * sum |c_i| in fp64 (recursive summation, Higham), factor 2 margin.
    n, npert = 8192 * 2 + 5, 160
    c = (np.random.default_rng(1).standard_normal(npert) * 1e-2).astype(np.float32)
    t = torch.zeros(n, dtype=torch.float32, device="cuda")
    zo.zo_update(ctx, t, 0, 7, to_dev_f32(c), 1.0)
    s_gpu = -t.cpu().numpy().astype(np.float64)
    s = oracle.probe_sums(n, 0, SEED, 7, c)
    u = 2.0 ** -53
    k = npert // 8 + 8
    gamma = k * u / (1 - k * u)
    half_ulp = 0.5 * np.spacing(np.abs(s).astype(np.float32)).astype(np.float64)
    bound = half_ulp + 2 * gamma * np.sum(np.abs(c.astype(np.float64)))
    assert np.all(np.abs(s_gpu - s) <= bound)


def test_update_single_probe_equals_perturb(ctx):
    for kind in ("f32", "bf16"):
        h = _theta(kind, 8192 * 2 + 100, seed=4, scale=0.02)
        a, b = _dev(kind, h), _dev(kind, h)
        eta = 2.0 ** -9
        zo.zo_update(ctx, a, 0, 6, torch.tensor([1.0], device="cuda"), eta)
        zo.zo_perturb(ctx, b, 0, 6, 0, -eta)
        assert np.array_equal(_host(kind, a), _host(kind, b))


def test_update_identity_cases(ctx):
    h = _theta("f32", 9000, seed=6)
    t = to_dev_f32(h)
    zo.zo_update(ctx, t, 0, 1, torch.zeros(16, device="cuda"), 0.7)
    zo.zo_update(ctx, t, 0, 1, torch.ones(16, device="cuda"), 0.0)
    assert np.array_equal(t.cpu().numpy().view(np.uint32), h.view(np.uint32))


def test_update_independent_of_split_and_geometry(ctx):
    # Updating [0, n) at once or as two buffers with their global offsets gives the same
    # bits: each element's sum is independent of the launch geometry.
    n, cut, npert = 8192 * 7 + 300, 128 * 131, 40
    h = _theta("bf16", n, seed=7, scale=0.02)
    c = to_dev_f32(np.random.default_rng(2).standard_normal(npert).astype(np.float32) * 1e-2)
    whole = to_dev_bf16(h)
    zo.zo_update(ctx, whole, 0, 2, c, 1.0)
    left, right = to_dev_bf16(h[:cut]), to_dev_bf16(h[cut:])
    zo.zo_update(ctx, left, 0, 2, c, 1.0)
    zo.zo_update(ctx, right, cut, 2, c, 1.0)
    assert np.array_equal(bf16_bits(whole), np.concatenate([bf16_bits(left), bf16_bits(right)]))


def test_update_brute_force_all_sign_patterns(ctx):
    # sum over all 2^8 patterns of (z^T A theta) z = 256 A theta, exactly.
    rng = np.random.Generator(np.random.PCG64(5))
    B = rng.integers(-8, 9, (8, 8)) / 16.0
    A = (B + B.T) / 2
    th0 = (rng.integers(-64, 65, 8) / 16.0).astype(np.float32)
    rows = np.zeros((256, 16), dtype=np.uint8)
    rows[:, 0] = np.arange(256, dtype=np.uint8)
    Z = np.array([[1.0 if (p >> j) & 1 else -1.0 for j in range(8)] for p in range(256)])
    v = A @ th0.astype(np.float64)
    c = (Z @ v).astype(np.float32)
    eta = 2.0 ** -10
    t = to_dev_f32(th0)
    zo.zo_update(ctx, t, 0, 0, to_dev_f32(c), eta, torch.from_numpy(rows).cuda())
    assert np.array_equal(t.cpu().numpy().astype(np.float64), th0 - eta * 256 * v)


# ------------------------------------------------------------------------------------
# loss kernel and argument checks
# ------------------------------------------------------------------------------------
# The loss kernel takes 2048-param chunks, one per wave of its 4096-wave grid at a time:
# sizes below, at and just above one chunk, exact chunks, a ragged tail, and more chunks
# than waves (each wave taking several).
@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 2047, 2049, 4096, 1_000_003, 16_777_293])
def test_quad_loss(ctx, kind, n):
    h = _theta(kind, n, seed=8, scale=0.5)
    a = np.power(10.0, np.random.default_rng(9).uniform(-2, 2, n)).astype(np.float32)
    got = zo.zo_quad_loss(ctx, _dev(kind, h), to_dev_f32(a)).item()
    ref = oracle.quad_loss(h, a)
    assert abs(got - ref) <= 1e-13 * abs(ref) + 1e-300
    assert zo.zo_quad_loss(ctx, _dev(kind, h), to_dev_f32(a)).item() == got  # deterministic


def test_argument_checks(ctx):
    t = torch.zeros(1024, dtype=torch.float32, device="cuda")
    c = torch.zeros(4, dtype=torch.float32, device="cuda")
    with pytest.raises(zo.ZOError) as e:
        zo.zo_perturb(ctx, t[1:], 0, 0, 0, 1.0)          # misaligned
    assert e.value.status == zo.ZO_EINVAL
    with pytest.raises(zo.ZOError) as e:
        zo.zo_perturb(ctx, t, 64, 0, 0, 1.0)             # offset not a multiple of 128
    assert e.value.status == zo.ZO_EINVAL
    with pytest.raises(zo.ZOError) as e:
        zo.zo_update(ctx, t, 0, 0, torch.zeros(zo.ZO_MAX_NPERT + 1, device="cuda"), 1.0)
    assert e.value.status == zo.ZO_EUNSUPPORTED
    d = torch.zeros(4, dtype=torch.float64, device="cuda")
    with pytest.raises(zo.ZOError) as e:
        zo.zo_probe_weights(ctx, d, d, d[:1], 0.0, 1e-6)   # eps = 0
    assert e.value.status == zo.ZO_EINVAL
    empty = torch.zeros(0, dtype=torch.float32, device="cuda")
    zo.zo_perturb(ctx, empty, 0, 0, 0, 1.0)               # empty calls are no-ops
    zo.zo_update(ctx, empty, 0, 0, c, 1.0)
    zo.zo_update(ctx, t, 0, 0, empty, 1.0)
    assert torch.all(t == 0)


def test_binding_requires_exact_packed_rows(ctx):
    """Rows generated over a larger range (say the whole model) are not rows of a
    sub-buffer: the library reads zo_bits_stride(n) bytes per row at a fixed row stride, so
    the binding refuses rows and row sets whose shape is not exactly the buffer's, and a
    weights output shorter than n_pert."""
    n = 4096
    t = torch.zeros(n, dtype=torch.float32, device="cuda")
    c = torch.zeros(4, dtype=torch.float32, device="cuda")
    wide = zo.zo_gen_probes(ctx, 0, 0, 4, 0, 2 * n)           # rows over 2n params
    with pytest.raises(ValueError):
        zo.zo_perturb(ctx, t, 0, 0, 0, 1.0, wide[0])
    with pytest.raises(ValueError):
        zo.zo_perturb2(ctx, t, 0, 0, 0, 1.0, 1, 1.0, wide[0], wide[1])
    with pytest.raises(ValueError):
        zo.zo_update(ctx, t, 0, 0, c, 1.0, wide)
    with pytest.raises(ValueError):
        zo.zo_restore_update(ctx, t, 0, 0, 0, 1.0, c, 1.0, wide)
    own = zo.zo_gen_probes(ctx, 0, 0, 4, 0, n)
    with pytest.raises(ValueError):
        zo.zo_update(ctx, t, 0, 0, c, 1.0, own.reshape(-1))   # right bytes, not n_pert rows
    with pytest.raises(ValueError):
        zo.zo_update(ctx, t, 0, 0, c[:3], 1.0, own)           # 4 rows for 3 probes
    zo.zo_update(ctx, t, 0, 0, c, 1.0, own)                   # the exact shape is accepted
    zo.zo_perturb(ctx, t, 0, 0, 0, 0.0, own[0])
    d = torch.zeros(4, dtype=torch.float64, device="cuda")
    with pytest.raises(ValueError):
        zo.zo_probe_weights_ex(ctx, d, d, d[:1], 1e-3, 1e-6, zo.ZO_WEIGHTS_PRECOND,
                               out=torch.empty(3, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(t == 0)


# ------------------------------------------------------------------------------------
# whole steps
# ------------------------------------------------------------------------------------
def _quad_loss_error_bound(theta, a):
    """Bound on |L_gpu - L_oracle| for the fp64 quadratic loss: both sides sum M products
    of size <= max(a theta^2) in fp64, each with at most M roundings (Higham's bound for
    recursive summation, doubled for the two sides), plus the products' own roundings."""
    t = theta.astype(np.float64) if theta.dtype == np.float32 else oracle.bf16_to_f32(theta).astype(np.float64)
    terms = 0.5 * a.astype(np.float64) * t * t
    M = t.size
    return 2 * (M + 3) * 2.0 ** -53 * np.sum(np.abs(terms)) * 1.01


@pytest.mark.parametrize("schedule", ["S4", "S2f"])
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_tiny_config_steps_from_seeded_theta(ctx, schedule, mode):
    """The tiny quadratic workload end to end, each side on its own: from the seeded theta,
    the GPU step (GPU losses) and the oracle step (oracle losses) for steps 0..9 (different
    probes each): the losses agree to the fp64 summation bound, the weights within the
    bound those loss differences imply, and theta within the update tolerance plus
    eta * sum |dc|."""
    cfg = CONFIGS["tiny"]
    local = zo.zo_init(cfg.seed)
    th0, a = gen.theta_and_a(cfg)
    ad = to_dev_f32(a)
    dL = _quad_loss_error_bound(th0, a) * 1.1
    lossf = lambda x, o: zo.zo_quad_loss(local, x, ad, out=o)  # noqa: E731
    for step in range(cfg.steps):
        t = to_dev_f32(th0)
        h = th0.copy()
        bits_d = zo.zo_gen_probes(local, step, 0, cfg.npert, 0, cfg.M) if mode == "bits" else None
        bits_h = oracle.gen_planes(cfg.seed, step, 0, cfg.npert, 0, cfg.M) if mode == "bits" else None
        out = spsa_step(local, t, step=step, npert=cfg.npert, eps=cfg.eps, eta=cfg.eta,
                        delta=cfg.delta, loss=lossf, bits=bits_d, schedule=schedule)
        res = oracle.spsa_step(h, seed=cfg.seed, step=step, npert=cfg.npert, eps=cfg.eps,
                               eta=cfg.eta, delta=cfg.delta, loss_fn=lambda x: oracle.quad_loss(x, a),
                               bits=bits_h, schedule=schedule)
        L0, Lp, Lm = out["L0"].item(), out["Lp"].cpu().numpy(), out["Lm"].cpu().numpy()
        assert abs(L0 - res["L0"]) <= dL
        assert np.all(np.abs(Lp - res["Lp"]) <= dL) and np.all(np.abs(Lm - res["Lm"]) <= dL)
        c = out["c"].cpu().numpy()
        eps = float(np.float32(cfg.eps))
        bound = weight_bound(res["Lp"], res["Lm"], res["L0"], dL, eps, cfg.delta, res["c"])
        assert np.all(np.abs(c.astype(np.float64) - res["c"]) <= bound)
        got = t.cpu().numpy()
        extra = float(np.float32(cfg.eta)) * float(np.sum(bound))
        scale = np.maximum(np.abs(h.astype(np.float64)),
                           float(np.float32(cfg.eta)) * float(np.sum(np.abs(res["c"]))))
        assert np.all(np.abs(got.astype(np.float64) - h) <= 1e-5 * scale + extra)
    local.close()


def _quad_sum_bound(theta, a, eps):
    """Bound on the difference of two fp64 evaluations of 1/2 sum a_j x_j^2 at the same
    point near theta (|x_j| <= |theta_j| + 2 eps), summed in different orders: Higham's
    recursive-summation bound on each side plus the products' own roundings."""
    x = np.abs(theta.astype(np.float64)) + 2 * eps
    return 2 * (theta.size + 3) * 2.0 ** -53 * np.sum(0.5 * a.astype(np.float64) * x * x) * 1.1


@pytest.mark.parametrize("schedule", ["S4", "S2f"])
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_tiny_config_trajectory(ctx, schedule, mode):
    """The tiny workload's 10-step trajectory, each side on its own from the seeded theta
    (GPU: library passes, GPU losses, weights and update; oracle: its own passes, losses,
    weights and update, probes of its own), compared after every step.

    The two states can part only through rounding: the update sums the probes in another
    order (at most one fp32 ulp of the new value per element and step), and a weight that
    differs in its last bit moves every element by eta * |dc|.  With D the measured state
    difference before a step, the step must satisfy
      * losses: |L_gpu - L_ora| <= fp64 summation bound + sum_j a_j (|x_j| E_j + E_j^2 / 2),
        with E_j = D_j + (passes) * ulp where D_j > 0, else 0 (the passes are bit-exact
        functions, so states that agree visit the same points);
      * weights: |c_gpu - c_ora| within the bound those loss differences imply, and that
        bound finite for every probe;
      * the new state: D'_j <= E_j + eta * (sum_i |dc_i| + fp64 sum error) + one fp32 ulp.
    After ten steps nearly every element is still bit-identical and both losses fell."""
    cfg = CONFIGS["tiny"]
    local = zo.zo_init(cfg.seed)
    th0, a = gen.theta_and_a(cfg)
    ad = to_dev_f32(a)
    af = a.astype(np.float64)
    eps = float(np.float32(cfg.eps))
    eta = float(np.float32(cfg.eta))
    npasses = 4 * cfg.npert + 1
    lossf = lambda x, o: zo.zo_quad_loss(local, x, ad, out=o)  # noqa: E731
    t, h = to_dev_f32(th0), th0.copy()
    first_gpu, first_ora = zo.zo_quad_loss(local, t, ad).item(), oracle.quad_loss(h, a)
    for step in range(cfg.steps):
        D = np.abs(t.cpu().numpy().astype(np.float64) - h.astype(np.float64))
        ulp = np.spacing((np.abs(h) + D + 4 * eps).astype(np.float32)).astype(np.float64)
        E = np.where(D > 0, D + npasses * ulp, 0.0)
        dL = _quad_sum_bound(h, a, eps) + float(np.sum(af * ((np.abs(h) + 4 * eps) * E
                                                             + 0.5 * E * E)))
        bits_d = zo.zo_gen_probes(local, step, 0, cfg.npert, 0, cfg.M) if mode == "bits" else None
        bits_h = oracle.gen_planes(cfg.seed, step, 0, cfg.npert, 0, cfg.M) if mode == "bits" else None
        out = spsa_step(local, t, step=step, npert=cfg.npert, eps=cfg.eps, eta=cfg.eta,
                        delta=cfg.delta, loss=lossf, bits=bits_d, schedule=schedule)
        res = oracle.spsa_step(h, seed=cfg.seed, step=step, npert=cfg.npert, eps=cfg.eps,
                               eta=cfg.eta, delta=cfg.delta,
                               loss_fn=lambda x: oracle.quad_loss(x, a), bits=bits_h,
                               schedule=schedule)
        L0, Lp, Lm = out["L0"].item(), out["Lp"].cpu().numpy(), out["Lm"].cpu().numpy()
        assert abs(L0 - res["L0"]) <= dL, (step, L0, res["L0"], dL)
        assert np.all(np.abs(Lp - res["Lp"]) <= dL) and np.all(np.abs(Lm - res["Lm"]) <= dL), step
        c = out["c"].cpu().numpy().astype(np.float64)
        bound = weight_bound(res["Lp"], res["Lm"], res["L0"], dL, eps, cfg.delta, res["c"])
        assert np.all(np.isfinite(bound)), (step, bound)
        dc = np.abs(c - res["c"])
        assert np.all(dc <= bound), (step, dc, bound)
        got = t.cpu().numpy()
        sum_err = 2 * (cfg.npert + 8) * 2.0 ** -53 * float(np.sum(np.abs(res["c"]))) * 1.01
        new_ulp = np.spacing(np.maximum(np.abs(got), np.abs(h))).astype(np.float64)
        allow = E + eta * (float(np.sum(dc)) + sum_err) + new_ulp
        D_next = np.abs(got.astype(np.float64) - h.astype(np.float64))
        assert np.all(D_next <= allow), (step, int(np.sum(D_next > allow)))
        print(f"[trajectory] {schedule}/{mode} step {step}: {int(np.sum(D_next > 0))} of "
              f"{cfg.M} elements differ, max |dc| {dc.max():.3e}", flush=True)
    same = float(np.mean(t.cpu().numpy().view(np.uint32) == h.view(np.uint32)))
    assert same >= 0.99, same
    assert zo.zo_quad_loss(local, t, ad).item() < first_gpu
    assert oracle.quad_loss(h, a) < first_ora
    local.close()


def test_bf16_synthetic_step_small(ctx):
    """A bf16 step with synthetic per-probe losses (the OPT-shaped workloads' loss model)
    on a small buffer: perturb passes bit-exact, weights bit-exact, update within 1 ulp."""
    cfg = CONFIGS["opt30b"]
    n, npert = 8192 * 4 + 555, cfg.npert
    h = _theta("bf16", n, seed=12, scale=0.02)
    t = to_dev_bf16(h)
    L0, Lp, Lm = gen.synthetic_losses(cfg.seed, 0, npert)
    dl = (torch.tensor([L0], dtype=torch.float64).cuda(), torch.from_numpy(Lp).cuda(),
          torch.from_numpy(Lm).cuda())
    out = spsa_step(ctx, t, step=0, npert=npert, eps=cfg.eps, eta=1.0, delta=cfg.delta,
                    losses=dl)
    res = oracle.spsa_step(h, seed=SEED, step=0, npert=npert, eps=cfg.eps, eta=1.0,
                           delta=cfg.delta, losses=(L0, Lp, Lm))
    assert np.array_equal(out["c"].cpu().numpy(), res["c"])
    assert_bf16_within_ulp(bf16_bits(t), h)


# ------------------------------------------------------------------------------------
# fused two-probe pass and the two-pass schedule
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("n,offset", [(8192 * 3 + 1000, 0), (127, 128), (1 << 22, 128 * 9)])
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_perturb2_bit_exact(ctx, kind, n, offset, mode):
    step, pa, pb = 2, 5, 6
    h = _theta(kind, n, seed=n + 1, scale=0.02, specials=True)
    t = _dev(kind, h)
    if mode == "bits":
        ra, rb = (oracle.gen_plane(SEED, step, p, offset, n) for p in (pa, pb))
        da, db = (zo.zo_gen_probes(ctx, step, p, 1, offset, n)[0] for p in (pa, pb))
    else:
        ra = rb = da = db = None
    for aa, ab in ((1e-3, 1e-3), (-2e-3, 1e-3), (1e-3, -3e-3), (2.0 ** -10, 0.0)):
        zo.zo_perturb2(ctx, t, offset, step, pa, aa, pb, ab, da, db)
        oracle.perturb2(h, offset, SEED, step, pa, aa, pb, ab, ra, rb)
        assert_same_bits_or_nan(_host(kind, t), h, kind)


def test_perturb2_requires_both_rows(ctx):
    t = torch.zeros(256, dtype=torch.float32, device="cuda")
    row = torch.zeros(zo.zo_bits_stride(256), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        zo.zo_perturb2(ctx, t, 0, 0, 0, 1.0, 1, 1.0, row, None)
    from forward_only_amd import _lib
    st = _lib.lib().zo_perturb2(ctx.handle, t.data_ptr(), 0, 0, 256, 0, 0, 1.0, 1, 1.0,
                                row.data_ptr(), None, None)
    assert st == zo.ZO_EINVAL


def test_bf16_synthetic_two_pass_step_small(ctx):
    cfg = CONFIGS["opt30b"]
    n, npert = 8192 * 4 + 555, cfg.npert
    h = _theta("bf16", n, seed=13, scale=0.02)
    t = to_dev_bf16(h)
    L0, Lp, Lm = gen.synthetic_losses(cfg.seed, 1, npert)
    dl = (torch.tensor([L0], dtype=torch.float64).cuda(), torch.from_numpy(Lp).cuda(),
          torch.from_numpy(Lm).cuda())
    spsa_step(ctx, t, step=1, npert=npert, eps=cfg.eps, eta=0.0, delta=cfg.delta, losses=dl,
              schedule="S2f")
    oracle.spsa_step(h, seed=SEED, step=1, npert=npert, eps=cfg.eps, eta=0.0,
                     delta=cfg.delta, losses=(L0, Lp, Lm), schedule="S2f")
    # eta = 0: the passes alone, which are bit-exact
    assert np.array_equal(bf16_bits(t), h)


@pytest.mark.parametrize("kind,npert,mode", [("bf16", 16, "regen"), ("f32", 160, "regen"),
                                             ("bf16", 512, "regen"), ("f32", 512, "bits"),
                                             ("bf16", 160, "bits")])
def test_step_calls_replay_from_a_captured_graph(ctx, kind, npert, mode):
    """The library's calls of one two-pass step (passes, fused passes, weights, the update
    carrying the last restore; with stored signs also the plane generator) captured into a
    HIP graph: no allocation, synchronisation, attribute call or memset node in them, so
    each replay equals the same calls made eagerly, replay after replay, with eager work and
    synchronisations in between.  n_pert = 512 runs the general update kernel with 138 KiB
    of dynamic LDS (the limit raised once by zo_init), stored signs the general kernel at
    any probe count."""
    n, step = 8192 * 5 + 77, 4
    h = _theta(kind, n, seed=17, scale=0.02)
    a = 1e-3 if kind == "bf16" else 2.0 ** -10
    L0, Lp, Lm = gen.synthetic_losses(5, step, npert)
    L0d = torch.tensor([L0], dtype=torch.float64).cuda()
    Lpd, Lmd = torch.from_numpy(Lp).cuda(), torch.from_numpy(Lm).cuda()
    c_eager = torch.empty(npert, dtype=torch.float32, device="cuda")
    c_graph = torch.empty(npert, dtype=torch.float32, device="cuda")
    eta = 1.0 if kind == "bf16" else 1e-2
    stride = zo.zo_bits_stride(n)
    planes = {}
    for name in ("eager", "graph", "warm"):
        planes[name] = (torch.empty((npert, stride), dtype=torch.uint8, device="cuda")
                        if mode == "bits" else None)

    def calls(t, c, bits):
        row = (lambda i: None) if bits is None else (lambda i: bits[i])
        if bits is not None:
            zo.zo_gen_probes(ctx, step, 0, npert, 0, n, out=bits)
        zo.zo_perturb(ctx, t, 0, step, 0, +a, row(0))
        for i in range(npert):
            zo.zo_perturb(ctx, t, 0, step, i, -2.0 * a, row(i))
            if i + 1 < npert:
                zo.zo_perturb2(ctx, t, 0, step, i, +a, i + 1, +a, row(i), row(i + 1))
        zo.zo_probe_weights(ctx, Lpd, Lmd, L0d, a, 1e-6, out=c)
        zo.zo_restore_update(ctx, t, 0, step, npert - 1, +a, c, eta, bits)

    eager, graphed, warm = _dev(kind, h), _dev(kind, h), _dev(kind, h)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(warm, c_graph, planes["warm"])      # first launches outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(graphed, c_graph, planes["graph"])
    torch.cuda.synchronize()
    assert np.array_equal(_host(kind, graphed), _host(kind, _dev(kind, h)))   # not yet run
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        calls(eager, c_eager, planes["eager"])
        torch.cuda.synchronize()
        assert np.array_equal(_host(kind, graphed), _host(kind, eager))
        assert torch.equal(c_graph, c_eager)
        if mode == "bits":
            assert torch.equal(planes["graph"], planes["eager"])


# ------------------------------------------------------------------------------------
# the other weight forms of the pages
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("mode,power", [(0, 1.0), (1, 0.1), (1, 0.5), (1, 0.0), (2, 1.0)])
@pytest.mark.parametrize("n", [16, 160, 300])
def test_probe_weights_ex(ctx, mode, power, n):
    L0, Lp, Lm = gen.synthetic_losses(3, n, n)
    Lp[2] = np.inf
    eps = float(np.float32(1e-3))
    zo.zo_reset_nonfinite(ctx)
    L0d = None if mode == 2 else torch.tensor([L0], dtype=torch.float64).cuda()
    c = zo.zo_probe_weights_ex(ctx, torch.from_numpy(Lp).cuda(), torch.from_numpy(Lm).cuda(),
                               L0d, eps, 1e-6, mode, power).cpu().numpy()
    ref, bad = oracle.probe_weights_ex(Lp, Lm, L0, eps, 1e-6, mode, power)
    assert zo.zo_nonfinite_count(ctx) == bad == 1
    if mode == 1 and power not in (0.0, 1.0):
        # pow() of the device library and of libm may differ in the last bit of the double;
        # after rounding to fp32 the weights agree to one ulp
        assert np.all(np.abs(c.astype(np.float64) - ref) <= np.spacing(np.abs(ref)))
    else:
        assert np.array_equal(c.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("nbytes", [16, 16384 - 16, 16384, 16384 * 13 + 32, (1 << 20) + 48,
                                    (64 << 20) + 16, 16384 * 8205 + 48])
def test_stream_rmw(ctx, nbytes):
    """The diagnostic in-place streaming pass touches every word exactly once: a non-zero
    mask flips every word of whole chunks and the ragged tail alike, flipping again restores
    them, and mask 0 leaves arbitrary bit patterns (NaN payloads, denormals, negative zero)
    identical."""
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    host[:4] = [0x7FC00001, 0x80000000, 0x00000001, 0xFF800000]
    buf = torch.from_numpy(host.view(np.int32).copy()).cuda()
    mask = 0xA5C3F00F
    zo.zo_stream_rmw(ctx, buf, mask)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy().view(np.uint32), host ^ np.uint32(mask))
    zo.zo_stream_rmw(ctx, buf, mask)
    zo.zo_stream_rmw(ctx, buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy().view(np.uint32), host)


def test_stream_rmw_argument_checks(ctx):
    L = zo._lib.lib()
    t = torch.zeros(64, dtype=torch.int32, device="cuda")
    assert L.zo_stream_rmw(ctx.handle, t.data_ptr(), 20, 0, None) == zo.ZO_EINVAL      # size % 16
    assert L.zo_stream_rmw(ctx.handle, t.data_ptr() + 4, 16, 0, None) == zo.ZO_EINVAL  # alignment
    assert L.zo_stream_rmw(ctx.handle, None, 0, 0, None) == zo.ZO_OK                    # empty


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["regen", "bits"])
def test_sliced_passes_equal_the_oracle(kind, mode):
    """Passes issued per 1 MiB slice (seven slices and a ragged tail, at a non-zero offset):
    zo_perturb and zo_perturb2 stay bit-exact with the oracle, slice boundaries included."""
    n = 3_300_001 if kind == "bf16" else 1_700_003
    offset, step = 128 * 5, 8
    local = zo.zo_init(SEED)
    zo.zo_set_slice_bytes(local, 1 << 20)
    assert zo.zo_get_slice_bytes(local) == 1 << 20
    h = _theta(kind, n, seed=n, scale=0.02, specials=True)
    t = _dev(kind, h)
    if mode == "bits":
        bh = [oracle.gen_plane(SEED, step, p, offset, n) for p in (2, 3)]
        bd = zo.zo_gen_probes(local, step, 2, 2, offset, n)
        rows = (bd[0], bd[1])
    else:
        bh, rows = [None, None], (None, None)
    zo.zo_perturb(local, t, offset, step, 2, 1e-3, rows[0])
    oracle.perturb(h, offset, SEED, step, 2, 1e-3, bh[0])
    zo.zo_perturb2(local, t, offset, step, 2, 1e-3, 3, -2e-3, rows[0], rows[1])
    oracle.perturb2(h, offset, SEED, step, 2, 1e-3, 3, -2e-3, bh[0], bh[1])
    assert_same_bits_or_nan(_host(kind, t), h, kind)
    local.close()


def test_relocate_keeps_the_contents_on_the_fastest_allocation():
    """placement.relocate: the buffer it returns holds the original contents, is the fastest
    of the allocations it tried (or the original when none beat it), and the context's pass
    form is the one tuned for it.  The search is forced (no placement counts as fast) so that
    a candidate is usually kept and the copy path runs."""
    local = zo.zo_init(SEED)
    t = torch.randint(-2 ** 15, 2 ** 15, (5 << 29,), dtype=torch.int16, device="cuda")  # 5 GiB
    ref = t.clone()
    out, rep = placement.relocate(local, t, tries=2, fast_ratio=100.0, min_gain=0.0)
    assert not rep["skipped"]
    assert 1 <= len(rep["tried"]) <= 3
    rates = [max(r["gbps_whole"], r["gbps_sliced"]) for r in rep["tried"]]
    assert rates[rep["kept"]] == max(rates)
    assert rep["copied"] == (rep["kept"] != 0)
    assert (out is t) == (rep["kept"] == 0)
    assert out.shape == t.shape and out.dtype == t.dtype
    assert torch.equal(out, ref)
    assert zo.zo_get_slice_bytes(local) == rep["final"]["slice_bytes"]
    small = torch.zeros(1000, dtype=torch.float32, device="cuda")
    o2, r2 = placement.relocate(local, small)
    assert o2 is small and r2["skipped"]
    del out, t, ref
    torch.cuda.empty_cache()


def test_tune_placement_keeps_the_buffer_and_chooses_a_form():
    local = zo.zo_init(SEED)
    t = torch.randint(-2 ** 15, 2 ** 15, (5 << 29,), dtype=torch.int16, device="cuda")  # 5 GiB
    ref = t.clone()
    r = zo.zo_tune_placement(local, t)
    assert r["slice_bytes"] in (0, 1 << 30)
    assert r["gbps_whole"] > 100 and r["gbps_sliced"] > 100
    assert zo.zo_get_slice_bytes(local) == r["slice_bytes"]
    assert torch.equal(t, ref)                                          # contents unchanged
    del ref
    small = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")      # 4 MiB: one launch
    r2 = zo.zo_tune_placement(local, small)
    assert r2["slice_bytes"] == 0 and r2["gbps_sliced"] == 0.0
    with pytest.raises(zo.ZOError):
        zo.zo_set_slice_bytes(local, 1000)                               # not a multiple of 1 MiB
    zo.zo_set_slice_bytes(local, 0)
    assert zo.zo_get_slice_bytes(local) == 0
    local.close()

