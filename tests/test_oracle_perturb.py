"""Pins of the oracle's roundings and of the in-place perturb / restore.

Independent anchors: exact rational arithmetic (fractions.Fraction) for round-to-nearest-
even to bf16, numpy's IEEE fp32 add, and closed-form properties of a single rounded add
(the in-place move theta <- theta + alpha*z of "Stanford's 1.5-SPSA Trains OPT-30B Without
Backpropagation", section "How 1.5-SPSA Works", done in place as the abstract of
"Probe-Space Preconditioning for Fast and Stable Zero-Order Training" describes).
"""
import math
from fractions import Fraction

import numpy as np

import oracle
from workloads import gen


def _f32_from_bits(p):
    return float(np.array([p], dtype=np.uint32).view(np.float32)[0])


def brute_bf16(x: float) -> int:
    """Nearest bf16 to x (ties to the even pattern) by exhaustive exact comparison over the
    neighbouring bit patterns; a value beyond the largest finite one rounds as if 2^128
    were representable (its pattern is the even infinity)."""
    s = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if math.isinf(a):
        return s | 0x7F80
    A = Fraction(a)
    with np.errstate(over="ignore"):
        h = int(np.array([a], dtype=np.float32).view(np.uint32)[0] >> 16)
    best = None
    for p in range(max(0, h - 2), min(0x7F80, h + 2) + 1):
        v = Fraction(2) ** 128 if p == 0x7F80 else Fraction(_f32_from_bits(p << 16))
        key = (abs(v - A), p & 1)
        if best is None or key < best[0]:
            best = (key, p)
    return s | best[1]


def _rounding_cases(rng, n_random=3000):
    xs = []
    # log-uniform magnitudes over the whole bf16 range, both signs
    mag = 2.0 ** rng.uniform(-140, 129, n_random)
    xs += list(mag * rng.choice([-1.0, 1.0], n_random))
    # exact ties and their neighbours, normal and subnormal binades
    for e in list(range(-133, 128, 7)) + [-126, -127, 127]:
        for m in (0, 1, 2, 0x7E, 0x7F):
            lo = (1.0 + m / 128.0) * 2.0 ** e if e >= -126 else m * 2.0 ** -133
            ulp = 2.0 ** (e - 7) if e >= -126 else 2.0 ** -133
            tie = lo + ulp / 2
            xs += [tie, math.nextafter(tie, 0.0), math.nextafter(tie, math.inf), -tie]
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    xs += [big, big + 2.0 ** 119, math.nextafter(big + 2.0 ** 119, 0.0), 2.0 ** 128, 1e300,
           0.0, -0.0, math.inf, -math.inf, 5e-324, 2.0 ** -134, 3 * 2.0 ** -135]
    return xs


def test_f64_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(0)
    xs = _rounding_cases(rng)
    got = oracle.f64_to_bf16(np.array(xs, dtype=np.float64))
    for x, g in zip(xs, got):
        assert int(g) == brute_bf16(x), (x, hex(int(g)), hex(brute_bf16(x)))


def test_f64_to_bf16_nan():
    got = oracle.f64_to_bf16(np.array([math.nan, -math.nan]))
    assert all((int(g) & 0x7F80) == 0x7F80 and (int(g) & 0x7F) != 0 for g in got)


def test_f32_to_bf16_ties_all_exponents():
    # every fp32 whose low half sits at or next to the rounding boundary, all high halves
    hi = np.arange(0, 1 << 16, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]                         # finite only
    pats = np.concatenate([(hi << 16) | lo for lo in (0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF)])
    f = pats.view(np.float32)
    got = oracle.f32_to_bf16(f)
    # The bf16 value is the fp32 rounded at bit 16: the exact rounding can be decided by
    # comparing the discarded half with 0x8000 (ties to the even kept half).
    keep = pats >> 16
    rem = pats & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & 1) == 1))
    expect = (keep + up).astype(np.uint16)
    assert np.array_equal(got, expect)
    # and a random sample checked against exact rational rounding
    rng = np.random.default_rng(1)
    sample = rng.choice(f, 400, replace=False)
    for x, g in zip(sample, oracle.f32_to_bf16(sample)):
        assert int(g) == brute_bf16(float(x))


def test_perturb_f32_sign_and_error_bound():
    n = 5000
    rng = np.random.default_rng(2)
    th0 = rng.standard_normal(n).astype(np.float32)
    alpha = 2.0 ** -10
    plane = oracle.gen_plane(0, 3, 5, 128, n)
    z = oracle.signs_from_plane(plane, n)
    th = th0.copy()
    oracle.perturb(th, 128, 0, 3, 5, alpha)
    d = th.astype(np.float64) - th0.astype(np.float64)
    assert np.array_equal(np.sign(d), z)                       # moved along z_j
    exact = th0.astype(np.float64) + alpha * z
    ulp = np.spacing(np.abs(th).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(th - exact) <= 0.5 * ulp)             # one correctly rounded add


def test_perturb_bits_mode_equals_regenerate():
    n = 1000
    rng = np.random.default_rng(3)
    for dt in ("f32", "bf16"):
        base = rng.standard_normal(n).astype(np.float32) * 0.02
        a = base if dt == "f32" else oracle.f32_to_bf16(base)
        b = a.copy()
        oracle.perturb(a, 256, 9, 2, 4, 1e-3)
        oracle.perturb(b, 256, 9, 2, 4, 1e-3, bits=oracle.gen_plane(9, 2, 4, 256, n))
        assert np.array_equal(a, b)


def test_restore_exact_on_dyadic_grid():
    # theta = k * 2^-12 with |theta| < 2^11 and alpha = 2^-10: theta +/- alpha is exact in
    # fp32, so +alpha then -alpha (and -alpha then +alpha) returns the original bits.
    th0 = gen.dyadic_theta(4096, seed=5, frac_bits=12, max_abs_log2=11)
    th = th0.copy()
    a = 2.0 ** -10
    oracle.perturb(th, 0, 0, 0, 1, +a)
    assert not np.array_equal(th, th0)
    oracle.perturb(th, 0, 0, 0, 1, -a)
    oracle.perturb(th, 0, 0, 0, 1, -a)
    oracle.perturb(th, 0, 0, 0, 1, +a)
    assert np.array_equal(th.view(np.uint32), th0.view(np.uint32))


def test_restore_changes_exactly_the_inexact_adds():
    # For |theta| < 8 and alpha = 2^-10 a rounded add theta + alpha*z is inexact only when
    # it crosses up into a coarser binade (or |theta| < alpha); the error is then one ulp
    # of theta's binade, itself representable, so the restore is off by exactly that.  So
    # the elements left changed by +alpha, -alpha are exactly those whose first add was
    # inexact, and they are off by at most half an ulp of |theta| + alpha.
    n = 4096
    rng = np.random.Generator(np.random.PCG64(0))
    th0 = rng.standard_normal(n).astype(np.float32)
    a = 2.0 ** -10
    z = oracle.signs_from_plane(oracle.gen_plane(0, 0, 0, 0, n), n)
    inexact = (th0.astype(np.float32) + np.float32(a) * z.astype(np.float32)).astype(np.float64) \
        != th0.astype(np.float64) + a * z
    th = th0.copy()
    oracle.perturb(th, 0, 0, 0, 0, +a)
    oracle.perturb(th, 0, 0, 0, 0, -a)
    changed = th != th0
    assert np.array_equal(changed, inexact)
    assert changed.sum() > 0
    bound = 0.5 * np.spacing((np.abs(th0) + np.float32(a)).astype(np.float32))
    assert np.all(np.abs(th.astype(np.float64) - th0) <= bound)


def test_perturb_bf16_two_roundings():
    n = 600
    rng = np.random.default_rng(4)
    h0 = oracle.f32_to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    h0[:4] = [0x0001, 0x8001, 0x7F7F, 0x0000]          # subnormals, max finite, zero
    alpha = np.float32(1e-3)
    z = oracle.signs_from_plane(oracle.gen_plane(1, 2, 3, 0, n), n).astype(np.float32)
    h = h0.copy()
    oracle.perturb(h, 0, 1, 2, 3, float(alpha))
    widened = oracle.bf16_to_f32(h0)
    with np.errstate(over="ignore"):
        s32 = widened + alpha * z                       # numpy's IEEE fp32 add
    for j in range(n):
        assert int(h[j]) == brute_bf16(float(s32[j])), j


def test_perturb_nan_inf_denormal():
    th = np.array([np.nan, np.inf, -np.inf, 1e-40, -1e-40, 0.0], dtype=np.float32)
    oracle.perturb(th, 0, 0, 0, 0, 1e-3)
    assert np.isnan(th[0]) and th[1] == np.inf and th[2] == -np.inf
    # denormals are kept (no flush to zero): the add of +/-1e-3 to a denormal is exact to
    # fp32 rounding of the sum
    z = oracle.signs_from_plane(oracle.gen_plane(0, 0, 0, 0, 6), 6)
    for j in (3, 4, 5):
        x0 = np.float32([1e-40, -1e-40, 0.0][j - 3])
        assert th[j] == np.float32(x0 + np.float32(1e-3) * np.float32(z[j]))
    d = np.array([1e-40], dtype=np.float32)
    oracle.perturb(d, 0, 0, 0, 0, 0.0)
    assert d[0] == np.float32(1e-40) and d[0] != 0.0


# ------------------------------------------------------------------------------------
# fused two-probe pass (restore of probe a + move of probe b in one pass)
# ------------------------------------------------------------------------------------
def test_perturb2_reduces_to_single_probe():
    n = 3000
    rng = np.random.default_rng(21)
    for kind in ("f32", "bf16"):
        base = (rng.standard_normal(n) * 0.02).astype(np.float32)
        t0 = base if kind == "f32" else oracle.f32_to_bf16(base)
        # alpha_b = 0: the single-probe move of probe a
        x, y = t0.copy(), t0.copy()
        oracle.perturb2(x, 128, 4, 1, 7, 1e-3, 9, 0.0)
        oracle.perturb(y, 128, 4, 1, 7, 1e-3)
        assert np.array_equal(x, y), kind
        # the same probe twice: one move by 2 alpha
        x, y = t0.copy(), t0.copy()
        oracle.perturb2(x, 0, 4, 1, 7, 1e-3, 7, 1e-3)
        oracle.perturb(y, 0, 4, 1, 7, 2e-3)
        assert np.array_equal(x, y), kind


def test_perturb2_bf16_against_exact_rounding():
    n = 500
    rng = np.random.default_rng(22)
    h0 = oracle.f32_to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    za = oracle.signs_from_plane(oracle.gen_plane(5, 2, 3, 0, n), n).astype(np.float32)
    zb = oracle.signs_from_plane(oracle.gen_plane(5, 2, 4, 0, n), n).astype(np.float32)
    aa, ab = np.float32(1e-3), np.float32(-3e-3)
    h = h0.copy()
    oracle.perturb2(h, 0, 5, 2, 3, float(aa), 4, float(ab))
    d = (aa * za) + (ab * zb)                    # numpy fp32 adds
    t = oracle.bf16_to_f32(h0) + d
    for j in range(n):
        assert int(h[j]) == brute_bf16(float(t[j])), j


def test_s2f_and_s4_visit_the_same_points_on_exact_inputs():
    # On a binary grid every move is exact, so both schedules evaluate the loss at exactly
    # theta +/- eps z_i and leave theta where it started: identical losses and weights.
    M, n = 4096, 12
    rng = np.random.Generator(np.random.PCG64(31))
    th0 = (rng.integers(-4095, 4096, M) / 256.0).astype(np.float32)
    a = (rng.integers(1, 256, M) / 16.0).astype(np.float32)
    lossf = lambda t: oracle.quad_loss(t, a)  # noqa: E731
    out = {}
    for sch in ("S4", "S2f"):
        th = th0.copy()
        out[sch] = oracle.spsa_step(th, seed=3, step=1, npert=n, eps=2.0 ** -8, eta=2.0 ** -12,
                                    delta=1e-6, loss_fn=lossf, schedule=sch)
        out[sch]["theta"] = th
    for k in ("Lp", "Lm", "c", "theta"):
        assert np.array_equal(out["S4"][k], out["S2f"][k]), k
    assert out["S4"]["L0"] == out["S2f"]["L0"]


def test_s2f_bf16_drift_is_bounded():
    # The two-pass schedule, run without an update, leaves bf16 theta within one ulp of
    # |theta| + eps of its start however many probes it runs.
    n = 20000
    rng = np.random.Generator(np.random.PCG64(0))
    h0 = oracle.f32_to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    x0 = oracle.bf16_to_f32(h0).astype(np.float64)
    ulp = np.spacing((np.abs(x0) + 1e-3).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    h = h0.copy()
    L = (np.zeros(64), np.zeros(64))
    oracle.spsa_step(h, seed=0, step=0, npert=64, eps=1e-3, eta=0.0, delta=1e-6,
                     losses=(0.0, L[0], L[1]), schedule="S2f")
    assert np.all(np.abs(oracle.bf16_to_f32(h) - x0) <= ulp)
