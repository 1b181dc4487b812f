"""The seeded input recipes of the workloads: parameter counts of the OPT-shaped sets and
the MLP, and the distribution of the synthetic per-probe losses (the standard deviations
are standard deviations; the +/- pair shares its u_i; every (seed, step) has its own
reproducible draw)."""
import numpy as np

from workloads import CONFIGS, gen, opt_param_count


def test_parameter_counts():
    # per layer 4 d^2 + 2 d F + (9 d + F) biases / layer norms, plus the vocab x d embedding
    assert opt_param_count(40, 5120, 20480, 50272) == 12_842_967_040
    assert opt_param_count(48, 7168, 28672, 50272) == 29_959_831_552
    assert CONFIGS["opt13b"].M == 12_842_967_040 and CONFIGS["opt30b"].M == 29_959_831_552
    e = CONFIGS["mlp"].extra
    assert CONFIGS["mlp"].M == e["d_hid"] * e["d_in"] + e["d_hid"] + e["d_out"] * e["d_hid"] \
        + e["d_out"] == 2_368_514


def test_synthetic_losses_are_reproducible_per_step():
    a = gen.synthetic_losses(0, 5, 160)
    b = gen.synthetic_losses(0, 5, 160)
    c = gen.synthetic_losses(0, 6, 160)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert not np.array_equal(a[1], c[1])


def test_synthetic_loss_statistics():
    n, steps, eps = 160, 400, 1e-3
    half_diff, mid = [], []
    g, h = [], []
    L0s = []
    for s in range(steps):
        L0, Lp, Lm = gen.synthetic_losses(0, s, n)
        L0s.append(L0)
        half_diff.append((Lp - Lm) / 2)          # u_i + (v+_i - v-_i) / 2
        mid.append((Lp + Lm) / 2 - L0)            # (v+_i + v-_i) / 2
        g.append((Lp - Lm) / (2 * eps))
        h.append((Lp + Lm - 2 * L0) / eps ** 2)
    half_diff, mid = np.concatenate(half_diff), np.concatenate(mid)
    g, h = np.concatenate(g), np.concatenate(h)
    N = half_diff.size
    sd_hd = np.sqrt(0.01 ** 2 + 0.001 ** 2 / 2)
    assert abs(half_diff.mean()) < 5 * sd_hd / np.sqrt(N)
    assert abs(half_diff.std() / sd_hd - 1) < 5 / np.sqrt(2 * N)
    sd_mid = 0.001 / np.sqrt(2)
    assert abs(mid.mean() - 0.002) < 5 * sd_mid / np.sqrt(N)
    assert abs(mid.std() / sd_mid - 1) < 5 / np.sqrt(2 * N)
    # the derived weights' scales: g ~ N(0, 10), h ~ 4000 +/- 1414 at eps = 1e-3
    assert abs(g.std() - 10.0) < 0.2 and abs(h.mean() - 4000) < 30 and abs(h.std() - 1414) < 30
    L0s = np.array(L0s)
    assert abs(L0s.mean() - 2.0) < 5 * 0.05 / np.sqrt(steps)
