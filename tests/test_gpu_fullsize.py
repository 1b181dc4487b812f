"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The whole parameter buffer goes through the same calls the benchmark makes (zo_perturb,
zo_perturb2, and zo_restore_update -- the update carrying a restore -- on the full buffer,
probes regenerated); 64 random windows of 2^20 parameters, the first window, the last one
(which ends at the buffer's ragged end) and one straddling the perturb kernel's last whole
chunk are copied to the host before and after and recomputed by the oracle from their
global offsets -- the probe bits are counter-based, so a window is an exact sub-problem.
Passes are compared bit for bit, the update within the update tolerance (fp32) or one bf16
ulp.  The oracle runs the windows on a pool of host threads.

Properties that hold at any size are checked on every element of the 30B buffer: the
drift bound of a whole two-pass step, the agreement of the three routes to a probe's signs
(update, perturb, packed plane), and the restore-carrying update against the two calls.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import forward_only_amd as zo
import oracle
from gpu_util import assert_bf16_within_ulp, assert_f32_update_close, bf16_bits
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu

WIN = 1 << 20
N_RANDOM = 64
THREADS = 16


def _windows(M, k, seed, extra_starts=()):
    """(start, length) of k random windows, the first, the last and the extra ones; starts
    are multiples of 128 (whole probe blocks), the last window runs to M."""
    rng = np.random.default_rng(seed)
    nblk = M // 128
    starts = set((rng.integers(1, nblk - WIN // 128 - 1, k) * 128).tolist())
    starts |= {0, (M // 8192) * 8192 - 4096}
    starts |= set(extra_starts)
    last = ((M - WIN) // 128) * 128
    wins = [(s, WIN) for s in sorted(starts) if 0 <= s and s + WIN <= last]
    wins.append((last, M - last))
    return wins


def _take(t, wins, kind):
    out = []
    for s, n in wins:
        w = t[s:s + n]
        out.append(w.cpu().numpy().copy() if kind == "f32" else bf16_bits(w).copy())
    return out


def _run_and_check(t, M, kind, seed, npert, eps, eta, label, slice_bytes=0, extra_starts=()):
    wins = _windows(M, N_RANDOM, seed=M % 1000, extra_starts=extra_starts)
    assert len(wins) >= N_RANDOM - 2 and wins[0][0] == 0 and sum(wins[-1]) == M
    before = _take(t, wins, kind)
    ctx = zo.zo_init(seed)
    zo.zo_set_slice_bytes(ctx, slice_bytes)
    a = float(np.float32(eps))
    c = (np.random.default_rng(7).standard_normal(npert) * 2.5e-3).astype(np.float32)
    print(f"[fullsize] {label}: M={M} passes, {len(wins)} windows", flush=True)
    zo.zo_perturb(ctx, t, 0, 1, 0, +a)
    zo.zo_perturb(ctx, t, 0, 1, 0, -2.0 * a)
    zo.zo_perturb2(ctx, t, 0, 1, 0, +a, 1, +a)
    torch.cuda.synchronize()
    after_passes = _take(t, wins, kind)
    print(f"[fullsize] {label}: restore + update n_pert={npert}", flush=True)
    zo.zo_restore_update(ctx, t, 0, 1, 1, -a, torch.from_numpy(c).cuda(), eta)
    torch.cuda.synchronize()
    after_update = _take(t, wins, kind)
    ctx.close()
    view = np.uint32 if kind == "f32" else np.uint16

    def recompute(i):
        s = wins[i][0]
        h = before[i].copy()
        oracle.perturb(h, s, seed, 1, 0, +a)
        oracle.perturb(h, s, seed, 1, 0, -2.0 * a)
        oracle.perturb2(h, s, seed, 1, 0, +a, 1, +a)
        passes = h.copy()
        oracle.perturb(h, s, seed, 1, 1, -a)
        oracle.update(h, s, seed, 1, c, eta)
        return passes, h

    print(f"[fullsize] {label}: oracle on {len(wins)} windows", flush=True)
    with cf.ThreadPoolExecutor(THREADS) as ex:
        refs = list(ex.map(recompute, range(len(wins))))
    for (s, _), hp, hu, (rp, ru) in zip(wins, after_passes, after_update, refs):
        assert np.array_equal(rp.view(view), hp.view(view)), (label, s)
        if kind == "f32":
            assert_f32_update_close(hu, ru, eta, c)
        else:
            assert_bf16_within_ulp(hu, ru)
    return len(wins)


def test_flat125m_full_size():
    cfg = CONFIGS["flat125m"]
    th0, _ = gen.theta_and_a(cfg)
    t = torch.from_numpy(th0).cuda()
    del th0
    n = _run_and_check(t, cfg.M, "f32", cfg.seed, cfg.npert, cfg.eps, cfg.eta, "flat125m")
    assert n >= N_RANDOM


@pytest.mark.parametrize("name", ["opt13b", "opt30b"])
def test_opt_shaped_bf16_full_size(name):
    cfg = CONFIGS[name]
    t = torch.empty(cfg.M, dtype=torch.bfloat16, device="cuda")
    gen.device_normal_(t, cfg.theta_std, cfg.seed)
    n = _run_and_check(t, cfg.M, "bf16", cfg.seed, cfg.npert, cfg.eps, 1.0, name)
    assert n >= N_RANDOM
    del t
    torch.cuda.empty_cache()


def test_opt30b_largest_probe_count():
    """The update at its largest probe count (ZO_MAX_NPERT = 512: 64 sign tables, 128 KiB of
    LDS per workgroup) over the whole 30B buffer, with the restore of the last probe
    folded in, against the oracle on the sampled windows."""
    cfg = CONFIGS["opt30b"]
    t = torch.empty(cfg.M, dtype=torch.bfloat16, device="cuda")
    gen.device_normal_(t, cfg.theta_std, cfg.seed)
    n = _run_and_check(t, cfg.M, "bf16", cfg.seed, int(zo.ZO_MAX_NPERT), cfg.eps, 1.0,
                       "opt30b n_pert=512")
    assert n >= N_RANDOM
    del t
    torch.cuda.empty_cache()


def test_opt30b_full_step_drift_without_update():
    """One whole two-pass step over the 30B buffer (160 probes: 320 passes, then the update
    carrying the last restore) with eta = 0, so the update adds exactly zero: every bf16
    parameter must end within one bf16 ulp of |theta| + eps of where it started -- the
    drift bound of the schedule, checked on all 29,959,831,552 elements rather than on
    windows.  Each pass is one rounding, so some elements do move."""
    from forward_only_amd.step import spsa_step
    cfg = CONFIGS["opt30b"]
    t = torch.empty(cfg.M, dtype=torch.bfloat16, device="cuda")
    gen.device_normal_(t, cfg.theta_std, cfg.seed)
    t0 = t.clone()
    L0, Lp, Lm = gen.synthetic_losses(cfg.seed, 0, cfg.npert)
    dl = (torch.tensor([L0], dtype=torch.float64, device="cuda"),
          torch.from_numpy(Lp).cuda(), torch.from_numpy(Lm).cuda())
    ctx = zo.zo_init(cfg.seed)
    print("[fullsize] opt30b: full S2f step, eta = 0", flush=True)
    spsa_step(ctx, t, step=0, npert=cfg.npert, eps=cfg.eps, eta=0.0, delta=cfg.delta,
              losses=dl, schedule="S2f")
    torch.cuda.synchronize()
    ctx.close()
    bad = changed = 0
    chunk = 1 << 30
    for i in range(0, cfg.M, chunk):
        a = t0[i:i + chunk].float()
        b = t[i:i + chunk].float()
        _, e = torch.frexp(a.abs() + 1e-3)
        ulp = torch.ldexp(torch.ones_like(a), e - 8)          # bf16 spacing of |theta| + eps
        bad += int(((b - a).abs() > ulp).sum())
        changed += int((b != a).sum())
        del a, b, e, ulp
    del t, t0
    torch.cuda.empty_cache()
    assert bad == 0, bad
    assert 0.01 * cfg.M < changed < 0.6 * cfg.M, changed / cfg.M


def test_opt30b_update_and_perturb_signs_agree_everywhere():
    """Over the whole 30B buffer, the signs the update regenerates equal the signs the
    perturb pass regenerates and the bits of the packed plane: from theta = 0, one-hot
    weights at probe k with eta = -1 give theta = z_k, and so does a perturb by +1 (bf16
    holds +/-1 exactly); the plane's bit j is 1 exactly where z_k,j = +1.  Probe k sits in
    the last sign group of the 160."""
    cfg = CONFIGS["opt30b"]
    k = 157
    ctx = zo.zo_init(cfg.seed)
    a = torch.zeros(cfg.M, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(cfg.npert, dtype=torch.float32, device="cuda")
    c[k] = 1.0
    print("[fullsize] opt30b: update signs", flush=True)
    zo.zo_update(ctx, a, 0, 3, c, -1.0)
    b = torch.zeros(cfg.M, dtype=torch.bfloat16, device="cuda")
    print("[fullsize] opt30b: perturb signs", flush=True)
    zo.zo_perturb(ctx, b, 0, 3, k, 1.0)
    print("[fullsize] opt30b: plane", flush=True)
    plane = zo.zo_gen_probes(ctx, 3, k, 1, 0, cfg.M)[0]
    torch.cuda.synchronize()
    ctx.close()
    chunk = 1 << 31
    same = all(torch.equal(a[i:i + chunk], b[i:i + chunk]) for i in range(0, cfg.M, chunk))
    ones = int((a[: 1 << 24].float().abs() == 1.0).sum())
    shifts = torch.arange(8, dtype=torch.uint8, device="cuda")
    plane_ok = True
    for i in range(0, cfg.M, chunk):             # chunk is a multiple of 8
        m = min(chunk, cfg.M - i)
        bytes_ = plane[i // 8:(i + m + 7) // 8]
        bits = ((bytes_.unsqueeze(1) >> shifts) & 1).reshape(-1)[:m]
        plane_ok &= torch.equal(bits.bool(), b[i:i + m] > 0)
        del bits
    del a, b, plane
    torch.cuda.empty_cache()
    assert same
    assert plane_ok
    assert ones == 1 << 24                      # every element is +/-1


def test_opt30b_restore_update_equals_two_calls_everywhere():
    """zo_restore_update is zo_perturb followed by zo_update bit for bit, on every element
    of the 30B buffer (n_pert = 160, eta = 1 so that the bf16 update moves parameters)."""
    cfg = CONFIGS["opt30b"]
    a = torch.empty(cfg.M, dtype=torch.bfloat16, device="cuda")
    gen.device_normal_(a, cfg.theta_std, cfg.seed)
    b = a.clone()
    c = torch.from_numpy((np.random.default_rng(9).standard_normal(cfg.npert) * 2.5e-3)
                         .astype(np.float32)).cuda()
    alpha = float(np.float32(cfg.eps))
    ctx = zo.zo_init(cfg.seed)
    print("[fullsize] opt30b: restore + update, fused and as two calls", flush=True)
    zo.zo_restore_update(ctx, a, 0, 4, cfg.npert - 1, alpha, c, 1.0)
    zo.zo_perturb(ctx, b, 0, 4, cfg.npert - 1, alpha)
    zo.zo_update(ctx, b, 0, 4, c, 1.0)
    torch.cuda.synchronize()
    ctx.close()
    chunk = 1 << 31
    same = all(torch.equal(a[i:i + chunk].view(torch.int16), b[i:i + chunk].view(torch.int16))
               for i in range(0, cfg.M, chunk))
    del a, b
    torch.cuda.empty_cache()
    assert same


def test_opt30b_passes_in_slices():
    """The bench's calls with the passes issued per 1 GiB slice (the form zo_tune_placement
    picks on slow placements), with windows straddling slice boundaries."""
    cfg = CONFIGS["opt30b"]
    t = torch.empty(cfg.M, dtype=torch.bfloat16, device="cuda")
    gen.device_normal_(t, cfg.theta_std, cfg.seed)
    per = (1 << 30) // 2                                    # params per slice
    extra = [per - WIN // 2, 17 * per - WIN // 2, (cfg.M // per) * per - WIN // 2]
    assert 17 * per < cfg.M
    assert all(x % 128 == 0 for x in extra)
    n = _run_and_check(t, cfg.M, "bf16", cfg.seed, cfg.npert, cfg.eps, 1.0, "opt30b sliced",
                       slice_bytes=1 << 30, extra_starts=extra)
    assert n >= N_RANDOM
    del t
    torch.cuda.empty_cache()

