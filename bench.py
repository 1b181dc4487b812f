#!/usr/bin/env python3
"""Throughput of one 1.5-SPSA step of the perturb / probe-weight / update path on one GPU.

A step (per "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation", sections "How
1.5-SPSA Works" and "Probe-Space Preconditioning") evaluates the loss at the clean
parameters and at theta +/- eps*z_i for each of n_pert probes, moving the parameters in
place between evaluations, then forms the probe weights from the 2 n_pert + 1 losses and
makes one update pass theta <- theta - eta * sum_i c_i z_i.  Schedules of the in-place
moves: S2f (default) -- +eps z_0, then per probe -2 eps z_i and one fused pass restoring
probe i and applying +eps z_(i+1), the last probe's restore folded into the update pass:
2 n_pert passes + the update; S4 -- +eps, restore, -eps, restore per probe: 4 n_pert
passes + the update.  Probes are regenerated from the counter-based generator in every
pass (nothing stored).

Default workload: an OPT-30B-shaped bf16 parameter set (48 layers, d = 7168, FFN 28672,
vocab 50272: 29,959,831,552 params, 59.9 GB) updated in place, n_pert = 160, eps = 1e-3;
theta ~ N(0, 0.02) drawn on the device; per-probe losses synthetic (drawn on the host per
step and uploaded before the timed region).

Prints one JSON line: probe*params/s for the whole job, plus the HBM roofline of the
dominant kernel (the perturb pass) and the CPU oracle timed on a bounded slice.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, vendor figure
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_perturb.json")
PERTURB_SOURCES = ["forward_only_amd/csrc/k_perturb.hip", "forward_only_amd/csrc/zo_device.hpp"]
PHILOX_FILE = os.path.join(ROOT, "profiles", "philox_ceiling.json")
PHILOX_SOURCES = ["forward_only_amd/csrc/zo_device.hpp", "forward_only_amd/ceiling/philox_ceiling.hip"]
UPDATE_VALU_FILE = os.path.join(ROOT, "profiles", "update_valu.json")
UPDATE_SOURCES = ["forward_only_amd/csrc/k_update.hip", "forward_only_amd/csrc/zo_device.hpp",
                  "forward_only_amd/csrc/zo_launch.hpp"]
# VALU issue limit: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 VALU instruction per SIMD every
# 4 cycles (16 lanes per cycle).
PEAK_VALU_WAVE_INSTS = 256 * 4 * 2.4e9 / 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: config's)")
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", default="opt30b",
                   choices=["tiny", "flat125m", "mlp", "lowrank", "opt13b", "opt30b"])
    p.add_argument("--schedule", default="S2f", choices=["S2f", "S4", "fused"],
                   help="S2f: two passes per probe (restore fused with the next probe's "
                        "move); S4: four passes per probe")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle leg (profiling runs)")
    p.add_argument("--no-relocate", action="store_true",
                   help="keep theta on its first allocation (no placement search)")
    p.add_argument("--no-other-sizes", action="store_true",
                   help="with the opt30b headline, skip the opt13b, flat125m and mlp measurements")
    p.add_argument("--cpu-params-per-thread", type=int, default=1 << 20)
    p.add_argument("--cpu-threads", type=int, default=None)
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 4 GiB device copy (counter calibration)")
    return p.parse_args(argv)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str, nbytes_alg: float):
    """HBM bytes per perturb pass from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash(PERTURB_SOURCES) or t.get("workload") != workload:
        return None
    return float(t["bytes_per_pass"])


def stored_philox_peak():
    """Measured Philox4x32-10 calls/s of the generator alone (the ceiling microbenchmark),
    if it was taken on the current generator source; else None."""
    try:
        with open(PHILOX_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash(PHILOX_SOURCES):
        return None
    return float(t["calls_per_s"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded slice of the same workload
# ------------------------------------------------------------------------------------
def cpu_baseline(cfg, params_per_thread: int, threads: int, schedule: str):
    import numpy as np

    import oracle
    from workloads import gen

    L0, Lp, Lm = gen.synthetic_losses(cfg.seed, 0, cfg.npert)
    rng = np.random.default_rng(1234)
    windows = []
    for w in range(threads):
        x = (rng.standard_normal(params_per_thread) * cfg.theta_std).astype(np.float32)
        windows.append(oracle.f32_to_bf16(x) if cfg.dtype == "bf16" else x)
    nblk_total = cfg.M // 128
    offsets = [int(o) * 128 for o in np.linspace(0, nblk_total - params_per_thread // 128 - 1,
                                                 threads).astype(np.int64)]
    oracle.lib()  # build/load outside the timed region

    def run(w):
        oracle.spsa_step(windows[w], seed=cfg.seed, step=0, npert=cfg.npert, eps=cfg.eps,
                         eta=cfg.eta, delta=cfg.delta, losses=(L0, Lp, Lm), offset=offsets[w],
                         schedule=schedule)

    ts = [threading.Thread(target=run, args=(w,)) for w in range(threads)]
    t0 = time.perf_counter()
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    dt = time.perf_counter() - t0
    work = cfg.npert * params_per_thread * threads

    # the same oracle on one core, over a quarter of one window
    n1 = max(128, params_per_thread // 4)
    w1 = windows[0][:n1].copy()
    t1 = time.perf_counter()
    oracle.spsa_step(w1, seed=cfg.seed, step=0, npert=cfg.npert, eps=cfg.eps, eta=cfg.eta,
                     delta=cfg.delta, losses=(L0, Lp, Lm), offset=offsets[0], schedule=schedule)
    dt1 = time.perf_counter() - t1
    return {
        "value": work / dt, "unit": "probe*params/s", "cores": threads, "kind": "oracle",
        "sample": (f"{threads} windows x {params_per_thread} {cfg.dtype} params of the "
                   f"{cfg.name} workload, one full step (n_pert={cfg.npert}, schedule "
                   f"{schedule}, weights, update), one window per thread; {dt:.1f} s"),
        "single_core_value": cfg.npert * n1 / dt1,
        "single_core_sample": f"{n1} params of the first window on one thread; {dt1:.1f} s",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
    }


# ------------------------------------------------------------------------------------
def copy_calibration():
    import torch
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "dispatches": 3}), flush=True)


def stored_update_valu(dtype: str, n: int, restore: bool):
    """VALU instructions per parameter and 8-probe group of the update kernel, from the
    committed rocprofv3 counter summary, if it was taken on the current kernel source and on
    the same kernel form (dtype, probe count, restore folded in or not); else None."""
    try:
        with open(UPDATE_VALU_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("source_sha256") != source_hash(UPDATE_SOURCES) or t.get("dtype") != dtype
            or t.get("n_pert") != n or t.get("restore") != restore):
        return None
    return float(t["valu_insts_per_param_group"])


def update_roofline(M: int, n: int, pass_bytes: float, upd_ms, dtype: str, restore: bool):
    """The update kernel against the VALU issue limit that bounds it (its instruction count
    from the counter summary x the work of one launch / the launch's time), beside its HBM
    bytes (one read and one write of theta) and the Philox calls it makes to regenerate n
    probes' bits (n / 128 per parameter)."""
    if not upd_ms:
        return None
    calls = M * n / 128.0 / (upd_ms * 1e-3)
    peak = stored_philox_peak()
    per = stored_update_valu(dtype, n, restore)
    insts = per * M * ((n + 7) // 8) / 64.0 if per is not None else None
    achieved = insts / (upd_ms * 1e-3) if insts is not None else None
    return {"kernel": "k_update", "bound": "alu",
            "achieved": achieved, "peak": PEAK_VALU_WAVE_INSTS,
            "unit": "wave64 VALU instructions/s",
            "frac": (achieved / PEAK_VALU_WAVE_INSTS) if achieved is not None else None,
            "valu_insts_per_param_group": per,
            "achieved_GBps": pass_bytes / (upd_ms * 1e-3) / 1e9,
            "hbm_frac": pass_bytes / (upd_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "probe_params_per_s": n * M / (upd_ms * 1e-3),
            "philox_calls_per_s": calls, "philox_peak_calls_per_s": peak,
            "philox_frac": (calls / peak) if peak else None}


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", flush=True)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    from workloads import CONFIGS

    cfg = CONFIGS[args.config]
    K = args.steps if args.steps is not None else cfg.steps
    W = args.warmup

    # CPU oracle leg first (host only; keeps the GPU phase uninterrupted).
    cpu = None
    if (not args.no_cpu_baseline and cfg.loss in ("synthetic", "quad")
            and args.schedule in ("S2f", "S4")):
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        log(f"[bench] cpu baseline: {threads} threads x {args.cpu_params_per_thread} params")
        cpu = cpu_baseline(cfg, args.cpu_params_per_thread, threads, args.schedule)
        log(f"[bench] cpu baseline: {cpu['value']:.3e} probe*params/s")

    result = run_workload(args, args.config, K, W, cpu=cpu, gen_plane=True)
    if args.config == "opt30b" and not args.no_other_sizes:
        # the other parameter-set sizes of the same path, measured after the headline (its
        # buffer freed first), each with its own step count and one warmup step
        other = {}
        for key, name, schedule in OTHER_SIZES:
            r = run_workload(args, name, CONFIGS[name].steps, 1, cpu=None, gen_plane=False,
                             schedule=schedule)
            other[key] = {k: r[k] for k in OTHER_KEYS}
        result["other_sizes"] = other
    print(json.dumps(result), flush=True)


# Parameter-set sizes measured beside the 30B headline (record key, workload, schedule; None:
# the workload's own, S2f passes or the MLP's fused forward), and what each reports.
OTHER_SIZES = (("opt13b", "opt13b", None), ("flat125m", "flat125m", None),
               ("flat125m_fused", "flat125m", "fused"), ("mlp", "mlp", None))
OTHER_KEYS = ("value", "unit", "steps", "warmup", "ms_per_step", "ms_per_step_median", "dtype",
              "config", "hbm_gbps", "hbm_frac_of_peak", "kernels_ms", "roofline",
              "pass_roofline", "update_roofline", "nonfinite_probes")


def run_workload(args, name: str, K: int, W: int, cpu=None, gen_plane: bool = True,
                 schedule: str | None = None) -> dict:
    """Time K steps (after W warmup steps) of workload `name` on cuda:0 with `schedule`
    (default: --schedule); returns the bench record (the device memory it used is released
    before it returns)."""
    import numpy as np
    import torch

    import forward_only_amd as zo
    from forward_only_amd import placement
    from forward_only_amd.step import applied_eps
    from workloads import CONFIGS, gen

    cfg = CONFIGS[name]
    n, M = cfg.npert, cfg.M
    esize = 2 if cfg.dtype == "bf16" else 4
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    schedule = schedule or args.schedule
    if schedule == "fused" and cfg.loss != "quad":
        raise SystemExit(f"--schedule fused applies to the quadratic workloads, not {name}")
    ctx = zo.zo_init(cfg.seed)
    log(f"[bench] {cfg.name}: M={M} {cfg.dtype} ({M * esize / 1e9:.2f} GB), n_pert={n}, "
        f"steps={K}, warmup={W}")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    theta = torch.empty(M, dtype=tdt, device=dev)
    a_dev = None
    mlp = None
    if cfg.loss == "mlp":
        e = cfg.extra
        X, y = gen.mlp_data(cfg)
        th0, _ = gen.theta_and_a(cfg)
        theta.copy_(torch.from_numpy(th0))
        mlp = {"X": torch.from_numpy(X).to(dev), "y": torch.from_numpy(y).to(dev),
               "ws": torch.empty(zo.zo_mlp_probes_workspace_bytes(e["batch"], e["d_in"], e["d_hid"],
                                                                  e["d_out"], n),
                                 dtype=torch.uint8,
                                 device=dev), "d_hid": e["d_hid"], "d_out": e["d_out"],
               "flop": 2.0 * e["batch"] * e["d_in"] * e["d_hid"]}
        del th0
    elif cfg.loss == "quad":
        th0, a = gen.theta_and_a(cfg)
        theta.copy_(torch.from_numpy(th0))
        a_dev = torch.from_numpy(a).to(dev)
        del th0, a
    elif cfg.loss == "lowrank":
        th0, a, U = gen.lowrank_problem(cfg)
        theta.copy_(torch.from_numpy(th0))
        a_dev = torch.from_numpy(a).to(dev)
        U_dev = torch.from_numpy(U).to(dev)
        del th0, a, U
    else:
        gen.device_normal_(theta, cfg.theta_std, cfg.seed)
    torch.cuda.synchronize()
    log("[bench] parameters ready")
    relocation = None
    if mlp is None and not args.no_relocate:
        # one-time set-up: keep theta on the fastest of a few allocations (a large buffer's
        # streaming bandwidth depends on the physical memory it lands on)
        theta, relocation = placement.relocate(ctx, theta)
        if not relocation["skipped"]:
            log("[bench] placement search: " + ", ".join(
                f"{r['gbps_whole']:.0f}/{r['gbps_sliced']:.0f}" for r in relocation["tried"]) +
                f" GB/s (one launch / 1 GiB slices); kept allocation {relocation['kept']}")

    total = W + K
    L0s = torch.empty((total, 1), dtype=torch.float64, device=dev)
    Lps = torch.empty((total, n), dtype=torch.float64, device=dev)
    Lms = torch.empty((total, n), dtype=torch.float64, device=dev)
    if cfg.loss == "synthetic":
        for s in range(total):
            l0, lp, lm = gen.synthetic_losses(cfg.seed, s, n)
            L0s[s, 0] = l0
            Lps[s].copy_(torch.from_numpy(lp))
            Lms[s].copy_(torch.from_numpy(lm))
    c_buf = torch.empty(n, dtype=torch.float32, device=dev)
    a = applied_eps(cfg.eps)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    per = {"perturb": [], "perturb2": [], "weights": [], "update": [], "loss": [],
           "mlp_probes": [], "loss_probes": []}

    def timed(kind, fn, record):
        if record:
            e0, e1 = ev(), ev()
            e0.record()
            fn()
            e1.record()
            per[kind].append((e0, e1))
        else:
            fn()

    def loss_into(out, record):
        if cfg.loss == "quad":
            timed("loss", lambda: zo.zo_quad_loss(ctx, theta, a_dev, out=out), record)
        elif cfg.loss == "lowrank":
            timed("loss", lambda: zo.zo_lowrank_quad_loss(ctx, theta, a_dev, U_dev, out=out),
                  record)

    def mlp_probes(op, om, oc, s, record):
        timed("mlp_probes", lambda: zo.zo_mlp_loss_probes(
            ctx, theta, 0, s, 0, n, a, mlp["X"], mlp["y"], mlp["d_hid"], mlp["d_out"],
            workspace=mlp["ws"], out_plus=op, out_minus=om, out_clean=oc), record)

    def one_step(s, record):
        L0, Lp, Lm = L0s[s], Lps[s], Lms[s]
        if mlp is not None:
            # the forward applies each probe while reading the weights: no passes over
            # theta; one launch sequence gives both losses of every probe and the clean loss
            mlp_probes(Lp, Lm, L0, s, record)
            timed("weights", lambda: zo.zo_probe_weights(ctx, Lp, Lm, L0, a, cfg.delta,
                                                         out=c_buf), record)
            timed("update", lambda: zo.zo_update(ctx, theta, 0, s, c_buf, cfg.eta), record)
            return
        if schedule == "fused":
            # each probe applied while theta and a are read (four probes per pass, the first
            # pass also summing the clean loss), theta written only by the update
            timed("loss_probes", lambda: zo.zo_quad_loss_probes(
                ctx, theta, a_dev, 0, s, 0, n, a, out_plus=Lp, out_minus=Lm, out_clean=L0),
                record)
            timed("weights", lambda: zo.zo_probe_weights(ctx, Lp, Lm, L0, a, cfg.delta,
                                                         out=c_buf), record)
            timed("update", lambda: zo.zo_update(ctx, theta, 0, s, c_buf, cfg.eta), record)
            return
        loss_into(L0, record)
        if schedule == "S4":
            for i in range(n):
                timed("perturb", lambda: zo.zo_perturb(ctx, theta, 0, s, i, +a), record)
                loss_into(Lp[i:i + 1], record)
                timed("perturb", lambda: zo.zo_perturb(ctx, theta, 0, s, i, -a), record)
                timed("perturb", lambda: zo.zo_perturb(ctx, theta, 0, s, i, -a), record)
                loss_into(Lm[i:i + 1], record)
                timed("perturb", lambda: zo.zo_perturb(ctx, theta, 0, s, i, +a), record)
        else:
            timed("perturb", lambda: zo.zo_perturb(ctx, theta, 0, s, 0, +a), record)
            for i in range(n):
                loss_into(Lp[i:i + 1], record)
                timed("perturb", lambda: zo.zo_perturb(ctx, theta, 0, s, i, -2.0 * a), record)
                loss_into(Lm[i:i + 1], record)
                if i + 1 < n:
                    timed("perturb2",
                          lambda: zo.zo_perturb2(ctx, theta, 0, s, i, +a, i + 1, +a), record)
        timed("weights", lambda: zo.zo_probe_weights(ctx, Lp, Lm, L0, a, cfg.delta, out=c_buf),
              record)
        if schedule == "S2f":
            # the last probe's restore rides on the update pass
            timed("update", lambda: zo.zo_restore_update(ctx, theta, 0, s, n - 1, +a, c_buf,
                                                         cfg.eta), record)
        else:
            timed("update", lambda: zo.zo_update(ctx, theta, 0, s, c_buf, cfg.eta), record)

    # The in-place ceiling of the memory theta landed on (a large buffer's bandwidth depends
    # on its physical placement): a pass that reads and writes back theta unchanged, in the
    # perturb kernel's order, timed before the warmup.
    placement_gbps = None
    tune = None
    if mlp is None:
        # one-time choice, on this very buffer, between one launch per pass and launches per
        # 1 GiB slice (contents unchanged); the passes below use the faster form
        tune = zo.zo_tune_placement(ctx, theta)
        log(f"[bench] placement: one launch {tune['gbps_whole']:.0f} GB/s, 1 GiB slices "
            f"{tune['gbps_sliced']:.0f} GB/s -> slice_bytes {tune['slice_bytes']}")
        zo.zo_stream_rmw(ctx, theta)
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(3):
            zo.zo_stream_rmw(ctx, theta)
        e1.record()
        torch.cuda.synchronize()
        placement_gbps = 2.0 * esize * M / (e0.elapsed_time(e1) / 3 * 1e-3) / 1e9
        log(f"[bench] in-place ceiling of theta's memory: {placement_gbps:.0f} GB/s")

    for s in range(W):
        one_step(s, False)
        torch.cuda.synchronize()
        log(f"[bench] warmup step {s} done")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_marks = [ev()]
    step_marks[0].record()
    for s in range(W, total):
        one_step(s, True)
        step_marks.append(ev())
        step_marks[-1].record()     # step boundary on the launch stream (no host sync)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log(f"[bench] {K} timed steps done in {t1 - t0:.2f} s")

    # The packed-plane generator (the step regenerates bits inline; planes serve callers
    # that store them): one probe's plane over the whole buffer, timed after the step.
    gen_probes = None
    if mlp is None and gen_plane:
        stride = zo.zo_bits_stride(M)
        plane = torch.empty((1, stride), dtype=torch.uint8, device=dev)
        zo.zo_gen_probes(ctx, 0, 0, 1, 0, M, out=plane)
        g0, g1 = ev(), ev()
        g0.record()
        for i in range(3):
            zo.zo_gen_probes(ctx, 0, i, 1, 0, M, out=plane)
        g1.record()
        torch.cuda.synchronize()
        gen_s = g0.elapsed_time(g1) / 3 * 1e-3
        gen_probes = {"kernel": "k_gen_probes", "bound": "hbm", "plane_bytes": stride,
                      "achieved_GBps": stride / gen_s / 1e9,
                      "frac": stride / gen_s / 1e9 / PEAK_HBM_GBPS,
                      "philox_calls_per_s": (stride // 16) / gen_s}
        del plane
    nonfinite = zo.zo_nonfinite_count(ctx)

    def times(kinds):
        return [e0.elapsed_time(e1) for k in kinds for e0, e1 in per[k]]

    def avg_ms(*kinds):
        xs = times(kinds)
        return (sum(xs) / len(xs)) if xs else None

    T = (t1 - t0) / K
    value = n * M / T
    step_ms = sorted(a.elapsed_time(b) for a, b in zip(step_marks, step_marks[1:]))
    median_ms = (step_ms[K // 2] if K % 2 else 0.5 * (step_ms[K // 2 - 1] + step_ms[K // 2]))
    kernel_ms_per_step = sum(times(list(per))) / K     # sum of every timed kernel call
    # every pass of either perturb entry point runs k_perturb_chunks (one or two probes)
    pert_ms, upd_ms, w_ms = avg_ms("perturb", "perturb2"), avg_ms("update"), avg_ms("weights")
    passes = 0 if mlp is not None or schedule == "fused" else (4 * n if schedule == "S4" else 2 * n)
    pass_bytes = 2.0 * esize * M                      # one read + one write of theta
    step_bytes = (passes + 1) * pass_bytes            # the passes + the update
    if schedule == "fused":                           # + the fused passes (the first one also
        step_bytes += ((n + 3) // 4) * float(esize + 4) * M   # sums the clean loss)
    pass_roofline = None
    if pert_ms:
        pa = pass_bytes / (pert_ms * 1e-3) / 1e9
        pass_roofline = {"kernel": "k_perturb_chunks", "bound": "hbm", "achieved": pa,
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": pa / PEAK_HBM_GBPS,
                         "bytes_per_pass": pass_bytes}
    if schedule == "fused":
        lp_ms = avg_ms("loss_probes")
        npass = (n + 3) // 4
        fb = npass * float(esize + 4) * M              # theta and a read once per 4 probes
        fa = fb / (lp_ms * 1e-3) / 1e9
        achieved = fa
        roofline = {"kernel": "k_quad_probes_partial (the quadratic loss at theta +/- alpha z "
                              "of four probes per pass, theta and a read once, the first pass "
                              "also summing the clean loss; time of the whole "
                              f"zo_quad_loss_probes call: {npass} passes and their sums)",
                    "bound": "hbm", "achieved": fa, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": fa / PEAK_HBM_GBPS, "traffic": None,
                    "losses_per_s": (2.0 * n + 1.0) / (lp_ms * 1e-3),
                    "note": "measured against HBM, but held by VALU issue: 13 fp64 operations "
                            "per param keep each loss equal to the fp64 loss kernel's; counters "
                            "show 82-84% of the VALU issue slots used, and the loads alone run "
                            "at 6.6 TB/s (profiles/flat125m_fused_kernel_trace_and_traffic.md)"}
    elif mlp is not None:
        mlp_ms = avg_ms("mlp_probes")
        achieved = (2.0 * n + 1.0) * mlp["flop"] / (mlp_ms * 1e-3) / 1e12
        roofline = {"kernel": "k_mlp_tiles (MFMA fp32 GEMM of the MLP forward, both signs of "
                              "up to 64 probes per launch sequence and the clean loss; time "
                              "of the whole zo_mlp_loss_probes call: tiles, row and mean "
                              "kernels of all n_pert probes' 2 n_pert + 1 forwards)",
                    "bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
                    "traffic": None,
                    "note": "peak at 2.4 GHz; under this load the counters give a clock near "
                            "2.11 GHz (GRBM_GUI_ACTIVE over the dispatch), where the fp32 "
                            "MFMA peak is about 138 TFLOP/s; MFMA busy 68% and VALU issue 25% "
                            "(profiles/k_mlp_tiles_mlp_trace_and_counters.md)"}
    else:
        achieved = pass_bytes / (pert_ms * 1e-3) / 1e9 if pert_ms else None
        roofline = None
        loss_times = times(["loss"])
        if loss_times and sum(loss_times) > sum(times(["perturb", "perturb2"])):
            # the loss evaluations dominate: theta, a (and U) read once per evaluation
            r = cfg.extra.get("rank", 0) if cfg.loss == "lowrank" else 0
            loss_bytes = float(esize + 4 + 4 * r) * M
            la = loss_bytes / (sum(loss_times) / len(loss_times) * 1e-3) / 1e9
            roofline = {"kernel": ("k_lowrank_partial" if r else "k_quad_loss_partial") +
                                  " (loss evaluation, fp64 accumulation)",
                        "bound": "hbm", "achieved": la, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": la / PEAK_HBM_GBPS, "traffic": None,
                        "note": f"{loss_bytes / 1e6:.0f} MB per evaluation; partly resident in "
                                f"the 256 MB last-level cache"}
    traffic = stored_traffic(f"{cfg.name}/{schedule}", pass_bytes)
    result = {
        "metric": "probe*params/s and HBM GB/s (% peak) per 1.5-SPSA step, n_pert=160, 1 GPU",
        "value": value,
        "unit": "probe*params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": T * 1e3,
        "ms_per_step_median": median_ms,
        "kernel_ms_per_step": kernel_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: {M} {cfg.dtype} params in one flat buffer, "
                                f"n_pert={n}, eps={cfg.eps}, eta={cfg.eta}, " +
                                ("probes applied inside the MFMA forward, both signs of up to 64 "
                                 "probes and the clean loss per launch sequence (no passes over "
                                 "theta) + update"
                                 if mlp is not None else
                                 "probes applied while theta is read, four per pass of the "
                                 "quadratic loss, the clean loss in the first pass (no passes "
                                 "that write theta) + update"
                                 if schedule == "fused" else
                                 f"schedule {schedule} ({passes} passes + update" +
                                 (" carrying the last restore)" if schedule == "S2f"
                                  else ")")) +
                                ", probes regenerated, losses " +
                                ("synthetic" if cfg.loss == "synthetic" else cfg.loss)),
                   "params": M, "n_pert": n,
                   "schedule": ("fused forward" if mlp is not None or schedule == "fused"
                                else schedule),
                   "passes_per_step": passes + 1},
        "hbm_gbps": step_bytes / T / 1e9,
        "hbm_frac_of_peak": step_bytes / T / 1e9 / PEAK_HBM_GBPS,
        "kernels_ms": {"pass_avg": pert_ms, "perturb_avg": avg_ms("perturb"),
                       "perturb2_avg": avg_ms("perturb2"), "update_avg": upd_ms,
                       "weights_avg": w_ms, "loss_avg": avg_ms("loss"),
                       "mlp_probes_avg": avg_ms("mlp_probes"),
                       "loss_probes_avg": avg_ms("loss_probes")},
        "roofline": roofline or {"kernel": f"k_perturb_chunks ({cfg.dtype}, probes regenerated; "
                                           f"every zo_perturb / zo_perturb2 pass)",
                                 "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                                 "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                                 "traffic": traffic,
                                 "placement_ceiling": placement_gbps,
                                 "placement_tuning": tune,
                                 "placement_relocation": relocation,
                                 "frac_of_placement_ceiling": (achieved / placement_gbps
                                                               if placement_gbps else None)},
        "pass_roofline": pass_roofline,
        "update_roofline": update_roofline(M, n, pass_bytes, upd_ms, cfg.dtype,
                                           mlp is None and schedule == "S2f"),
        "gen_probes": gen_probes,
        "nonfinite_probes": nonfinite,
        "cpu_baseline": cpu,
    }
    ctx.close()
    del theta, L0s, Lps, Lms, c_buf, a_dev, mlp, per, step_marks
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


if __name__ == "__main__":
    main()
