"""One 1.5-SPSA step on the GPU, sequenced from the C entry points.

Order of work ("Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation", sections "How
1.5-SPSA Works" and "Probe-Space Preconditioning"; the ZOO loop flowchart of "Pretraining
Transformers Without Backprop: What Two Zero-Order Papers Actually Measure"): the clean
loss, then per probe four in-place passes +eps, -eps (restore), -eps, +eps (restore) with
a loss after the first and third, then the probe weights, then one update pass.

schedule="S2f" makes two passes per probe: +eps z_0, then per probe a -2 eps z_i pass (to
theta - eps z_i) and one fused pass (zo_perturb2) that restores probe i and applies
+eps z_(i+1); the last probe's restore is folded into the update pass (zo_restore_update),
which nothing reads in between (the weights read only the losses).  Its points are S4's
exactly where every move is exact (e.g. dyadic fp32 values); otherwise each pass rounds
once from where the previous one left theta -- in bf16 the -eps point is
rnd(rnd(theta + eps z) - 2 eps z), not S4's rnd(theta - eps z) -- so the points may differ
from S4's by rounding.

Python only orders the launches; every pass over the parameters, the weights and the
update run in libzo's kernels on torch's current stream.  Losses stay on the device.
"""
from __future__ import annotations

import numpy as np
import torch

from . import zo_perturb, zo_perturb2, zo_probe_weights, zo_restore_update, zo_update


def applied_eps(eps: float) -> float:
    """The step the passes really add: eps rounded to fp32."""
    return float(np.float32(eps))


def spsa_step(ctx, theta: torch.Tensor, *, step: int, npert: int, eps: float, eta: float,
              delta: float, loss=None, losses=None, offset: int = 0, bits=None,
              buffers: dict | None = None, schedule: str = "S4") -> dict:
    """Run one step in place on `theta`.

    loss(theta, out) writes the loss at `theta` into the one-element float64 GPU tensor
    `out`; alternatively `losses` = (L0[1], Lp[n], Lm[n]) float64 GPU tensors supply them
    (synthetic or measured elsewhere) and the perturb / restore passes still run.
    bits: optional (npert, stride) uint8 GPU tensor of packed rows (else regenerated).
    Returns the device tensors L0, Lp, Lm and c.
    """
    a = applied_eps(eps)
    b = buffers if buffers is not None else {}
    if losses is not None:
        L0, Lp, Lm = losses
    else:
        L0 = b.get("L0")
        if L0 is None:
            L0 = torch.empty(1, dtype=torch.float64, device=theta.device)
        Lp = b.get("Lp")
        if Lp is None:
            Lp = torch.empty(npert, dtype=torch.float64, device=theta.device)
        Lm = b.get("Lm")
        if Lm is None:
            Lm = torch.empty(npert, dtype=torch.float64, device=theta.device)
        loss(theta, L0)
    row = (lambda i: None) if bits is None else (lambda i: bits[i])
    if schedule == "S4":
        for i in range(npert):
            zo_perturb(ctx, theta, offset, step, i, +a, row(i))
            if losses is None:
                loss(theta, Lp[i:i + 1])
            zo_perturb(ctx, theta, offset, step, i, -a, row(i))
            zo_perturb(ctx, theta, offset, step, i, -a, row(i))
            if losses is None:
                loss(theta, Lm[i:i + 1])
            zo_perturb(ctx, theta, offset, step, i, +a, row(i))
    elif schedule == "S2f":
        if npert > 0:
            zo_perturb(ctx, theta, offset, step, 0, +a, row(0))
        for i in range(npert):
            if losses is None:
                loss(theta, Lp[i:i + 1])
            zo_perturb(ctx, theta, offset, step, i, -2.0 * a, row(i))
            if losses is None:
                loss(theta, Lm[i:i + 1])
            if i + 1 < npert:
                zo_perturb2(ctx, theta, offset, step, i, +a, i + 1, +a, row(i), row(i + 1))
    else:
        raise ValueError(f"unknown schedule {schedule!r}")
    c = zo_probe_weights(ctx, Lp, Lm, L0, a, delta, out=b.get("c"))
    if schedule == "S2f" and npert > 0:
        zo_restore_update(ctx, theta, offset, step, npert - 1, +a, c, eta, bits)
    else:
        zo_update(ctx, theta, offset, step, c, eta, bits)
    return {"L0": L0, "Lp": Lp, "Lm": Lm, "c": c}


def spsa_step_fused(ctx, theta: torch.Tensor, *, step: int, npert: int, eps: float, eta: float,
                    delta: float, loss_at=None, offset: int = 0, bits=None,
                    buffers: dict | None = None, loss_pair_at=None,
                    loss_probes_at=None, probes_give_clean: bool = False) -> dict:
    """One step whose forward applies each probe while reading the parameters.

    loss_at(probe, alpha, row, out) writes the loss at theta + alpha * z_probe (probe None:
    the clean loss) into `out`; theta itself is only written by the update.  Used with
    zo_mlp_loss_perturbed: no perturb or restore pass over the parameters at all.  With
    loss_pair_at(probe, alpha, row, out_plus, out_minus) (zo_mlp_loss_pair) each probe's two
    losses come from one call; with loss_probes_at(probe0, n, alpha, rows, out_plus,
    out_minus) (zo_mlp_loss_probes) all probes' losses come from one call; with
    probes_give_clean it is called with a seventh argument, the clean loss's output, which it
    fills from the same call (the out_clean of zo_mlp_loss_probes / zo_quad_loss_probes), and
    loss_at is not called (it may be None then; otherwise it is required).
    """
    if loss_at is None and not (loss_probes_at is not None and probes_give_clean):
        raise ValueError("loss_at is required unless loss_probes_at gives the clean loss")
    a = applied_eps(eps)
    b = buffers if buffers is not None else {}
    dev = theta.device
    L0 = b.get("L0") if b.get("L0") is not None else torch.empty(1, dtype=torch.float64, device=dev)
    Lp = b.get("Lp") if b.get("Lp") is not None else torch.empty(npert, dtype=torch.float64, device=dev)
    Lm = b.get("Lm") if b.get("Lm") is not None else torch.empty(npert, dtype=torch.float64, device=dev)
    if loss_probes_at is not None and probes_give_clean:
        loss_probes_at(0, npert, +a, bits, Lp, Lm, L0)
    else:
        loss_at(None, 0.0, None, L0)
        if loss_probes_at is not None and npert > 0:
            loss_probes_at(0, npert, +a, bits, Lp, Lm)
    for i in range(npert if loss_probes_at is None else 0):
        row = None if bits is None else bits[i]
        if loss_pair_at is not None:
            loss_pair_at(i, +a, row, Lp[i:i + 1], Lm[i:i + 1])
        else:
            loss_at(i, +a, row, Lp[i:i + 1])
            loss_at(i, -a, row, Lm[i:i + 1])
    c = zo_probe_weights(ctx, Lp, Lm, L0, a, delta, out=b.get("c"))
    zo_update(ctx, theta, offset, step, c, eta, bits)
    return {"L0": L0, "Lp": Lp, "Lm": Lm, "c": c}
