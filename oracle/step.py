"""One 1.5-SPSA step on the CPU, built from the oracle's primitives.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Order of work ("Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation", sections
"How 1.5-SPSA Works" and "Probe-Space Preconditioning"; the ZOO training-loop flowchart
of "Pretraining Transformers Without Backprop: What Two Zero-Order Papers Actually
Measure"):

  1. the clean loss L0 at the unperturbed parameters;
  2. for each probe i: perturb to theta + eps*z_i, loss L+_i, restore; perturb to
     theta - eps*z_i, loss L-_i, restore.  Each move is one in-place pass, so the
     schedule is +eps, -eps (restore), -eps, +eps (restore): four passes per probe;
  3. the probe weights c_i from (L+_i, L-_i, L0);
  4. the update theta <- theta - eta * sum_i c_i z_i.

The eps handed to the weights is the fp32 value that the passes actually added.

schedule="none" runs no passes at all (the losses must be given): the step of a forward
that applies the probe on the fly while reading the parameters, leaving them untouched.

schedule="S2f" makes two passes per probe instead of four: +eps z_0; then for each i a
pass of -2 eps z_i (to theta - eps z_i) and a fused pass that restores probe i and applies
+eps z_(i+1) (the last one only restores).  Each pass rounds once from where the previous
one left theta, so its points equal S4's only where every move is exact; in bf16 its -eps
point is rnd(rnd(theta + eps z) - 2 eps z) rather than S4's rnd(theta - eps z).
"""
from __future__ import annotations

import numpy as np


def spsa_step(theta: np.ndarray, *, seed: int, step: int, npert: int, eps: float,
              eta: float, delta: float, loss_fn=None, losses=None, offset: int = 0,
              bits=None, schedule: str = "S4") -> dict:
    """Run one step in place on `theta` (float32, or uint16 bf16 bits).

    loss_fn(theta) -> float gives the losses; alternatively `losses` = (L0, Lp, Lm)
    supplies them (synthetic losses, or losses measured elsewhere), and the perturb and
    restore passes still run.  bits: optional (npert, plane_bytes) packed rows.
    """
    from . import perturb, perturb2, probe_weights, update  # late import: package init order

    a = float(np.float32(eps))
    if losses is not None:
        L0, Lp, Lm = float(losses[0]), np.array(losses[1], dtype=np.float64), \
            np.array(losses[2], dtype=np.float64)
    else:
        L0 = float(loss_fn(theta))
        Lp = np.zeros(npert, dtype=np.float64)
        Lm = np.zeros(npert, dtype=np.float64)
    row = (lambda i: None) if bits is None else (lambda i: bits[i])
    if schedule == "S4":
        for i in range(npert):
            perturb(theta, offset, seed, step, i, +a, row(i))
            if losses is None:
                Lp[i] = loss_fn(theta)
            perturb(theta, offset, seed, step, i, -a, row(i))
            perturb(theta, offset, seed, step, i, -a, row(i))
            if losses is None:
                Lm[i] = loss_fn(theta)
            perturb(theta, offset, seed, step, i, +a, row(i))
    elif schedule == "S2f":
        if npert > 0:
            perturb(theta, offset, seed, step, 0, +a, row(0))
        for i in range(npert):
            if losses is None:
                Lp[i] = loss_fn(theta)
            perturb(theta, offset, seed, step, i, -2.0 * a, row(i))
            if losses is None:
                Lm[i] = loss_fn(theta)
            if i + 1 < npert:
                perturb2(theta, offset, seed, step, i, +a, i + 1, +a, row(i), row(i + 1))
            else:
                perturb(theta, offset, seed, step, i, +a, row(i))
    elif schedule == "none":
        if losses is None:
            raise ValueError("schedule 'none' needs the losses")
    else:
        raise ValueError(schedule)
    c, bad = probe_weights(Lp, Lm, L0, a, delta)
    update(theta, offset, seed, step, c, eta, bits)
    return {"L0": L0, "Lp": Lp, "Lm": Lm, "c": c, "nonfinite": bad}
