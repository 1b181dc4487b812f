"""The five workloads of the 1.5-SPSA path, by name.

Hyperparameters the pages fix: n_pert = 160 with effective batch 128 ("Stanford's 1.5-SPSA
Trains OPT-30B Without Backpropagation", "The Budget Reallocation Insight"); model
shapes are OPT-13B and OPT-30B (the same page's results and the abstract of "Probe-Space
Preconditioning for Fast and Stable Zero-Order Training").  The remaining sizes, seeds and
step counts are the synthetic stand-ins chosen for this path; delta and eta where the
workload leaves them open are 1e-6 and 1e-2 (flat vector) or 1e-3 (bf16 OPT-shaped sets).
"""
from __future__ import annotations

from dataclasses import dataclass, field


def opt_param_count(layers: int, d: int, ffn: int, vocab: int) -> int:
    """Parameters of an OPT-shaped set: per layer four d x d attention matrices, the two
    FFN matrices, and 9d + ffn biases / layer-norm entries (4d attention biases, ffn + d
    FFN biases, 2 x 2d layer norms); plus the vocab x d token embedding."""
    per_layer = 4 * d * d + 2 * d * ffn + (9 * d + ffn)
    return layers * per_layer + vocab * d


@dataclass(frozen=True)
class Config:
    name: str
    M: int                  # number of parameters
    dtype: str              # "fp32" | "bf16"
    npert: int
    eps: float
    eta: float
    delta: float
    steps: int
    loss: str               # "quad" | "mlp" | "synthetic"
    theta_std: float        # theta ~ N(0, theta_std)
    a_range: tuple = (0.0, 0.0)   # log10 range of the diagonal quadratic's a_j
    bits: str = "regen"     # "regen" | "read" | "both"
    seed: int = 0           # probe-RNG seed and theta seed
    extra: dict = field(default_factory=dict)


MLP_SHAPE = {"d_in": 768, "d_hid": 3072, "d_out": 2, "batch": 128,
             "teacher_seed": 1, "input_seed": 2}

CONFIGS = {
    "tiny": Config("tiny", 4096, "fp32", 16, 2.0 ** -10, 1e-2, 1e-6, 10, "quad", 1.0,
                   (-2.0, 2.0), bits="both"),
    "flat125m": Config("flat125m", 125_000_000, "fp32", 32, 2.0 ** -10, 1e-2, 1e-6, 20,
                       "quad", 0.02, (-3.0, 3.0), bits="regen"),
    "mlp": Config("mlp", 768 * 3072 + 3072 + 2 * 3072 + 2, "fp32", 64, 1e-3, 1e-3, 1e-6, 50,
                  "mlp", 0.02, bits="read", extra=dict(MLP_SHAPE)),
    "lowrank": Config("lowrank", 1 << 20, "fp32", 16, 2.0 ** -10, 1e-2, 1e-6, 100, "lowrank",
                      1.0, bits="regen", extra={"rank": 4, "spike": 1e4, "diag": 1.0}),
    "opt13b": Config("opt13b", opt_param_count(40, 5120, 20480, 50272), "bf16", 160, 1e-3,
                     1e-3, 1e-6, 5, "synthetic", 0.02, bits="regen",
                     extra={"layers": 40, "d": 5120, "ffn": 20480, "vocab": 50272}),
    "opt30b": Config("opt30b", opt_param_count(48, 7168, 28672, 50272), "bf16", 160, 1e-3,
                     1e-3, 1e-6, 3, "synthetic", 0.02, bits="regen",
                     extra={"layers": 48, "d": 7168, "ffn": 28672, "vocab": 50272}),
}
