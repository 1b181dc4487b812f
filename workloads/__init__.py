"""Seeded synthetic inputs for the 1.5-SPSA path: parameter sets, loss coefficients,
synthetic per-probe losses and the MLP classification data.

This package holds no arithmetic of the method (no probes, perturbations, weights or
updates).  It is the only code that both the HIP path's tests/benchmark and the CPU
oracle consume, so that both sides see identical inputs.
"""
from .configs import CONFIGS, Config, opt_param_count  # noqa: F401
from . import gen  # noqa: F401
