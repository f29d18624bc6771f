"""fp64 steps either side of the KDA path -- TEST INFRASTRUCTURE ONLY.

Readings (the pages name these steps without defining them):
  * key/query normalisation: the delta rule's keys are unit vectors; rows of
    q and k are divided by sqrt(sum of squares + eps), eps = 1e-6;
  * output gate: o <- Sigmoid(og) * o elementwise, og the gate's
    pre-activation [B,T,H,dv] ("Key claims", section 2.1.2: the sigmoid
    output gate named for MLA, "matching KDA's gating").

Pinned by tests/test_oracle_pins.py: normalised rows have unit norm up to
the eps term, positive scaling of a row does not change it, zero rows stay
zero; the gate halves o at og = 0, passes it at og -> +inf, closes at
og -> -inf, and Sigmoid(x) + Sigmoid(-x) = 1.
"""
from __future__ import annotations

import numpy as np

NORM_EPS = 1e-6


def l2norm_rows(x, eps: float = NORM_EPS) -> np.ndarray:
    """x / sqrt(sum(x^2, last axis) + eps), fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def output_gate(o, og) -> np.ndarray:
    """Sigmoid(og) * o, fp64, with Sigmoid(x) = 1 / (1 + exp(-x))."""
    og = np.asarray(og, dtype=np.float64)
    with np.errstate(over="ignore"):
        return np.asarray(o, dtype=np.float64) / (1.0 + np.exp(-og))
