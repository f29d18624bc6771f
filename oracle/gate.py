"""fp64 decay gate and chunk-local cumulative log-decay -- TEST INFRASTRUCTURE ONLY.

Kimi K3 technical report summary ("Key claims", section 2.1.1 and Fig. 3;
"Method", section 2.1): the log-decay is a scaled sigmoid bounded below,
g = gmin * Sigmoid(exp(A) * z) with gmin = -5 and A learnable per head.
Sigmoid is the logistic function 1/(1+exp(-x)).

The chunk-local inclusive cumulative sum Gamma_t = sum of g over the rows of
t's chunk up to and including t is the quantity whose exponentials form the
rescaling factors of the chunkwise form (same section 2.1).

The same section contrasts this with the predecessor's (Kimi Linear's)
unbounded negative-Softplus log-decay; `gate_softplus` is that gate in the
same form, g = -Softplus(exp(A) * z) with Softplus(x) = log(1 + exp(x))
(reading: the same exp(A) * z argument as the bounded gate; the pages give
only the name).  It has no lower bound.

Pinned by tests/test_oracle_pins.py: z = 0 gives gmin/2 for every A,
exp(A) z = ln 3 gives 3/4 gmin, odd symmetry g(z) + g(-z) = gmin,
monotonicity, range [gmin, 0); cumsum against the segment definition;
Softplus gate: z = 0 gives -ln 2, exp(A) z = ln(e - 1) gives -1, the
identity g(z) - g(-z) = -exp(A) z, and -x asymptotics for large x.
"""
from __future__ import annotations

import numpy as np

GMIN = -5.0


def gate(z, A, gmin: float = GMIN) -> np.ndarray:
    """g[b,t,h,c] = gmin / (1 + exp(-exp(A[h]) * z[b,t,h,c])) in fp64.
    z [..., H, dk] with heads on axis -2; A [H]."""
    z = np.asarray(z, dtype=np.float64)
    a = np.exp(np.asarray(A, dtype=np.float64))
    x = a[:, None] * z
    with np.errstate(over="ignore"):
        return gmin / (1.0 + np.exp(-x))


def gate_softplus(z, A) -> np.ndarray:
    """g[b,t,h,c] = -log(1 + exp(exp(A[h]) * z[b,t,h,c])) in fp64, written as
    -(max(x, 0) + log1p(exp(-|x|))) so that large |x| neither overflows nor
    loses the small term.  z [..., H, dk] with heads on axis -2; A [H]."""
    z = np.asarray(z, dtype=np.float64)
    a = np.exp(np.asarray(A, dtype=np.float64))
    x = a[:, None] * z
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def chunk_cumsum(g, chunk: int) -> np.ndarray:
    """Inclusive cumulative sum of g along the token axis (axis 1 of
    [B,T,H,dk]), restarted at every multiple of `chunk`; fp64."""
    g = np.asarray(g, dtype=np.float64)
    B, T = g.shape[:2]
    out = np.empty_like(g)
    for s in range(0, T, chunk):
        out[:, s:s + chunk] = np.cumsum(g[:, s:s + chunk], axis=1)
    return out
