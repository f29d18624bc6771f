"""fp64 sequential KDA recurrence (ctypes wrapper of kda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Follows the Kimi K3 technical report summary
("Key claims"/"Method", section 2.1): per head, a fixed-size state
S in R^{dk x dv} updated once per token by a delta rule after a channel-wise
decay Diag(exp(g_t)); the output reads the updated state, o_t = scale*S_t^T q_t.
Pinned by: brute force (tests/test_oracle_pins.py::test_seq_matches_brute_force),
beta = 0 closed form, orthonormal write/readback, pad identity, segment split.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(str(path))
        f = lib.kda_oracle_seq
        f.restype = ctypes.c_int
        P = ctypes.c_void_p
        L = ctypes.c_long
        f.argtypes = [P, P, P, P, P, P, ctypes.c_double, L, L, L, L, L, P, P, ctypes.c_int]
        lib.kda_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads_default() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def kda_seq(q, k, v, g, beta, h0=None, scale=None, nthreads=None):
    """Run the recurrence.  q,k,g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H];
    h0 [B,H,dk,dv] or None.  Inputs are converted to fp32 (exact for fp32/bf16
    values); arithmetic is fp64.  Returns (o fp64 [B,T,H,dv], ht fp64 [B,H,dk,dv])."""
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape == g.shape and v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    h0p = None
    if h0 is not None:
        h0a = np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
        assert h0a.shape == (B, H, dk, dv)
        h0p = h0a.ctypes.data
    o = np.empty((B, T, H, dv), np.float64)
    ht = np.empty((B, H, dk, dv), np.float64)
    nt = threads_default() if nthreads is None else int(nthreads)
    rc = _load().kda_oracle_seq(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
                                beta.ctypes.data, h0p, float(scale), B, T, H, dk, dv,
                                o.ctypes.data, ht.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_seq failed with code {rc}")
    return o, ht


def kda_decode_ref(q, k, v, g, beta, state, scale=None, nthreads=None):
    """One decode token per (b, h): the recurrence with T = 1.
    q,k,g [B,H,dk]; v [B,H,dv]; beta [B,H]; state [B,H,dk,dv].
    Returns (o fp64 [B,H,dv], new_state fp64)."""
    o, ht = kda_seq(np.asarray(q)[:, None], np.asarray(k)[:, None], np.asarray(v)[:, None],
                    np.asarray(g)[:, None], np.asarray(beta)[:, None], state, scale, nthreads)
    return o[:, 0], ht
