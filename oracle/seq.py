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
        fb = lib.kda_oracle_seq_bwd
        fb.restype = ctypes.c_int
        fb.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_double, L, L, L, L, L, L, P, P, P, P, P, P, ctypes.c_int]
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


def kda_seq_bwd(q, k, v, g, beta, h0, do, dht=None, scale=None, seg: int = 64, nthreads=None):
    """Gradient of the recurrence (the reverse-mode chain rule through each
    token's decay, delta step and output, from the last token back).

    do [B,T,H,dv] = dL/do, dht [B,H,dk,dv] = dL/dS_T or None (zero).
    Returns dict of fp64 arrays dq, dk, dg [B,T,H,dk], dv [B,T,H,dv],
    dbeta [B,T,H], dh0 [B,H,dk,dv].  States are recomputed from ones kept every
    `seg` tokens; the arithmetic does not depend on seg.
    Pinned by tests/test_oracle_pins.py (central finite differences of
    kda_seq, linearity in (do, dht), the T = 1 closed form)."""
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    f64 = lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    h0a = None if h0 is None else f64(h0)
    doa = f64(do)
    dhta = None if dht is None else f64(dht)
    assert doa.shape == (B, T, H, dv)
    out = {"dq": np.empty((B, T, H, dk)), "dk": np.empty((B, T, H, dk)), "dv": np.empty((B, T, H, dv)),
           "dg": np.empty((B, T, H, dk)), "dbeta": np.empty((B, T, H)), "dh0": np.empty((B, H, dk, dv))}
    ptr = lambda a: None if a is None else a.ctypes.data
    nt = threads_default() if nthreads is None else int(nthreads)
    rc = _load().kda_oracle_seq_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data, beta.ctypes.data,
                                    ptr(h0a), doa.ctypes.data, ptr(dhta), float(scale), B, T, H, dk, dv, int(seg),
                                    *(out[n].ctypes.data for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0")), nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_seq_bwd failed with code {rc}")
    return out


def kda_decode_ref(q, k, v, g, beta, state, scale=None, nthreads=None):
    """One decode token per (b, h): the recurrence with T = 1.
    q,k,g [B,H,dk]; v [B,H,dv]; beta [B,H]; state [B,H,dk,dv].
    Returns (o fp64 [B,H,dv], new_state fp64)."""
    o, ht = kda_seq(np.asarray(q)[:, None], np.asarray(k)[:, None], np.asarray(v)[:, None],
                    np.asarray(g)[:, None], np.asarray(beta)[:, None], state, scale, nthreads)
    return o[:, 0], ht
