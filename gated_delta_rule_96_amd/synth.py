"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no gate, no decay, no recurrence), so both the HIP path
and the CPU oracle may consume what it produces.

Distributions (Kimi K3 technical report summary, "Key claims" / "Method",
section 2.1.1: the decay gate takes a per-channel pre-activation z and a
learnable per-head A; the recurrent state is a fixed-size matrix per head):

* q, k   : N(0, 1) per element, then divided by their L2 norm over the key
           channels of each (batch, token, head).
* v      : N(0, 1).
* beta   : logistic(N(0, 1)), one scalar per (batch, token, head).
* z      : N(0, 1) per channel (the gate's pre-activation).
* A      : U(-1, 1), one scalar per head.
* h0     : N(0, std=0.02) fp32 initial state [B, H, dk, dv].

Each (tensor, batch, head) stream has its own generator keyed by
SeedSequence([seed, part, tensor_id, b, h]); `part` separates segments of a
long sequence or steps of a decode loop.  Values are drawn in fp32; casting
to the compute dtype is the caller's job (both sides then see identical
values).

Variants (parity-only input families):
* "base"    : the distributions above.
* "extreme" : z = 200 everywhere, so the gate saturates at its floor.
* "slow"    : z ~ N(-8, 1), so the per-token decay is close to 1.
"""
from __future__ import annotations

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "beta": 3, "z": 4, "A": 5, "h0": 6, "do": 7, "dht": 8}
VARIANTS = ("base", "extreme", "slow")


def _rng(seed: int, part: int, tid: int, b: int = 0, h: int = 0) -> np.random.Generator:
    key = [seed, part, tid] + ([b, h] if b >= 0 else [])
    return np.random.default_rng(np.random.SeedSequence(key))


def _normal(seed, part, name, b, h, shape, mean=0.0, std=1.0) -> np.ndarray:
    x = _rng(seed, part, TENSOR_ID[name], b, h).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _unit_rows(x: np.ndarray) -> np.ndarray:
    """Divide each row (last axis) by its Euclidean length (fp64 norm, fp32 out)."""
    n = np.sqrt(np.einsum("...i,...i->...", x.astype(np.float64), x.astype(np.float64)))
    n[n == 0] = 1.0
    return (x / n[..., None]).astype(np.float32)


def _logistic(x: np.ndarray) -> np.ndarray:
    # distribution recipe for beta only (beta = logistic of a normal draw)
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def head_stream(name: str, seed: int, part: int, b: int, h: int, T: int, d: int,
                variant: str = "base") -> np.ndarray:
    """One (batch, head) slice of a token-major tensor: fp32 [T, d] ([T] for beta)."""
    if name in ("q", "k"):
        return _unit_rows(_normal(seed, part, name, b, h, (T, d)))
    if name == "v":
        return _normal(seed, part, name, b, h, (T, d))
    if name == "beta":
        return _logistic(_normal(seed, part, name, b, h, (T,)))
    if name == "z":
        if variant == "extreme":
            return np.full((T, d), 200.0, dtype=np.float32)
        if variant == "slow":
            return _normal(seed, part, name, b, h, (T, d), mean=-8.0)
        return _normal(seed, part, name, b, h, (T, d))
    raise KeyError(name)


def head_A(seed: int, H: int) -> np.ndarray:
    """Per-head gate parameter A ~ U(-1, 1), fp32 [H]; shared by every part."""
    return _rng(seed, 0, TENSOR_ID["A"]).uniform(-1.0, 1.0, size=H).astype(np.float32)


def initial_state(seed: int, B: int, H: int, dk: int, dv: int, std: float = 0.02) -> np.ndarray:
    """fp32 [B, H, dk, dv] with N(0, std) entries (std is a standard deviation)."""
    out = np.empty((B, H, dk, dv), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = _normal(seed, 0, "h0", b, h, (dk, dv), std=std)
    return out


def output_grads(seed: int, B: int, T: int, H: int, dk: int, dv: int, std_ht: float = 1.0):
    """Seeded upstream gradients for the backward: do [B,T,H,dv] and dht
    [B,H,dk,dv], fp32 N(0, 1) (dht N(0, std_ht))."""
    do = np.empty((B, T, H, dv), np.float32)
    dht = np.empty((B, H, dk, dv), np.float32)
    for b in range(B):
        for h in range(H):
            do[b, :, h, :] = _normal(seed, 0, "do", b, h, (T, dv))
            dht[b, h] = _normal(seed, 0, "dht", b, h, (dk, dv), std=std_ht)
    return do, dht


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, seed: int, part: int = 0,
                variant: str = "base", with_h0: bool = True,
                heads: list[int] | None = None) -> dict:
    """Token-major fp32 tensors q,k,z [B,T,Hs,dk], v [B,T,Hs,dv], beta [B,T,Hs],
    A [Hs], h0 [B,Hs,dk,dv] (or None).  `heads` selects a subset of the H heads
    (values identical to the same heads of the full draw); default all."""
    if variant not in VARIANTS:
        raise ValueError(variant)
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)
    out = {
        "q": np.empty((B, T, Hs, dk), np.float32),
        "k": np.empty((B, T, Hs, dk), np.float32),
        "z": np.empty((B, T, Hs, dk), np.float32),
        "v": np.empty((B, T, Hs, dv), np.float32),
        "beta": np.empty((B, T, Hs), np.float32),
    }
    for b in range(B):
        for i, h in enumerate(hs):
            for name in ("q", "k", "z"):
                out[name][b, :, i, :] = head_stream(name, seed, part, b, h, T, dk, variant)
            out["v"][b, :, i, :] = head_stream("v", seed, part, b, h, T, dv, variant)
            out["beta"][b, :, i] = head_stream("beta", seed, part, b, h, T, 1, variant)
    out["A"] = head_A(seed, H)[hs]
    if with_h0:
        full = initial_state(seed, B, H, dk, dv) if heads is None else None
        if full is None:
            h0 = np.empty((B, Hs, dk, dv), np.float32)
            for b in range(B):
                for i, h in enumerate(hs):
                    h0[b, i] = _normal(seed, 0, "h0", b, h, (dk, dv), std=0.02)
            out["h0"] = h0
        else:
            out["h0"] = full
    else:
        out["h0"] = None
    return out


def decode_tokens(B: int, H: int, dk: int, dv: int, seed: int, step: int) -> dict:
    """Inputs of one decode step: q, k, z [B, H, dk], v [B, H, dv], beta [B, H]
    (fp32) and A [H].  Same distributions as make_inputs; each tensor of a
    step is one stream keyed by (seed, step, tensor), so a batch of 8192
    sequences costs five draws per step."""
    def nrm(name, shape):
        return _rng(seed, step, TENSOR_ID[name], -1, -1).standard_normal(shape, dtype=np.float32)
    return {
        "q": _unit_rows(nrm("q", (B, H, dk))),
        "k": _unit_rows(nrm("k", (B, H, dk))),
        "z": nrm("z", (B, H, dk)),
        "v": nrm("v", (B, H, dv)),
        "beta": _logistic(nrm("beta", (B, H))),
        "A": head_A(seed, H),
    }


def orthonormal_keys(seed: int, T: int, dk: int) -> np.ndarray:
    """T <= dk orthonormal rows (fp64), from a QR of a Gaussian draw."""
    g = _rng(seed, 0, 99).standard_normal((dk, T))
    qmat, _ = np.linalg.qr(g)
    return qmat.T.copy()
