"""Shared helpers for the GPU parity tests (inputs, casting, tolerances)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from gated_delta_rule_96_amd import synth
from oracle import gate as ogate

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(msg: str):
    print(f"[kda-test] {msg}", flush=True)
    sys.stdout.flush()


def cast(x: np.ndarray, dtype) -> torch.Tensor:
    """fp32/fp64 numpy -> torch tensor of `dtype` (RNE), on the CPU."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def err_ratio(x, ref) -> float:
    """max |x - ref| / rms(ref)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(x - ref))) / max(rms, 1e-300)


def prefill_case(B, T, H, dk, dv, seed, dtype, variant="base", with_h0=True, part=0, heads=None):
    """Seeded inputs cast to `dtype` (CPU tensors) plus the gate's g from the
    oracle (fp64, cast).  Returns dict of CPU tensors: q,k,v,g,beta (dtype),
    h0 (fp32 or None), z (dtype), A (fp32)."""
    d = synth.make_inputs(B, T, H, dk, dv, seed, part=part, variant=variant, with_h0=with_h0, heads=heads)
    out = {n: cast(d[n], dtype) for n in ("q", "k", "v", "beta", "z")}
    out["A"] = torch.from_numpy(d["A"].copy())
    out["g"] = cast(ogate.gate(f32(out["z"]), d["A"]), dtype)
    out["h0"] = torch.from_numpy(d["h0"]) if d["h0"] is not None else None
    return out


def to_dev(d: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
