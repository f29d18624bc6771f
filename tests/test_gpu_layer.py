"""GPU parity of the prefill and the decode step with the layer's steps fused
in (kda_fwd_chunked_layer, kda_decode_step_layer): the decay gate of z
inside the kernel, in-kernel q/k row L2 normalisation, and the sigmoid
output gate, against the fp64 oracle (oracle/gate.py, oracle/layer.py,
oracle/seq.py).

The oracle sees the cast inputs the GPU receives and applies each step in
fp64: g = gate(z) (not rounded: the kernel keeps the gate in fp32), rows of
q and k normalised (and, with bf16 inputs, rounded to bf16: the normalised
rows are the recurrence's bf16 inputs, as with a separate normalisation),
o gated.  Pass rule as the other parity tests (tau = 1e-4 fp32 inputs,
2e-2 bf16 inputs, max error over rms, o and final state).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_96_amd import kda, synth
from oracle import gate as ogate
from oracle import layer, seq
from kda_testutil import TOL, cast, err_ratio, f32, say

pytestmark = pytest.mark.gpu
DTYPES = [torch.float32, torch.bfloat16]


def _case(B, T, H, dk, dv, seed, dtype, raw_scale=1.0):
    d = synth.make_inputs(B, T, H, dk, dv, seed)
    rng = np.random.default_rng(seed + 1000)
    c = {n: cast(d[n], dtype) for n in ("v", "beta", "z")}
    if raw_scale != 1.0:   # un-normalised q and k for the in-kernel normalisation
        c["q"] = cast(raw_scale * rng.standard_normal((B, T, H, dk)), dtype)
        c["k"] = cast(raw_scale * rng.standard_normal((B, T, H, dk)), dtype)
    else:
        c["q"], c["k"] = cast(d["q"], dtype), cast(d["k"], dtype)
    c["og"] = cast(2.0 * rng.standard_normal((B, T, H, dv)), dtype)
    c["A"] = torch.from_numpy(d["A"].copy())
    c["h0"] = torch.from_numpy(d["h0"])
    return c


def _oracle(c, norm, gated):
    q, k = f32(c["q"]).astype(np.float64), f32(c["k"]).astype(np.float64)
    if norm:
        # normalised rows enter the recurrence in the input precision (bf16
        # mode: bf16, as the separate normalisation would hand them over)
        q, k = layer.l2norm_rows(q), layer.l2norm_rows(k)
        if c["q"].dtype == torch.bfloat16:
            q, k = f32(cast(q, torch.bfloat16)), f32(cast(k, torch.bfloat16))
    g = ogate.gate(f32(c["z"]), c["A"].numpy())
    o, ht = seq.kda_seq(q, k, f32(c["v"]), g, f32(c["beta"]), f32(c["h0"]))
    if gated:
        o = layer.output_gate(o, f32(c["og"]))
    return o, ht


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("norm,gated", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("B,T,H,dk,dv", [(2, 200, 2, 128, 128), (1, 97, 3, 64, 64)])
def test_layer_matches_oracle(dtype, norm, gated, B, T, H, dk, dv):
    say(f"layer dtype={dtype} norm={norm} gate={gated} B={B} T={T} H={H} dk={dk} dv={dv}")
    c = _case(B, T, H, dk, dv, seed=51, dtype=dtype, raw_scale=3.0 if norm else 1.0)
    o_ref, h_ref = _oracle(c, norm, gated)
    dev = {n: t.cuda() for n, t in c.items()}
    o, ht = kda.fwd_chunked_layer(dev["q"], dev["k"], dev["v"], dev["z"], dev["A"], dev["beta"], dev["h0"],
                                  og=dev["og"] if gated else None, qk_l2norm=norm)
    torch.cuda.synchronize()
    eo, eh = err_ratio(f32(o), o_ref), err_ratio(ht.cpu().numpy(), h_ref)
    say(f"  o err/rms {eo:.3e}, state err/rms {eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_layer_agrees_with_the_unfused_steps(dtype):
    # The fused steps give what the separate ones give (decay pass, then the
    # prefill on normalised q/k, then the gate on o), to the parity tolerance:
    # the separate path rounds g and the normalised rows to the input type.
    c = _case(1, 300, 2, 128, 128, seed=52, dtype=dtype, raw_scale=2.0)
    dev = {n: t.cuda() for n, t in c.items()}
    o1, h1 = kda.fwd_chunked_layer(dev["q"], dev["k"], dev["v"], dev["z"], dev["A"], dev["beta"], dev["h0"],
                                   og=dev["og"], qk_l2norm=True)
    g, _ = kda.prepare_decay(dev["z"], dev["A"], want_gcum=False)
    nrm = lambda x: (x.float() / torch.sqrt((x.float() ** 2).sum(-1, keepdim=True) + 1e-6)).to(dtype)
    o2, h2 = kda.fwd_chunked(nrm(dev["q"]), nrm(dev["k"]), dev["v"], g, dev["beta"], dev["h0"])
    o2 = o2 * torch.sigmoid(dev["og"].float())
    torch.cuda.synchronize()
    assert err_ratio(f32(o1), f32(o2)) <= TOL[dtype] and err_ratio(f32(h1), f32(h2)) <= TOL[dtype]


# ------------------------------------------------------------------ decode step with the layer's steps
def _decode_oracle(d, A, norm, gated, st_ref):
    """One step of the fp64 oracle on the cast inputs d: gate of z (unrounded),
    normalised q/k (rounded to bf16 in bf16 mode), recurrence, output gate."""
    q, k = f32(d["q"]).astype(np.float64), f32(d["k"]).astype(np.float64)
    if norm:
        q, k = layer.l2norm_rows(q), layer.l2norm_rows(k)
        if d["q"].dtype == torch.bfloat16:
            q, k = f32(cast(q, torch.bfloat16)), f32(cast(k, torch.bfloat16))
    g = ogate.gate(f32(d["z"])[:, None], A)[:, 0]
    o, st_ref = seq.kda_decode_ref(q, k, f32(d["v"]), g, f32(d["beta"]), st_ref)
    if gated:
        o = layer.output_gate(o, f32(d["og"]))
    return o, st_ref


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("norm,gated", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_decode_layer_matches_oracle(dtype, norm, gated, dk, dv):
    say(f"decode layer dtype={dtype} norm={norm} gate={gated} dk={dk} dv={dv}")
    B, H, steps = 3, 2, 6
    A = synth.head_A(61, H)
    st_ref = synth.initial_state(61, B, H, dk, dv).astype(np.float64)
    st = torch.from_numpy(st_ref.astype(np.float32)).cuda()
    rng = np.random.default_rng(62)
    Ad = torch.from_numpy(np.asarray(A, dtype=np.float32).copy()).cuda()
    for s in range(steps):
        t = synth.decode_tokens(B, H, dk, dv, seed=61, step=s)
        d = {n: cast(t[n], dtype) for n in ("q", "k", "v", "z", "beta")}
        if norm:   # un-normalised rows for the in-kernel normalisation
            d["q"] = cast(3.0 * rng.standard_normal((B, H, dk)), dtype)
            d["k"] = cast(3.0 * rng.standard_normal((B, H, dk)), dtype)
        d["og"] = cast(2.0 * rng.standard_normal((B, H, dv)), dtype)
        dev = {n: x.cuda() for n, x in d.items()}
        o = kda.decode_step_layer(dev["q"], dev["k"], dev["v"], dev["z"], Ad, dev["beta"], st,
                                  og=dev["og"] if gated else None, qk_l2norm=norm)
        torch.cuda.synchronize()
        o_ref, st_ref = _decode_oracle(d, A, norm, gated, st_ref)
        eo, eh = err_ratio(f32(o), o_ref), err_ratio(st.cpu().numpy(), st_ref)
        assert eo <= TOL[dtype] and eh <= TOL[dtype], (s, eo, eh)


@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_layer_continues_the_layer_prefill(dtype):
    # A sequence prefilled with the layer call and continued token by token
    # with the layer decode step is the same recurrence: both against the
    # oracle over the whole sequence (outputs of the decoded tokens, final
    # state).
    say(f"layer prefill + layer decode dtype={dtype}")
    T, extra = 130, 5
    c = _case(2, T + extra, 2, 128, 128, seed=63, dtype=dtype, raw_scale=2.0)
    o_ref, h_ref = _oracle(c, True, True)
    dev = {n: t.cuda() for n, t in c.items()}
    pre = lambda x: x[:, :T].contiguous()
    _, st = kda.fwd_chunked_layer(pre(dev["q"]), pre(dev["k"]), pre(dev["v"]), pre(dev["z"]), dev["A"],
                                  pre(dev["beta"]), dev["h0"], og=pre(dev["og"]), qk_l2norm=True)
    outs = []
    for t in range(T, T + extra):
        step = {n: dev[n][:, t].contiguous() for n in ("q", "k", "v", "z", "beta", "og")}
        outs.append(kda.decode_step_layer(step["q"], step["k"], step["v"], step["z"], dev["A"], step["beta"], st,
                                          og=step["og"], qk_l2norm=True))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1)
    eo, eh = err_ratio(f32(o_dec), o_ref[:, T:]), err_ratio(st.cpu().numpy(), h_ref)
    say(f"  decoded o err/rms {eo:.3e}, state err/rms {eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]
