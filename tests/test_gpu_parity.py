"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Pass rule: max |x_gpu - x_ref| <= tau * rms(x_ref) for o and the final state,
tau = 1e-4 with fp32 inputs and 2e-2 with bf16 inputs.  The oracle sees
exactly the cast values the GPU receives.  Shapes span several 64-row chunks,
ragged tails and the supported head dims.
"""
import math

import numpy as np
import pytest
import torch

from gated_delta_rule_96_amd import kda, synth
from oracle import gate as ogate
from oracle import seq
from kda_testutil import TOL, cast, err_ratio, f32, prefill_case, say, to_dev

pytestmark = pytest.mark.gpu
DTYPES = [torch.float32, torch.bfloat16]


def _oracle(c, h0=None):
    return seq.kda_seq(f32(c["q"]), f32(c["k"]), f32(c["v"]), f32(c["g"]), f32(c["beta"]),
                       None if h0 is None else f32(h0))


def _gpu(c, h0=None, **kw):
    d = to_dev(c)
    o, ht = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            None if h0 is None else h0.cuda(), **kw)
    torch.cuda.synchronize()
    return o, ht


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_decode_steps_match_oracle(dtype, dk, dv):
    say(f"decode dtype={dtype} dk={dk} dv={dv}")
    B, H, steps = 3, 2, 6
    st_ref = synth.initial_state(3, B, H, dk, dv).astype(np.float64)
    st = torch.from_numpy(st_ref.astype(np.float32)).cuda()
    A = synth.head_A(3, H)
    for s in range(steps):
        d = synth.decode_tokens(B, H, dk, dv, seed=3, step=s)
        q, k, v, beta = (cast(d[n], dtype) for n in ("q", "k", "v", "beta"))
        g = cast(ogate.gate(d["z"][:, None], A)[:, 0], dtype)
        o = kda.decode_step(q.cuda(), k.cuda(), v.cuda(), g.cuda(), beta.cuda(), st)
        torch.cuda.synchronize()
        o_ref, st_ref = seq.kda_decode_ref(f32(q), f32(k), f32(v), f32(g), f32(beta), st_ref)
        assert err_ratio(f32(o), o_ref) <= TOL[dtype], s
        assert err_ratio(st.cpu().numpy(), st_ref) <= TOL[dtype], s


# ------------------------------------------------------------------ decay preparation
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("T,dk", [(200, 64), (64, 128), (1, 128), (257, 128)])
def test_prepare_decay_matches_oracle(dtype, T, dk):
    say(f"prepare_decay dtype={dtype} T={T} dk={dk}")
    B, H = 2, 3
    d = synth.make_inputs(B, T, H, dk, 8, seed=9, with_h0=False)
    z = cast(d["z"], dtype)
    A = torch.from_numpy(d["A"].copy())
    g, gcum = kda.prepare_decay(z.cuda(), A.cuda())
    torch.cuda.synchronize()
    g_ref = ogate.gate(f32(z), d["A"])
    gg = f32(g).astype(np.float64)
    # Error bound from the fp32 arithmetic: the argument x = exp(A) z carries
    # ~2 ulp of fp32 rounding, which the gate amplifies by dg/dx * x =
    # g (1 - sigmoid(x)) x; exp, add and divide add a few ulp of g; the
    # final rounding to the output dtype adds at most 1/2 ulp of it.
    mant = 7 if dtype == torch.bfloat16 else 23
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(g_ref), 1e-30))) - mant)
    x = np.exp(d["A"].astype(np.float64))[None, None, :, None] * f32(z)
    sig = g_ref / -5.0
    fp32_err = np.abs(g_ref) * ((1 - sig) * np.abs(x) + 4) * 2.0 ** -23
    assert np.all(np.abs(gg - g_ref) <= ulp + fp32_err)
    assert gg.min() >= -5.0 and gg.max() <= 0.0
    # cumsum of the stored g, restarted every 64 rows.  fp32 accumulation:
    # each addition rounds at the scale of its partial sum, so the error at
    # row t is bounded by 2^-24 * (sum of |partial sums| up to t).
    G_ref = ogate.chunk_cumsum(gg, 64)
    bound = 2.0 ** -23 * ogate.chunk_cumsum(np.abs(G_ref), 64)
    assert np.all(np.abs(f32(gcum) - G_ref) <= bound)
    # scan-only mode reproduces it exactly
    gcum2 = kda.prepare_decay(g=g)
    torch.cuda.synchronize()
    assert torch.equal(gcum2, gcum)


# ------------------------------------------------------------------ chunked prefill
def test_config0_tiny_fp32():
    """B=1, H=2, T=256, dk=dv=64, chunk 64, zero initial state, fp32."""
    say("fwd config0 fp32")
    c = prefill_case(1, 256, 2, 64, 64, seed=0, dtype=torch.float32, with_h0=False)
    o, ht = _gpu(c)
    o_ref, h_ref = _oracle(c)
    assert err_ratio(f32(o), o_ref) <= 1e-4
    assert err_ratio(ht.cpu().numpy(), h_ref) <= 1e-4


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,T,H,dk,dv", [
    (1, 64, 1, 128, 128), (2, 200, 3, 128, 128), (1, 1, 2, 128, 128), (1, 65, 2, 64, 64),
    (2, 130, 2, 128, 64), (1, 300, 2, 64, 128), (1, 1000, 2, 128, 128),
])
def test_fwd_matches_oracle(dtype, B, T, H, dk, dv):
    say(f"fwd dtype={dtype} B={B} T={T} H={H} dk={dk} dv={dv}")
    c = prefill_case(B, T, H, dk, dv, seed=11 + T, dtype=dtype)
    o, ht = _gpu(c, c["h0"])
    o_ref, h_ref = _oracle(c, c["h0"])
    assert err_ratio(f32(o), o_ref) <= TOL[dtype]
    assert err_ratio(ht.cpu().numpy(), h_ref) <= TOL[dtype]


@pytest.mark.parametrize("variant", ["extreme", "slow"])
def test_fwd_decay_extremes_bf16(variant):
    say(f"fwd variant={variant}")
    c = prefill_case(2, 512, 2, 128, 128, seed=21, dtype=torch.bfloat16, variant=variant)
    if variant == "extreme":
        assert torch.all(c["g"] == -5.0)
    o, ht = _gpu(c, c["h0"])
    assert torch.isfinite(o.float()).all() and torch.isfinite(ht).all()
    o_ref, h_ref = _oracle(c, c["h0"])
    assert err_ratio(f32(o), o_ref) <= 2e-2
    assert err_ratio(ht.cpu().numpy(), h_ref) <= 2e-2


@pytest.mark.parametrize("dtype", DTYPES)
def test_fwd_gcum_input_and_in_kernel_scan(dtype):
    """The two ways of supplying the decay: g (scanned inside the kernel into
    sums local to each 16-row block) and gcum (the chunk-local cumulative
    sum from kda_prepare_decay; the block-local sums are formed as its
    differences).  Different rounding, same result within the tolerance."""
    say(f"fwd gcum path dtype={dtype}")
    c = prefill_case(1, 200, 2, 128, 128, seed=5, dtype=dtype)
    d = to_dev(c)
    gcum = kda.prepare_decay(g=d["g"])
    o1, h1 = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    o2, h2 = kda.fwd_chunked(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], gcum=gcum)
    torch.cuda.synchronize()
    o_ref, h_ref = _oracle(c, c["h0"])
    for o, h in ((o1, h1), (o2, h2)):
        assert err_ratio(f32(o), o_ref) <= TOL[dtype]
        assert err_ratio(h.cpu().numpy(), h_ref) <= TOL[dtype]


def test_fwd_final_state_may_alias_h0_and_segments_carry():
    say("fwd segment carry with ht aliasing h0")
    c = prefill_case(1, 384, 2, 128, 128, seed=6, dtype=torch.bfloat16)
    d = to_dev(c)
    o_full, h_full = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    state = d["h0"].clone()
    outs = []
    for a, b in ((0, 128), (128, 192), (192, 384)):
        sl = {n: d[n][:, a:b].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o, _ = kda.fwd_chunked(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], state, ht=state)
        outs.append(o)
    torch.cuda.synchronize()
    # chunk boundaries coincide, so the segmented run does the same arithmetic
    assert torch.equal(torch.cat(outs, 1), o_full)
    assert torch.equal(state, h_full)
    o_ref, h_ref = _oracle(c, c["h0"])
    assert err_ratio(f32(o_full), o_ref) <= 2e-2 and err_ratio(state.cpu().numpy(), h_ref) <= 2e-2


def test_fwd_beta_zero_is_pure_decay():
    say("fwd beta=0")
    # slow decay keeps exp(G_T) S_0 of order one over 256 tokens, so the
    # final-state comparison is not against a vanishing reference
    c = prefill_case(1, 256, 2, 128, 128, seed=8, dtype=torch.float32, variant="slow")
    c["beta"].zero_()
    o, ht = _gpu(c, c["h0"])
    G = np.cumsum(f32(c["g"]).astype(np.float64), axis=1)
    h0 = f32(c["h0"]).astype(np.float64)
    o_cf = np.einsum("bthc,bhcj->bthj", np.exp(G) * f32(c["q"]), h0) / math.sqrt(128)
    h_cf = np.exp(G[:, -1])[..., None] * h0
    assert err_ratio(f32(o), o_cf) <= 1e-4
    assert err_ratio(ht.cpu().numpy(), h_cf) <= 1e-4


def test_fwd_orthonormal_write_readback():
    say("fwd orthonormal readback")
    dk = dv = 128
    T = 100
    K = synth.orthonormal_keys(2, T, dk)
    rng = np.random.default_rng(2)
    V = rng.standard_normal((T, dv))
    k = torch.from_numpy(K.reshape(1, T, 1, dk).astype(np.float32)).cuda()
    v = torch.from_numpy(V.reshape(1, T, 1, dv).astype(np.float32)).cuda()
    q = torch.zeros_like(k)
    g = torch.zeros_like(k)
    beta = torch.ones((1, T, 1), device="cuda")
    h0 = torch.from_numpy(rng.standard_normal((1, 1, dk, dv)).astype(np.float32)).cuda()
    _, ht = kda.fwd_chunked(q, k, v, g, beta, h0)
    torch.cuda.synchronize()
    read = K @ ht[0, 0].double().cpu().numpy()
    assert np.max(np.abs(read - V)) <= 1e-4 * np.sqrt(np.mean(V * V))


def test_decode_equals_prefill():
    say("decode == prefill")
    c = prefill_case(2, 70, 2, 128, 128, seed=12, dtype=torch.bfloat16)
    d = to_dev(c)
    o_p, h_p = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    st = d["h0"].clone()
    outs = []
    for t in range(70):
        outs.append(kda.decode_step(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), st))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    o_ref, h_ref = _oracle(c, c["h0"])
    assert err_ratio(f32(o_d), o_ref) <= 2e-2 and err_ratio(f32(o_p), o_ref) <= 2e-2
    assert err_ratio(st.cpu().numpy(), h_ref) <= 2e-2 and err_ratio(h_p.cpu().numpy(), h_ref) <= 2e-2


def test_fwd_is_deterministic():
    say("fwd determinism")
    d = to_dev(prefill_case(2, 500, 3, 128, 128, seed=13, dtype=torch.bfloat16))
    r1 = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    r2 = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_fused_and_two_stage_schedules_agree_bitwise():
    say("fused vs two-stage schedule")
    d = to_dev(prefill_case(2, 333, 3, 128, 128, seed=14, dtype=torch.bfloat16))
    o1, h1 = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    o2, h2 = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], stages=3)
    ws = kda.alloc_workspace(2, 333, 3, 128, 128, torch.bfloat16, "cuda", stages=True)
    kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], stages=1, workspace=ws)
    o3, h3 = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], stages=2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    assert torch.equal(o1, o3) and torch.equal(h1, h3)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64)])
def test_fused_rounds_one_state_pass_per_head(dk, dv):
    """d_v = 64: one state-pass work-group per head, and 200 heads run as
    several rounds of one launch (five of 40 by the launch cost model); all
    heads against the oracle."""
    B, H, T = 2, 100, 130
    say(f"fused rounds dk={dk} dv={dv} B={B} H={H} T={T}")
    c = prefill_case(B, T, H, dk, dv, seed=16, dtype=torch.bfloat16)
    d = to_dev(c)
    ws = kda.alloc_workspace(B, T, H, dk, dv, torch.bfloat16, "cuda")
    o, ht = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], workspace=ws)
    assert kda.workspace_error(ws) == 0
    o_ref, h_ref = _oracle(c, c["h0"])
    assert err_ratio(f32(o), o_ref) <= 2e-2 and err_ratio(ht.cpu().numpy(), h_ref) <= 2e-2


@pytest.mark.parametrize("B,H", [(2, 64), (1, 3), (3, 1)])
def test_fused_head_batching(B, H):
    """More heads than one round of the persistent launch serves (B*H = 128
    > 96), and fewer heads than XCDs."""
    say(f"fused head batching B={B} H={H}")
    c = prefill_case(B, 130, H, 128, 128, seed=15, dtype=torch.bfloat16)
    d = to_dev(c)
    ws = kda.alloc_workspace(B, 130, H, 128, 128, torch.bfloat16, "cuda")
    o, ht = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], workspace=ws)
    assert kda.workspace_error(ws) == 0
    o_ref, h_ref = _oracle(c, c["h0"])
    assert err_ratio(f32(o), o_ref) <= 2e-2 and err_ratio(ht.cpu().numpy(), h_ref) <= 2e-2
