"""GPU parity of the variable-length packed prefill with prefix-state
snapshots (kda_fwd_chunked_varlen) against the fp64 oracle.

Each packed sequence is an independent recurrence with its own initial and
final state ("Method", section 2.1); the snapshots are the states at its
chunk boundaries ("Key claims", Infrastructure: states kept at prefix
boundaries).  The oracle runs each sequence alone, and its prefix up to each
snapshot boundary alone.  Length mixes include empty sequences, a single
token, exactly one chunk, ragged tails and a long sequence.

Pass rule as the other parity tests (tau = 1e-4 fp32, 2e-2 bf16, max error
over rms, for o, final states and snapshots).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_96_amd import kda, synth
from oracle import gate as ogate
from oracle import seq
from kda_testutil import TOL, cast, err_ratio, f32, say

pytestmark = pytest.mark.gpu
DTYPES = [torch.float32, torch.bfloat16]


def _packed(lengths, H, dk, dv, seed, dtype, with_h0=True):
    T = int(sum(lengths))
    d = synth.make_inputs(1, max(T, 1), H, dk, dv, seed, with_h0=False)
    c = {n: cast(d[n][:, :T], dtype) for n in ("q", "k", "v", "beta", "z")}
    c["g"] = cast(ogate.gate(f32(c["z"]), d["A"]), dtype)
    N = len(lengths)
    c["h0"] = torch.from_numpy(synth.initial_state(seed, N, H, dk, dv)) if with_h0 else None
    c["cu"] = np.concatenate([[0], np.cumsum(lengths)]).astype(int)
    return c


def _oracle_seq(c, i, upto=None):
    a, b = c["cu"][i], c["cu"][i + 1]
    if upto is not None:
        b = a + upto
    sl = lambda n: f32(c[n][:, a:b])
    h0 = None if c["h0"] is None else f32(c["h0"][i:i + 1])
    return seq.kda_seq(sl("q"), sl("k"), sl("v"), sl("g"), sl("beta"), h0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("lengths,dk,dv,every,H", [
    ([1, 64, 130, 0, 257, 33], 128, 128, 2, 2),
    ([700, 5, 128], 64, 64, 3, 2),
    ([0, 190, 64], 128, 64, 1, 2),
    ([130, 1, 257], 128, 128, 2, 70),   # the fused launch runs 70 heads as rounds of 40 and 30
])
def test_varlen_matches_oracle_with_snapshots(dtype, lengths, dk, dv, every, H):
    say(f"varlen dtype={dtype} lengths={lengths} dk={dk} dv={dv} every={every} H={H}")
    c = _packed(lengths, H, dk, dv, seed=41, dtype=dtype)
    dev = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in c.items()}
    o, ht, snaps = kda.fwd_chunked_varlen(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], c["cu"], dev["h0"],
                                          snap_every=every)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    j = 0
    for i, L in enumerate(lengths):
        if L == 0:
            np.testing.assert_array_equal(ht[i].cpu().numpy(), f32(c["h0"][i]))
            continue
        o_ref, h_ref = _oracle_seq(c, i)
        a = c["cu"][i]
        assert err_ratio(f32(o[:, a:a + L]), o_ref) <= tol, i
        assert err_ratio(ht[i:i + 1].cpu().numpy(), h_ref) <= tol, i
        nch = (L + 63) // 64
        for m in range(every, nch, every):   # snapshot after 64 m tokens
            _, s_ref = _oracle_seq(c, i, upto=64 * m)
            assert err_ratio(snaps[j:j + 1].cpu().numpy(), s_ref) <= tol, (i, m)
            j += 1
    assert j == (0 if snaps is None else snaps.shape[0]) == kda.varlen_snapshots(c["cu"], every)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H", [3, 70])
def test_varlen_equals_separate_calls_bitwise(dtype, H):
    # Packing changes nothing: each sequence gets exactly the result of its
    # own kda_fwd_chunked call (same chunking from its start; with 70 heads
    # both run the fused launch in two rounds, of 40 and 30 heads).
    lengths = [300, 1, 64, 129]
    dk, dv = 128, 128
    c = _packed(lengths, H, dk, dv, seed=42, dtype=dtype)
    dev = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in c.items()}
    o, ht, _ = kda.fwd_chunked_varlen(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], c["cu"], dev["h0"])
    for i, L in enumerate(lengths):
        a = c["cu"][i]
        sl = lambda n: dev[n][:, a:a + L].clone()   # own, aligned allocation
        oi, hi = kda.fwd_chunked(sl("q"), sl("k"), sl("v"), sl("g"), sl("beta"), dev["h0"][i:i + 1].clone())
        torch.cuda.synchronize()
        assert torch.equal(oi, o[:, a:a + L]) and torch.equal(hi, ht[i:i + 1]), i


def test_varlen_zero_states_and_in_place_carry():
    # h0 = NULL starts every sequence from zero (an empty one then ends at
    # zero); ht may be h0 itself.
    lengths = [0, 80, 0, 20]
    H, dk, dv = 2, 64, 64
    c = _packed(lengths, H, dk, dv, seed=43, dtype=torch.float32, with_h0=False)
    dev = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in c.items()}
    ht = torch.full((4, H, dk, dv), 7.0, device="cuda")
    o, ht, _ = kda.fwd_chunked_varlen(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], c["cu"], None, ht=ht)
    torch.cuda.synchronize()
    assert float(ht[0].abs().max()) == 0.0 and float(ht[2].abs().max()) == 0.0
    for i in (1, 3):
        o_ref, h_ref = _oracle_seq(c, i)
        a, L = c["cu"][i], lengths[i]
        assert err_ratio(f32(o[:, a:a + L]), o_ref) <= TOL[torch.float32]
        assert err_ratio(ht[i:i + 1].cpu().numpy(), h_ref) <= TOL[torch.float32]
    # in-place: a second pass continuing from the first pass's states
    c2 = _packed(lengths, H, dk, dv, seed=44, dtype=torch.float32, with_h0=False)
    dev2 = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in c2.items()}
    h_first = ht.clone()
    _, ht2, _ = kda.fwd_chunked_varlen(dev2["q"], dev2["k"], dev2["v"], dev2["g"], dev2["beta"], c2["cu"], ht, ht=ht)
    torch.cuda.synchronize()
    c2["h0"] = h_first.cpu()
    for i in (1, 3):
        _, h_ref = _oracle_seq(c2, i)
        assert err_ratio(ht2[i:i + 1].cpu().numpy(), h_ref) <= TOL[torch.float32]
