"""The allocation-free prefill (kda_fwd_chunked_noalloc, for callers that
cannot allocate device memory) against kda_fwd_chunked, through the C ABI.

Both entry points run the same kernels, so their outputs must agree bit for
bit; each is also held to the oracle's bf16 / fp32 tolerance.  Two calls in
a row on the library's scratch, the second with a smaller input: the first
has more heads than the scratch holds at once (fp32 inputs, 40 heads: two
launches), so the second also checks that nothing left in the scratch by
the first changes its result.
"""
import ctypes

import pytest
import torch

from gated_delta_rule_96_amd import kda
from kda_testutil import TOL, err_ratio, f32, prefill_case, say, to_dev
from oracle import seq

pytestmark = pytest.mark.gpu


def _noalloc(c, dtype):
    B, T, H, dk = c["q"].shape
    dv = c["v"].shape[-1]
    o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device="cuda")
    ht = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    code = kda.KDA_BF16 if dtype == torch.bfloat16 else kda.KDA_F32
    st = kda.lib().kda_fwd_chunked_noalloc(
        c["q"].data_ptr(), c["k"].data_ptr(), c["v"].data_ptr(), c["g"].data_ptr(), None, c["beta"].data_ptr(),
        ctypes.c_float(dk ** -0.5), c["h0"].data_ptr(), ht.data_ptr(), o.data_ptr(), code, B, T, H, dk, dv, 64,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kda.status_str(st)
    assert kda.lib().kda_fwd_status(None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    return o, ht


@pytest.mark.parametrize("first,second", [
    ((1, 300, 40, 128, 128, torch.float32), (1, 100, 3, 128, 128, torch.bfloat16)),
    ((2, 200, 36, 128, 128, torch.bfloat16), (1, 70, 2, 64, 64, torch.float32)),
])
def test_noalloc_matches_kda_fwd_chunked_twice(first, second):
    for i, (B, T, H, dk, dv, dtype) in enumerate((first, second)):
        say(f"noalloc call {i}: B={B} T={T} H={H} dk={dk} dv={dv} {dtype}")
        c = prefill_case(B, T, H, dk, dv, 95 + i, dtype)
        d = to_dev(c)
        o_n, ht_n = _noalloc(d, dtype)
        o_w, ht_w = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], check=True)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_w) and torch.equal(ht_n, ht_w)
        o_ref, h_ref = seq.kda_seq(f32(c["q"]), f32(c["k"]), f32(c["v"]), f32(c["g"]), f32(c["beta"]),
                                   f32(c["h0"]))
        eo, eh = err_ratio(f32(o_n), o_ref), err_ratio(f32(ht_n), h_ref)
        say(f"  o err/rms {eo:.3e}, state err/rms {eh:.3e}")
        assert eo <= TOL[dtype] and eh <= TOL[dtype]
