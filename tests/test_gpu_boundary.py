"""GPU tests of the boundary's run-time checks: the opt-in range check of
the log-decay (KDA_VALIDATE=1 -> KDA_ERR_RANGE, nothing enqueued, outputs
untouched) and the status word of the fused prefill (kda_fwd_status).

The range is the gate's floor: g in [-5, 0] keeps 16 rows of decay inside
the bf16 range that the rescaled dense tiles rely on ("Key claims",
section 2.1.1); the unbounded-decay calls take any finite g <= 0.
"""
import math
import os

import pytest
import torch

from gated_delta_rule_96_amd import kda
from kda_testutil import prefill_case, say, to_dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


@pytest.fixture
def validate_on():
    old = os.environ.get("KDA_VALIDATE")
    os.environ["KDA_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["KDA_VALIDATE"]
    else:
        os.environ["KDA_VALIDATE"] = old


def _case(dtype=BF, T=200, H=2):
    return to_dev(prefill_case(1, T, H, 128, 128, 71, dtype))


def _fwd(c, g=None, gcum=None, unbounded=False, sentinel=7.0):
    o = torch.full((1, c["q"].shape[1], c["q"].shape[2], 128), sentinel, dtype=torch.float32, device="cuda")
    try:
        kda.fwd_chunked(c["q"], c["k"], c["v"], g, c["beta"], c["h0"], gcum=gcum, out=o, unbounded=unbounded)
        status = 0
    except kda.KDAError as e:
        status = e.status
    torch.cuda.synchronize()
    return status, o


@pytest.mark.parametrize("dtype", [torch.float32, BF])
def test_validate_accepts_in_range_and_rejects_out_of_range_decay(validate_on, dtype):
    c = _case(dtype)
    say(f"KDA_VALIDATE range check dtype={dtype}")
    st, o = _fwd(c, c["g"])
    assert st == 0 and not torch.all(o == 7.0)
    # the floor itself and exactly zero are in range
    g = c["g"].clone()
    g[0, 5, 1, 3] = -5.0
    g[0, 6, 0, 4] = 0.0
    assert _fwd(c, g)[0] == 0
    for bad in (-5.5, 0.25, float("nan"), float("-inf")):
        g = c["g"].clone()
        g[0, 133, 1, 77] = bad
        st, o = _fwd(c, g)
        assert st == kda.KDA_ERR_RANGE, bad
        assert torch.all(o == 7.0), "an output was written although the call was rejected"
    # the unbounded call accepts any finite g <= 0, not a positive or NaN one
    g = c["g"].clone()
    g[0, 10, 0, 0] = -300.0
    assert _fwd(c, g, unbounded=True)[0] == 0
    for bad in (0.5, float("nan"), float("-inf")):
        g = c["g"].clone()
        g[0, 10, 0, 0] = bad
        assert _fwd(c, g, unbounded=True)[0] == kda.KDA_ERR_RANGE, bad


def test_validate_checks_the_decay_a_gcum_encodes(validate_on):
    c = _case(torch.float32)
    gcum = kda.prepare_decay(g=c["g"])
    assert _fwd(c, None, gcum)[0] == 0
    # a step of -6 between two rows of one chunk
    bad = gcum.clone()
    bad[0, 70:128, 0, 9] -= 6.0
    assert _fwd(c, None, bad)[0] == kda.KDA_ERR_RANGE
    # an increasing cumulative sum (positive decay)
    bad = gcum.clone()
    bad[0, 20, 1, 2] = bad[0, 19, 1, 2] + 0.5
    assert _fwd(c, None, bad)[0] == kda.KDA_ERR_RANGE


def test_validate_decode_and_backward(validate_on):
    c = _case(BF, T=64)
    q, k, v, g, beta = (c[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta"))
    st = c["h0"].clone()
    kda.decode_step(q, k, v, g, beta, st)
    g2 = g.clone()
    g2[0, 1, 5] = -7.0
    with pytest.raises(kda.KDAError) as ei:
        kda.decode_step(q, k, v, g2, beta, st)
    assert ei.value.status == kda.KDA_ERR_RANGE
    do = torch.randn((1, 64, 2, 128), device="cuda")
    gb = c["g"].clone()
    gb[0, 3, 0, 0] = float("nan")
    with pytest.raises(kda.KDAError) as ei:
        kda.bwd_chunked(c["q"], c["k"], c["v"], gb, c["beta"], c["h0"], do)
    assert ei.value.status == kda.KDA_ERR_RANGE


def test_status_word_clear_after_complete_calls():
    # every call clears the status word first; complete calls leave it clear
    c = _case(BF, T=300, H=3)
    ws = kda.alloc_workspace(1, 300, 3, 128, 128, BF, "cuda")
    for _ in range(2):
        kda.fwd_chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], c["h0"], workspace=ws, check=True)
        assert kda.workspace_error(ws) == 0
    # the word's device address is the one kda_fwd_status reads
    addr = kda.lib().kda_fwd_status_word(ws.data_ptr())
    assert addr == ws.data_ptr() + 32
    assert int(ws[32:36].view(torch.int32).item()) == 0
    say(f"status word clear after complete calls ({math.prod(c['q'].shape)} q elements)")
