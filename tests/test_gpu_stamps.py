"""The profiling build libkda_stamps.so (the fused prefill with cycle stamps,
include/kda_stamps.h) computes what libkda.so computes, bit for bit, and its
stamps describe the launch: every (chunk, head) item counted once by the
producers, every chunk once by each state-pass wave, no slot beyond the
documented ones used."""
import numpy as np
import pytest
import torch

from gated_delta_rule_96_amd import kda
from kda_testutil import prefill_case, say, to_dev

pytestmark = pytest.mark.gpu

PRODUCER, OWNER, STAGING = 1, 2, 3
PRODUCER_SLOTS = set(range(0, 11)) | set(range(17, 25))
STATE_SLOTS = set(range(0, 8))


def _run(path, d):
    kda._lib = None
    kda.LIB_PATH = path
    o, ht = kda.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    return o.cpu(), ht.cpu()


@pytest.mark.parametrize("T,H", [(4096, 16), (1000, 3)])
def test_stamped_build_same_output_and_consistent_stamps(T, H):
    say(f"stamped build T={T} H={H}")
    d = to_dev(prefill_case(1, T, H, 128, 128, seed=17, dtype=torch.bfloat16))
    saved = (kda._lib, kda.LIB_PATH)
    try:
        ref = _run(kda.LIB_PATH, d)
        got = _run(kda.STAMPS_LIB_PATH, d)
        s = kda.stamps_read()
    finally:
        kda._lib, kda.LIB_PATH = saved
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])

    nch = (T + 63) // 64
    role, count = s[:, :, kda.STAMP_ROLE], s[:, :, kda.STAMP_COUNT]
    # a work-group is a producer (all 8 waves) or a state pass (waves 0-3
    # own value columns, waves 4-7 stage records); the grid is one per CU
    prod = (role == PRODUCER).all(axis=1)
    cons = (role[:, :4] == OWNER).all(axis=1) & (role[:, 4:] == STAGING).all(axis=1)
    assert (prod | cons).all()
    # producers: each item once (all 8 waves count it); state pass: two
    # work-groups per head (dv = 128), every chunk counted by every wave
    assert int(count[prod, 0].sum()) == H * nch
    assert (count[prod] == count[prod][:, :1]).all()
    assert int(cons.sum()) == 2 * H
    assert (count[cons] == nch).all()
    # only the documented slots hold cycles, and the busy ones are non-zero
    for mask, slots in ((prod, PRODUCER_SLOTS), (cons, STATE_SLOTS)):
        cyc = s[mask][:, :, :kda.STAMP_ROLE]
        unused = [i for i in range(kda.STAMP_ROLE) if i not in slots]
        assert (cyc[:, :, unused] == 0).all()
    busy = prod & (count[:, 0] > 0)         # (small launches leave producers idle)
    assert busy.any() and (s[busy][:, :, 4] > 0).all()   # Gram phase
    assert (s[cons][:, :4, 4] > 0).all()    # owner products
    say(f"  producers {int(prod.sum())} work-groups, state pass {int(cons.sum())}; "
        f"cycles per item {float(s[prod][:, :, :kda.STAMP_ROLE].sum(-1).mean()) / max(1, float(count[prod, 0].mean())):.0f}")
