"""The C-ABI library loads and exports every symbol include/kda.h declares;
argument validation rejects bad calls before anything is enqueued (these
calls never reach a kernel launch, so they run without a GPU)."""
import ctypes
import re
from pathlib import Path

import pytest

from gated_delta_rule_96_amd import kda

ROOT = Path(__file__).resolve().parents[1]


def declared_functions():
    text = (ROOT / "include" / "kda.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("kda_prepare_decay", "kda_fwd_chunked", "kda_decode_step", "kda_fwd_workspace_bytes",
              "kda_fwd_chunked_stages", "kda_fwd_stages_workspace_bytes", "kda_status_str", "kda_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = kda.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_profiling_build_exports_the_same_calls_and_the_stamps():
    # libkda_stamps.so: the same sources with the fused prefill's cycle
    # stamps (include/kda_stamps.h); the product library has no stamps
    L = ctypes.CDLL(str(kda.STAMPS_LIB_PATH))
    text = re.sub(r"/\*.*?\*/", "", (ROOT / "include" / "kda_stamps.h").read_text(), flags=re.S)
    stamps = sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))
    assert stamps == ["kda_stamps_read"]
    for n in declared_functions() + stamps:
        assert hasattr(L, n), n
    assert not hasattr(kda.lib(), "kda_stamps_read")
    L.kda_stamps_read.restype = ctypes.c_int
    L.kda_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    n = kda.STAMP_WGS * kda.STAMP_WAVES * kda.STAMP_SLOTS
    assert L.kda_stamps_read(None, n) == 1                     # KDA_ERR_NULL
    buf = (ctypes.c_uint64 * n)()
    assert L.kda_stamps_read(ctypes.addressof(buf), n - 1) == 2   # KDA_ERR_SHAPE


def test_version_and_status_strings():
    assert kda.abi_version() == 1
    for s in range(9):
        assert kda.status_str(s)
    assert "unknown" in kda.status_str(99)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gcum=None, beta=FAKE, scale=0.1, h0=None, ht=None, o=FAKE,
             dtype=1, B=1, T=64, H=1, dk=128, dv=128, chunk=64, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return kda.lib().kda_fwd_chunked(a["q"], a["k"], a["v"], a["g"], a["gcum"], a["beta"], a["scale"], a["h0"],
                                     a["ht"], a["o"], a["dtype"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                     a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(beta=None), 1), (dict(g=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(T=0), 2), (dict(H=-1), 2),
    (dict(dtype=7), 3),
    (dict(q=FAKE + 4), 4), (dict(h0=FAKE + 8), 4), (dict(ws=FAKE + 16), 4),
    (dict(dk=96), 5), (dict(dv=32), 5), (dict(chunk=32), 5),
    (dict(ws=None), 6), (dict(wsb=1024), 6),
])
def test_fwd_validation(kw, code):
    assert fwd(**kw) == code


def test_workspace_bytes():
    n = kda.fwd_workspace_bytes(1, 65536, 32, 128, 128)
    assert n > 0 and n % 256 == 0
    # fused schedule: ring buffers, independent of T, capped at one launch's heads
    assert kda.fwd_workspace_bytes(1, 65536, 32, 128, 128) == kda.fwd_workspace_bytes(1, 64, 32, 128, 128)
    assert kda.fwd_workspace_bytes(8, 64, 64, 128, 128) == kda.fwd_workspace_bytes(4, 64, 64, 128, 128)
    assert n < 64 << 20
    # two-stage schedule: one record per chunk
    s = lambda T: kda.fwd_workspace_bytes(1, T, 1, 128, 128, stages=True)
    assert s(65) == 2 * s(64) and s(64) % 256 == 0
    for f in (kda.lib().kda_fwd_workspace_bytes, kda.lib().kda_fwd_stages_workspace_bytes):
        assert f(1, 64, 1, 96, 128, 64, 1) == 0
        assert f(1, 64, 1, 128, 128, 32, 1) == 0


def test_decode_validation():
    L = kda.lib()
    args = [FAKE] * 5 + [0.1, FAKE, FAKE, 1, 2, 2, 128, 128, None]
    bad = list(args); bad[0] = None
    assert L.kda_decode_step(*bad) == 1
    bad = list(args); bad[11] = 32
    assert L.kda_decode_step(*bad) == 5
    bad = list(args); bad[6] = FAKE + 4
    assert L.kda_decode_step(*bad) == 4
    bad = list(args); bad[8] = 2
    assert L.kda_decode_step(*bad) == 3


def test_decode_layer_validation():
    L = kda.lib()
    args = [FAKE] * 6 + [None, 0.1, FAKE, FAKE, 1, 1, 2, 2, 128, 128, None]
    for i in (3, 4):   # z, A
        bad = list(args); bad[i] = None
        assert L.kda_decode_step_layer(*bad) == 1
    bad = list(args); bad[10] = 4   # unknown flag bit
    assert L.kda_decode_step_layer(*bad) == 2
    bad = list(args); bad[6] = FAKE + 8   # og misaligned
    assert L.kda_decode_step_layer(*bad) == 4
    bad = list(args); bad[14] = 32
    assert L.kda_decode_step_layer(*bad) == 5
    bad = list(args); bad[11] = 2
    assert L.kda_decode_step_layer(*bad) == 3


def test_prepare_decay_validation():
    L = kda.lib()
    # gate mode without A, scan mode without gcum, unsupported chunk
    assert L.kda_prepare_decay(FAKE, None, -5.0, FAKE, FAKE, 1, 1, 64, 1, 128, 64, None) == 1
    assert L.kda_prepare_decay(None, None, -5.0, FAKE, None, 1, 1, 64, 1, 128, 64, None) == 1
    assert L.kda_prepare_decay(None, None, -5.0, FAKE, FAKE, 1, 1, 64, 1, 128, 16, None) == 5
    assert L.kda_prepare_decay(None, None, -5.0, FAKE, FAKE, 1, 0, 64, 1, 128, 64, None) == 2


def test_unbounded_entry_points_validate_like_the_bounded_ones():
    L = kda.lib()
    a = [FAKE, FAKE, FAKE, FAKE, None, FAKE, 0.1, None, None, FAKE, 1, 1, 64, 1, 128, 128, 64, FAKE, 1 << 40, None]
    for i, code in ((0, 1), (5, 1), (9, 1)):
        bad = list(a); bad[i] = None
        assert L.kda_fwd_chunked_unbounded(*bad) == code
    bad = list(a); bad[14] = 96
    assert L.kda_fwd_chunked_unbounded(*bad) == 5
    bad = list(a); bad[18] = 1024
    assert L.kda_fwd_chunked_unbounded(*bad) == 6
    # stage mask: the unbounded bit needs at least one stage; other bits are rejected
    st = a[:19] + [kda.KDA_STAGES_UNBOUNDED, None]
    assert L.kda_fwd_chunked_stages(*st) == 2
    st = a[:19] + [8 | 1, None]
    assert L.kda_fwd_chunked_stages(*st) == 2
    # softplus gate: z and A are required
    assert L.kda_prepare_decay_softplus(None, FAKE, FAKE, FAKE, 1, 1, 64, 1, 128, 64, None) == 1
    assert L.kda_prepare_decay_softplus(FAKE, None, FAKE, FAKE, 1, 1, 64, 1, 128, 64, None) == 1
    assert L.kda_prepare_decay_softplus(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 1, 96, 64, None) == 5


def test_varlen_validation_and_snapshot_count():
    L = kda.lib()
    cu = lambda *xs: (ctypes.c_int * len(xs))(*xs)

    def call(c, N, T=100, snap=None, every=0, ws=FAKE, wsb=1 << 40):
        return L.kda_fwd_chunked_varlen(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0.1, c, N, None, None, FAKE, snap,
                                        every, 1, T, 2, 128, 128, 64, ws, wsb, None)

    assert call(None, 1) == 1
    assert call(cu(0, 50, 40), 2) == 2         # decreasing
    assert call(cu(1, 100), 1) == 2            # does not start at 0
    assert call(cu(0, 99), 1) == 2             # does not end at T
    assert call(cu(0, 100), 0) == 2            # N = 0
    assert call(cu(0, 100), 1, every=-1) == 2
    assert call(cu(0, 100), 1, snap=FAKE + 4, every=1) == 4
    assert call(cu(0, 100), 1, wsb=1024) == 6
    n = L.kda_fwd_varlen_snapshots
    n.restype = ctypes.c_longlong
    assert n(cu(0, 64, 200, 200, 1000), 4, 2, 64) == 0 + 1 + 0 + 6
    assert n(cu(0, 65), 1, 1, 64) == 1 and n(cu(0, 64), 1, 1, 64) == 0
    assert n(cu(0, 10), 1, 0, 64) == -1 and n(cu(0, 10), 1, 1, 32) == -1 and n(cu(5, 1), 1, 1, 64) == -1


def test_layer_entry_validation():
    L = kda.lib()
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, None, None, FAKE, 0, 1, 1, 64, 1, 128, 128, 64, FAKE,
         1 << 40, None]
    for i in (3, 4):                       # z, A required
        bad = list(a); bad[i] = None
        assert L.kda_fwd_chunked_layer(*bad) == 1
    bad = list(a); bad[11] = 2             # unknown flag bit
    assert L.kda_fwd_chunked_layer(*bad) == 2
    bad = list(a); bad[6] = FAKE + 2       # misaligned output gate
    assert L.kda_fwd_chunked_layer(*bad) == 4
    bad = list(a); bad[20] = 1024
    assert L.kda_fwd_chunked_layer(*bad) == 6


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.1, h0=None, do=FAKE, dht=None, dq=FAKE, dk_=FAKE,
             dv_=FAKE, dg=FAKE, dbeta=FAKE, dh0=None, dtype=1, B=1, T=200, H=2, dk=128, dv=128, chunk=64, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return kda.lib().kda_bwd_chunked(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(g=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dbeta=None), 1),
    (dict(T=0), 2), (dict(B=0), 2), (dict(dtype=5), 3),
    (dict(dg=FAKE + 4), 4), (dict(dht=FAKE + 8), 4), (dict(dh0=FAKE + 4), 4), (dict(ws=FAKE + 64), 4),
    (dict(dk=32), 5), (dict(chunk=16), 5),
    (dict(ws=None), 6), (dict(wsb=4096), 6),
])
def test_bwd_validation(kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_bytes():
    L = kda.lib()
    n1 = L.kda_bwd_workspace_bytes(1, 64, 2, 128, 128, 64, 1)
    n2 = L.kda_bwd_workspace_bytes(1, 6400, 2, 128, 128, 64, 1)
    assert n1 > 0 and n1 % 256 == 0 and n2 > n1
    # per chunk and head the backward keeps a state, its gradient and a record
    assert n2 - n1 >= 99 * 2 * (3 * 128 * 128 * 4)
    assert L.kda_bwd_workspace_bytes(1, 64, 2, 96, 128, 64, 1) == 0
    assert L.kda_bwd_workspace_bytes(1, 64, 2, 128, 128, 32, 1) == 0


def test_status_codes_and_status_word():
    L = kda.lib()
    assert "incomplete" in kda.status_str(kda.KDA_ERR_INCOMPLETE)
    assert "range" in kda.status_str(kda.KDA_ERR_RANGE)
    # the status word sits at ints [8] of a (256-byte aligned) workspace
    assert L.kda_fwd_status_word(FAKE) == FAKE + 32
    assert L.kda_fwd_status_word(None) is None
    # kda_fwd_status validates before it touches the device
    assert L.kda_fwd_status(FAKE + 16, None) == 4


def test_gate_floor_outside_supported_range_is_rejected():
    # the bounded gate's floor keeps 16 rows of decay within the bf16 range
    # only for gmin >= -5 ("Key claims", section 2.1.1); a floor at or
    # above 0 is no decay gate at all
    L = kda.lib()
    for gmin in (-5.5, -6.0, 0.0, 1.0, float("nan"), float("-inf")):
        assert L.kda_prepare_decay(FAKE, FAKE, gmin, FAKE, None, 1, 1, 64, 1, 128, 64, None) == kda.KDA_ERR_RANGE
    # the unbounded gate has no floor argument; scan mode ignores gmin
    assert L.kda_prepare_decay(None, None, -9.0, FAKE, FAKE, 1, 0, 64, 1, 128, 64, None) == 2


def test_varlen_rejects_packed_gcum():
    # a gcum of the packed token axis restarts at multiples of 64 tokens, not
    # at each sequence's own chunks
    L = kda.lib()
    cu = (ctypes.c_int * 3)(0, 30, 100)
    assert L.kda_fwd_chunked_varlen(FAKE, FAKE, FAKE, None, FAKE, FAKE, 0.1, cu, 2, None, None, FAKE, None, 0, 1,
                                    100, 2, 128, 128, 64, FAKE, 1 << 40, None) == kda.KDA_ERR_UNSUPPORTED


def test_noalloc_entry_validates_like_kda_fwd_chunked():
    L = kda.lib()
    a = [FAKE, FAKE, FAKE, FAKE, None, FAKE, 0.1, None, None, FAKE, 1, 1, 64, 1, 128, 128, 64, None]
    for i in (0, 5, 9):
        bad = list(a); bad[i] = None
        assert L.kda_fwd_chunked_noalloc(*bad) == 1
    bad = list(a); bad[3] = None                     # neither g nor gcum
    assert L.kda_fwd_chunked_noalloc(*bad) == 1
    bad = list(a); bad[11] = 0
    assert L.kda_fwd_chunked_noalloc(*bad) == 2
    bad = list(a); bad[10] = 4
    assert L.kda_fwd_chunked_noalloc(*bad) == 3
    bad = list(a); bad[7] = FAKE + 8
    assert L.kda_fwd_chunked_noalloc(*bad) == 4
    bad = list(a); bad[15] = 96
    assert L.kda_fwd_chunked_noalloc(*bad) == 5
