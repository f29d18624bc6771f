"""Benchmark of the KDA forward hot path on one MI355X.

Step = one KDA chunked prefill (decay scan, intra-chunk Gram/UT solve and
state pass: kda_fwd_chunked) over the long-prefill workload
B=1, H=32, T=65536, dk=dv=128, chunk 64, bf16 q/k/v/beta/g inputs, fp32
initial/final state and fp32 output; the log-decay g is produced by the
library's own gate (kda_prepare_decay) before timing.  Inputs are seeded
synthetic data (gated_delta_rule_96_amd.synth), already resident in HBM when
the timed region starts.

Printed: ONE JSON line with the prefill tokens/s (value), the roofline of
the prefill call (HBM-bound: algorithmic bytes / measured time), the MFMA
fraction on the algorithmic flop count, per-kernel times (HIP events on the
launch stream), the B=4 H=16 T=8192 prefill and the million-token prefill
(16 segments of 65536 carrying the state) with the linear-cost check, the
batched decode step (B=256, H=32, 1000 steps) against the HBM roofline, a
parity check of the timed output against the CPU oracle on a sample, and the
CPU oracle's own throughput (cpu_baseline).

Profiling helpers (for rocprofv3 runs; they print no JSON line):
  bench.py --probe fused|stages|copy [--calls N] [--heads H]
      a few calls of one prefill schedule on the benchmark workload (with H
      heads in place of 32, if given), or a plain 1 GiB device copy that
      calibrates the memory counters;
  bench.py --probe stamps [--calls N]
      the fused prefill from the profiling build libkda_stamps.so: cycles
      per item of each producer phase and per chunk of the state pass;
  bench.py --summarize RESULTS.db|kernel_stats.csv
      the kernel trace as a short table;
  bench.py --summarize-pmc KERNEL FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv COPY_BYTES
      FETCH_SIZE / WRITE_SIZE of one kernel scaled by what they read for
      the copy of COPY_BYTES, as HBM bytes per launch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 MFMA
METRIC = "KDA chunked prefill tokens/s + % bf16 MFMA peak (T=64K); decode % HBM peak"

# prefill workload
B, H, T, DK, DV, CHUNK = 1, 32, 65536, 128, 128, 64
# the other prefill workloads: B=4 H=16 T=8192, and 16 segments of 65536 (1M tokens)
C1 = (4, 16, 8192)
C3_SEGMENTS = 16
# decode workload
DB, DH, DSTEPS, DPOOL = 256, 32, 1000, 8


def prefill_alg_counts(B, T, H, dk, dv, C=64, out_bytes=2):
    """Algorithmic flop and HBM bytes of one prefill call (no dense upper-triangle
    work, no intermediates): per token-head 6 dk dv + 1.25 C (3 dk + 2 dv) + C^2/3
    flop; bytes = bf16 q, k, g, v, beta read and o written at `out_bytes` per
    element (2: the 1282 B per token-head of a bf16 output at dk = dv = 128;
    4: the fp32 output this library writes, 1538 B), plus fp32 h0 read and
    ht written per (b, h)."""
    th = B * T * H
    flop = th * (6 * dk * dv + 1.25 * C * (3 * dk + 2 * dv) + C * C / 3.0)
    bytes_ = th * (2 * (3 * dk + dv) + 2 + out_bytes * dv) + B * H * 2 * 4 * dk * dv
    return flop, bytes_


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "kda_fused_fwd_B1H32T65536_hbm_traffic.txt")
KERNEL_SOURCES = ("kda_chunk.hip", "kda_device.h")


def source_sha256() -> str:
    """sha256 over the fused prefill kernel's sources (the code the counters describe)."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_96_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per fused prefill launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    summary is missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != source_sha256():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- profiling helpers
COPY_BYTES = 1 << 30


def probe(what: str, calls: int, heads: int = H):
    """A few calls of one prefill schedule on the benchmark workload, or on
    it with fewer heads (fewer records in each XCD's L2 at once), or a plain
    device copy of COPY_BYTES, which reads and writes exactly that many bytes
    and so calibrates FETCH_SIZE / WRITE_SIZE, for rocprofv3 runs."""
    import torch

    from gated_delta_rule_96_amd import kda, synth

    dev = torch.device("cuda:0")
    if what == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(calls):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[probe] copy of {COPY_BYTES} bytes x {calls}", file=sys.stderr, flush=True)
        return
    d = synth.make_inputs(B, T, heads, DK, DV, seed=2)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
    q, k, v, beta, z = (bf(d[n]) for n in ("q", "k", "v", "beta", "z"))
    A = torch.from_numpy(d["A"].copy()).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    g, _ = kda.prepare_decay(z, A, want_gcum=False)
    stages = what == "stages"
    ws = kda.alloc_workspace(B, T, heads, DK, DV, torch.bfloat16, dev, stages=stages)
    o = torch.empty((B, T, heads, DV), dtype=torch.float32, device=dev)
    ht = torch.empty((B, heads, DK, DV), dtype=torch.float32, device=dev)
    for _ in range(calls):
        kda.fwd_chunked(q, k, v, g, beta, h0, ht=ht, workspace=ws, out=o, stages=3 if stages else None)
    torch.cuda.synchronize()
    print(f"[probe] {what} H={heads} x {calls} done", file=sys.stderr, flush=True)


STAMP_NAMES = {
    1: {0: "entry (item start, LDS free)", 1: "stage k/q/g/beta", 2: "block scans, exponentials",
        3: "factors, K-hat to the record", 4: "Gram tiles, diagonal inverses, Q-bar",
        5: "K-bar/V transposes, inverse d=1", 6: "inverse d=2", 7: "inverse d=3", 8: "Tm",
        9: "W and U to the record", 10: "hand-off (publish)"},
    2: {0: "loop top", 1: "barrier (record staged)", 2: "abort word", 3: "range scale, U accumulators",
        4: "U and Q-bar products issued", 5: "K-hat/M/decay reads, U range", 6: "state update, output, stores",
        7: "snapshots, next range scale and Sh"},
    3: {0: "loop top", 1: "barrier", 2: "abort word, progress store", 3: "wait for the next record",
        4: "record loads issued", 5: "loads completed, LDS writes"},
}


def probe_stamps(calls: int):
    """Cycle stamps of the fused prefill on the benchmark workload, from the
    profiling build libkda_stamps.so: cycles per item for the producers
    (phase work and the barrier that ends it) and per chunk for the state
    pass's owner and staging waves, averaged over the launch's waves."""
    import numpy as np
    import torch

    from gated_delta_rule_96_amd import kda, synth

    kda.LIB_PATH = kda.STAMPS_LIB_PATH
    dev = torch.device("cuda:0")
    d = synth.make_inputs(B, T, H, DK, DV, seed=2)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
    q, k, v, beta, z = (bf(d[n]) for n in ("q", "k", "v", "beta", "z"))
    A = torch.from_numpy(d["A"].copy()).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    g, _ = kda.prepare_decay(z, A, want_gcum=False)
    ws = kda.alloc_workspace(B, T, H, DK, DV, torch.bfloat16, dev)
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=dev)
    ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    for _ in range(10):
        kda.fwd_chunked(q, k, v, g, beta, h0, ht=ht, workspace=ws, out=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        kda.fwd_chunked(q, k, v, g, beta, h0, ht=ht, workspace=ws, out=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    kda.check_workspace(ws)
    s = kda.stamps_read().astype(np.float64)   # [wg][wave][slot], the last call
    role, cnt = s[:, :, kda.STAMP_ROLE], s[:, :, kda.STAMP_COUNT]
    print(f"fused prefill B={B} H={H} T={T} dk={DK} dv={DV}, stamped build: {ms:.3f} ms per call "
          f"(mean of {calls}); stamps of the last call")
    longest = s[:, :, :kda.STAMP_ROLE].sum(-1).max()
    print(f"longest wave: {longest:.0f} cycles = {longest / (ms * 1e6):.2f} GHz over the call's duration")
    for r, what in ((1, "producer, cycles per item"), (2, "state-pass owner waves, cycles per chunk"),
                    (3, "state-pass staging waves, cycles per chunk")):
        sel = (role == r) & (cnt > 0)
        if not sel.any():
            continue
        per = s[sel] / cnt[sel][:, None]            # [waves, slots]
        nwg = int(((role == r).any(1)).sum())
        print(f"\n{what}: {int(sel.sum())} waves in {nwg} work-groups, "
              f"{cnt[sel].mean():.1f} {'items' if r == 1 else 'chunks'} per wave")
        if r == 1:
            # per-wave-index means (waves 0-3 and 4-7 take different tiles)
            wi = np.nonzero(sel)[1]
            byw = np.stack([per[wi == w].mean(0) for w in range(kda.STAMP_WAVES)])
            print(f"  {'phase':<36} {'total':>7} {'work':>7} {'barrier':>8}   work by wave 0..7")
            tot = 0.0
            for sl, name in STAMP_NAMES[1].items():
                work = per[:, sl].mean()
                bar = per[:, 16 + sl].mean() if 1 <= sl <= 8 else 0.0
                tot += work + bar
                ww = " ".join(f"{x:6.0f}" for x in byw[:, sl]) if 1 <= sl <= 8 else ""
                print(f"  {name:<36} {work + bar:7.0f} {work:7.0f} {bar:8.0f}   {ww}")
            print(f"  {'total':<36} {tot:7.0f}")
        else:
            tot = 0.0
            for sl, name in STAMP_NAMES[r].items():
                x = per[:, sl].mean()
                tot += x
                print(f"  {name:<36} {x:7.0f}")
            print(f"  {'total':<36} {tot:7.0f}")


def summarize_trace(path: str):
    """Kernel trace (rocpd SQLite database or kernel_stats CSV) as a table:
    kernel, calls, total and average duration (us), share of GPU time."""
    import csv
    import sqlite3

    if path.endswith(".db"):
        con = sqlite3.connect(path)
        cur = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels")
        rows = [(r[0], int(r[1]), float(r[2]), float(r[3]), float(r[4])) for r in cur]   # microseconds
    else:
        with open(path) as f:
            rows = [(r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3,
                     float(r["Percentage"])) for r in csv.DictReader(f)]
    print(f"{'kernel':<60} {'calls':>6} {'total_us':>12} {'avg_us':>10} {'pct':>6}")
    for name, calls, tot, avg, pct in rows:
        short = name if len(name) <= 60 else name[:57] + "..."
        print(f"{short:<60} {calls:>6} {tot:>12.1f} {avg:>10.2f} {pct:>6.2f}")


def summarize_pmc(kernel_sub, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernels whose name
    contains kernel_sub, each scaled by copy_bytes / (the same counter for the
    copy), as HBM bytes per launch; records the kernel sources' sha256."""
    import csv

    def per_dispatch(path, counter, sub):
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and sub in r["Kernel_Name"]:
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not per:
            raise SystemExit(f"no {counter} rows for kernels matching {sub!r} in {path}")
        return sum(per.values()) / len(per), len(per)

    copy_bytes = float(copy_bytes)
    cf, ncf = per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cw, ncw = per_dispatch(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    kf, nkf = per_dispatch(fetch_csv, "FETCH_SIZE", kernel_sub)
    kw, nkw = per_dispatch(write_csv, "WRITE_SIZE", kernel_sub)
    sf, sw = copy_bytes / cf, copy_bytes / cw
    print(f"kernel: {kernel_sub}")
    print(f"copy calibration: {copy_bytes:.0f} bytes each way; FETCH_SIZE {cf:.1f} KiB/dispatch "
          f"({ncf} dispatches) -> scale {sf:.4f} bytes per unit; WRITE_SIZE {cw:.1f} KiB/dispatch "
          f"({ncw}) -> scale {sw:.4f}")
    print(f"kernel FETCH_SIZE {kf:.1f} KiB/dispatch ({nkf} dispatches) -> {kf * sf:.0f} bytes read")
    print(f"kernel WRITE_SIZE {kw:.1f} KiB/dispatch ({nkw} dispatches) -> {kw * sw:.0f} bytes written")
    print(f"traffic_bytes_per_launch: {kf * sf + kw * sw:.0f}")
    print(f"source_sha256: {source_sha256()}")


def bwd_alg_counts(B, T, H, dk, dv, C=64):
    """Algorithmic flop of one backward call (chunkwise gradient, lower
    triangles only, excluding the forward recompute): per token-head
    14 dk dv + 8.5 C dk + 5.5 C dv + C^2/3; HBM bytes: bf16 q, k, v, g, beta
    and fp32 do read, fp32 dq, dk, dv, dg, dbeta written, h0/dht read and dh0
    written."""
    th = B * T * H
    flop = th * (14 * dk * dv + 8.5 * C * dk + 5.5 * C * dv + C * C / 3.0)
    bytes_ = th * (2 * (3 * dk + dv) + 2 + 4 * dv + 4 * (3 * dk + dv) + 4) + B * H * 3 * 4 * dk * dv
    return flop, bytes_


def decode_alg_bytes(B, H, dk, dv):
    """fp32 state read + written, bf16 q, k, g, v, beta read, fp32 o written."""
    return B * H * (2 * 4 * dk * dv + 2 * (3 * dk + dv) + 2 + 4 * dv)


def extra_configs(args, torch, kda, synth, dev, stream, log, ms_c2):
    """The other two prefill workloads, timed like the headline one:
    B=4 H=16 T=8192 (inputs from synth, oracle parity on every head) and the
    million-token prefill B=1 H=32 as 16 segments of 65536 carrying the fp32
    state in place (inputs drawn on the device with the same distributions;
    segment 0's four sampled heads from synth, checked against the oracle,
    whose time on them is extrapolated to the whole run).  Then the
    linear-cost check: throughput per token-head of the three prefills."""
    BF = torch.bfloat16
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(BF)

    def timed(fn, n, warm=3):
        for _ in range(warm):   # warm-up (the clock settles after a change of kernel)
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = {}
    # ---- B=4 H=16 T=8192
    Bc, Hc, Tc = C1
    log(f"prefill B={Bc} H={Hc} T={Tc}")
    d = synth.make_inputs(Bc, Tc, Hc, DK, DV, seed=21)
    host = {n: bf(d[n]) for n in ("q", "k", "v", "beta", "z")}
    q, k, v, beta, z = (host[n].to(dev) for n in ("q", "k", "v", "beta", "z"))
    A = torch.from_numpy(d["A"].copy()).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    g, _ = kda.prepare_decay(z, A, want_gcum=False)
    ws = kda.alloc_workspace(Bc, Tc, Hc, DK, DV, BF, dev)
    o = torch.empty((Bc, Tc, Hc, DV), dtype=torch.float32, device=dev)
    ht = torch.empty((Bc, Hc, DK, DV), dtype=torch.float32, device=dev)
    # a call takes about half a millisecond: 30 warm-up calls (15 ms) for the
    # clock to settle, then at least 40 timed ones
    ms1 = timed(lambda: kda.fwd_chunked(q, k, v, g, beta, h0, ht=ht, workspace=ws, out=o), max(40, 2 * args.steps),
                warm=30)
    kda.check_workspace(ws)
    c1 = {"workload": f"KDA chunked prefill B={Bc} H={Hc} T={Tc} dk=dv={DK}, bf16 inputs, fp32 state and output",
          "ms_per_call": round(ms1, 4), "tokens_per_s": round(Bc * Tc / (ms1 * 1e-3), 1),
          "token_heads_per_s": round(Bc * Tc * Hc / (ms1 * 1e-3), 1)}
    if not args.no_cpu_baseline:
        from oracle import gate as ogate
        from oracle import seq

        f = lambda t: t.float().numpy()
        g_ref = f(bf(ogate.gate(f(host["z"]), d["A"]).astype(np.float32)))
        t0 = time.perf_counter()
        o_ref, h_ref = seq.kda_seq(f(host["q"]), f(host["k"]), f(host["v"]), g_ref, f(host["beta"]), d["h0"],
                                   nthreads=seq.threads_default())
        c1_cpu = time.perf_counter() - t0
        rms = lambda x: math.sqrt(float(np.mean(x * x)))
        c1["parity"] = {"sample": "every output and final state, all heads, vs fp64 oracle (its own gate of the "
                                  "same z, rounded to bf16)",
                        "max_err_over_rms_o": float(np.max(np.abs(o.cpu().double().numpy() - o_ref)) / rms(o_ref)),
                        "max_err_over_rms_ht": float(np.max(np.abs(ht.cpu().double().numpy() - h_ref)) / rms(h_ref)),
                        "tolerance": 2e-2}
        c1["cpu_oracle_tokens_per_s"] = round(Bc * Tc / c1_cpu, 1)
    out["B4_H16_T8192"] = c1
    log(f"  {ms1:.3f} ms per call" + (f"; parity o {c1['parity']['max_err_over_rms_o']:.2e}" if "parity" in c1 else ""))
    del q, k, v, beta, z, g, o, ht, ws, host, d

    # ---- 1M tokens: 16 segments of 65536, state carried in place
    nseg, heads = C3_SEGMENTS, [0, 9, 18, 27]
    log(f"million-token prefill: {nseg} segments of {T}, B={B} H={H}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(23)
    A = torch.from_numpy(synth.head_A(23, H).copy()).to(dev)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    segs = []
    for s in range(nseg):
        shp = (B, T, H, DK)
        x = {"q": unit(torch.randn(shp, generator=gen, device=dev)), "k": unit(torch.randn(shp, generator=gen,
                                                                                           device=dev)),
             "z": torch.randn(shp, generator=gen, device=dev), "v": torch.randn(shp, generator=gen, device=dev),
             "beta": torch.sigmoid(torch.randn((B, T, H), generator=gen, device=dev))}
        if s == 0:
            ds = synth.make_inputs(B, T, H, DK, DV, seed=23, part=0, with_h0=False, heads=heads)
            for n in x:
                x[n][:, :, heads] = torch.from_numpy(ds[n]).to(dev)
        x = {n: t_.to(BF) for n, t_ in x.items()}
        x["g"] = kda.prepare_decay(x["z"], A, want_gcum=False)[0]
        del x["z"]
        segs.append(x)
    h0_host = synth.initial_state(23, B, H, DK, DV)
    h0 = torch.from_numpy(h0_host).to(dev)
    state = torch.empty_like(h0)
    ws = kda.alloc_workspace(B, T, H, DK, DV, BF, dev)
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=dev)
    o0 = torch.empty_like(o)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]

    def one_pass(record):
        state.copy_(h0)
        for s, x in enumerate(segs):
            if record:
                evs[s].record(stream)
            kda.fwd_chunked(x["q"], x["k"], x["v"], x["g"], x["beta"], state, ht=state, workspace=ws,
                            out=o0 if s == 0 else o)
        if record:
            evs[nseg].record(stream)

    one_pass(False)
    torch.cuda.synchronize()
    reps = max(2, args.steps // 8)
    tot, per_seg = 0.0, np.zeros(nseg)
    for _ in range(reps):
        one_pass(True)
        torch.cuda.synchronize()
        seg_ms = np.array([evs[s].elapsed_time(evs[s + 1]) for s in range(nseg)])
        per_seg += seg_ms
        tot += seg_ms.sum()
    kda.check_workspace(ws)
    ms3 = tot / reps
    per_seg /= reps
    c3 = {"workload": f"KDA million-token prefill B={B} H={H} T={nseg * T} as {nseg} segments of {T} carrying the "
                      f"fp32 state in place, bf16 inputs (drawn on the device, same distributions)",
          "ms_per_pass": round(ms3, 4), "tokens_per_s": round(B * nseg * T / (ms3 * 1e-3), 1),
          "token_heads_per_s": round(B * nseg * T * H / (ms3 * 1e-3), 1),
          "segment_ms": [round(float(x), 4) for x in per_seg]}
    if not args.no_cpu_baseline:
        from oracle import gate as ogate
        from oracle import seq

        f = lambda t_: t_.float().numpy()
        sel = lambda n: f(bf(ds[n]))
        g_ref = f(bf(ogate.gate(sel("z"), synth.head_A(23, H)[heads]).astype(np.float32)))
        t0 = time.perf_counter()
        o_ref, _ = seq.kda_seq(sel("q"), sel("k"), sel("v"), g_ref, sel("beta"), h0_host[:, heads],
                               nthreads=seq.threads_default())
        cpu_s = time.perf_counter() - t0
        o_gpu = o0[:, :, heads].cpu().double().numpy()
        rms = math.sqrt(float(np.mean(o_ref * o_ref)))
        c3["parity"] = {"sample": f"segment 0, heads {heads}, every output, vs fp64 oracle",
                        "max_err_over_rms": float(np.max(np.abs(o_gpu - o_ref)) / rms), "tolerance": 2e-2}
        rate = len(heads) * T / cpu_s
        c3["cpu_oracle"] = {"sample": f"{len(heads)} heads x {T} tokens (segment 0), {cpu_s:.2f} s on "
                                      f"{min(len(heads), seq.threads_default())} threads (one per head)",
                            "token_heads_per_s": round(rate, 1),
                            "extrapolated_s_for_whole_run": round(B * nseg * T * H / rate, 1),
                            "extrapolation": "labelled estimate: the measured per-token-head rate times the run's "
                                             f"{B * nseg * T * H} token-heads"}
    out["B1_H32_T1048576_16_segments"] = c3
    log(f"  {ms3:.3f} ms per pass ({ms3 / nseg:.3f} ms per segment)"
        + (f"; parity {c3['parity']['max_err_over_rms']:.2e}" if "parity" in c3 else ""))
    del segs, state, o, o0, ws

    # ---- linear cost (page "How a Frontier Model Gets Built...", Technical
    # Details: cost proportional to n): throughput per token-head should not
    # depend on the length or the batch shape
    th2 = B * T * H / (ms_c2 * 1e-3)
    rates = {"B4_H16_T8192": c1["token_heads_per_s"], "B1_H32_T65536": round(th2, 1),
             "B1_H32_T1048576_16_segments": c3["token_heads_per_s"]}
    ratio = {n: round(r / th2, 4) for n, r in rates.items()}
    out["linear_cost_check"] = {"token_heads_per_s": rates, "ratio_to_T65536": ratio,
                                "within_15_percent": all(0.85 <= x <= 1.15 for x in ratio.values()),
                                "note": "token-heads/s (the configurations differ in H, so tokens/s alone would "
                                        "compare different work per token)"}
    log(f"  linear cost: ratios to T=65536 {ratio}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=DSTEPS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the B=4 H=16 T=8192 and million-token prefill lines")
    ap.add_argument("--probe", choices=("fused", "stages", "copy", "stamps"))
    ap.add_argument("--calls", type=int, default=3)
    ap.add_argument("--heads", type=int, default=H, help="heads of the --probe fused/stages workload")
    ap.add_argument("--summarize")
    ap.add_argument("--summarize-pmc", nargs=6)
    args = ap.parse_args()
    if args.summarize:
        summarize_trace(args.summarize)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.probe == "stamps":
        probe_stamps(args.calls)
        return
    if args.probe:
        probe(args.probe, args.calls, args.heads)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards by "
              "(batch, head) with no exchange, see DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_96_amd import kda, synth

    dev = torch.device("cuda:0")
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)

    # ---------------- inputs (seeded, synthetic), resident in HBM
    log(f"generating prefill inputs B={B} H={H} T={T} dk={DK} dv={DV}")
    t_gen = time.time()
    d = synth.make_inputs(B, T, H, DK, DV, seed=2)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16)
    host = {n: bf(d[n]) for n in ("q", "k", "v", "beta", "z")}
    q, k, v, beta, z = (host[n].to(dev) for n in ("q", "k", "v", "beta", "z"))
    A = torch.from_numpy(d["A"].copy()).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    log(f"inputs ready in {time.time() - t_gen:.1f}s")
    g, _ = kda.prepare_decay(z, A, want_gcum=False)
    ws = kda.alloc_workspace(B, T, H, DK, DV, torch.bfloat16, dev)
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=dev)
    ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        kda.fwd_chunked(q, k, v, g, beta, h0, ht=ht, workspace=ws, out=o)

    # ---------------- timed prefill
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"prefill: {ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f})")

    if kda.workspace_error(ws) != 0:
        raise RuntimeError("fused prefill reported a hand-off timeout")

    # reference: the two-kernel schedule (every chunk record through HBM), per kernel
    ws2 = kda.alloc_workspace(B, T, H, DK, DV, torch.bfloat16, dev, stages=True)
    o2 = torch.empty_like(o)

    def time_stage(stages, n):
        for _ in range(3):
            kda.fwd_chunked(q, k, v, g, beta, h0, ht=None, final_state=False, workspace=ws2, out=o2, stages=stages)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            kda.fwd_chunked(q, k, v, g, beta, h0, ht=None, final_state=False, workspace=ws2, out=o2, stages=stages)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n_k = max(4, args.steps // 2)
    ms_intra = time_stage(1, n_k)
    ms_state = time_stage(2, n_k)
    same = bool(torch.equal(o, o2))
    del ws2, o2
    log(f"two-kernel schedule: intra-chunk {ms_intra:.3f} ms + state pass {ms_state:.3f} ms; same output {same}")

    flop, abytes = prefill_alg_counts(B, T, H, DK, DV, CHUNK)
    _, abytes32 = prefill_alg_counts(B, T, H, DK, DV, CHUNK, out_bytes=4)

    # ---------------- decay gate (z -> g) at the same shape, on its own
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g_tmp = torch.empty_like(g)

    def gate_call():
        kda.lib().kda_prepare_decay(z.data_ptr(), A.data_ptr(), -5.0, g_tmp.data_ptr(), None, kda.KDA_BF16, B, T, H,
                                    DK, CHUNK, stream.cuda_stream)

    gate_call()
    e0.record(stream)
    for _ in range(n_k):
        gate_call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_gate = e0.elapsed_time(e1) / n_k
    gate_bytes = 2 * 2 * B * T * H * DK + 4 * H
    assert torch.equal(g_tmp, g)
    del g_tmp
    log(f"decay gate z -> g: {ms_gate * 1e3:.1f} us ({gate_bytes / (ms_gate * 1e-3) / 1e9:.0f} GB/s)")

    extra = None if args.no_extra_configs else extra_configs(args, torch, kda, synth, dev, stream, log, ms_step)

    # ---------------- unbounded-decay ablation: the same workload through the
    # kernel for a log-decay with no lower bound (diagonal tiles by position
    # pairs), on the bounded g and on the unbounded -Softplus gate of the same
    # z and A; parity of the latter on two whole heads
    ablation = None
    if not args.no_ablation:
        o_a = torch.empty_like(o)
        ht_a = torch.empty_like(ht)

        def time_unbounded(gg, n):
            for _ in range(3):
                kda.fwd_chunked(q, k, v, gg, beta, h0, ht=ht_a, workspace=ws, out=o_a, unbounded=True)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                kda.fwd_chunked(q, k, v, gg, beta, h0, ht=ht_a, workspace=ws, out=o_a, unbounded=True)
            e1.record(stream)
            torch.cuda.synchronize()
            if kda.workspace_error(ws) != 0:
                raise RuntimeError("unbounded prefill reported a hand-off timeout")
            return e0.elapsed_time(e1) / n

        ms_u_bounded = time_unbounded(g, n_k)
        g_sp, _ = kda.prepare_decay(z, A, want_gcum=False, softplus=True)
        ms_u_sp = time_unbounded(g_sp, n_k)
        g_sp_min = float(g_sp.float().min())
        ab_parity = None
        if not args.no_cpu_baseline:
            from oracle import gate as ogate
            from oracle import seq

            heads = [3, 28]
            f = lambda t: t.float().numpy()
            sel = lambda t: f(t[:, :, heads].cpu())
            o_ref, _ = seq.kda_seq(sel(q), sel(k), sel(v), sel(g_sp), sel(beta), d["h0"][:, heads],
                                   nthreads=seq.threads_default())
            o_gpu = o_a[:, :, heads].cpu().double().numpy()
            rms = math.sqrt(float(np.mean(o_ref * o_ref)))
            ab_parity = {"sample": f"o of heads {heads}, all {T} tokens, vs fp64 oracle on the same bf16 g",
                         "max_err_over_rms": float(np.max(np.abs(o_gpu - o_ref)) / rms), "tolerance": 2e-2}
        ablation = {
            "what": "same workload through kda_fwd_chunked_unbounded (decay with no lower bound: the 4 diagonal "
                    "16x16 tiles of A and M per chunk as fp32 position-pair sums instead of rescaled dense MFMA "
                    "tiles)",
            "bounded_kernel_ms": round(ms_step, 4),
            "unbounded_kernel_ms_bounded_g": round(ms_u_bounded, 4),
            "unbounded_kernel_ms_softplus_g": round(ms_u_sp, 4),
            "softplus_g_min": round(g_sp_min, 2),
            "slowdown": round(ms_u_sp / ms_step, 3),
            "mfma_frac_bounded": round(flop / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "mfma_frac_unbounded": round(flop / (ms_u_sp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "parity_unbounded_softplus_g": ab_parity,
        }
        log(f"ablation: unbounded kernel {ms_u_bounded:.3f} ms (bounded g), {ms_u_sp:.3f} ms (softplus g, "
            f"min {g_sp_min:.1f}) vs bounded {ms_step:.3f} ms"
            + (f"; parity {ab_parity['max_err_over_rms']:.2e}" if ab_parity else ""))
        del o_a, ht_a, g_sp

    # ---------------- variable-length packed batch with prefix-state snapshots:
    # the same 65536 tokens and 32 heads as 11 sequences of a geometric length
    # mix, a state snapshot every 64 chunks (4096 tokens)
    varlen = None
    if not args.no_varlen:
        lengths = [32768, 16384, 8192, 4096, 2048, 1024, 512, 256, 128, 64, 64]
        cu = [0]
        for L_ in lengths:
            cu.append(cu[-1] + L_)
        assert cu[-1] == T
        every = 64
        h0v = torch.zeros((len(lengths), H, DK, DV), dtype=torch.float32, device=dev)
        o_v = torch.empty_like(o)
        res = {}

        def run_varlen():
            res["o"], res["ht"], res["snaps"] = kda.fwd_chunked_varlen(q, k, v, g, beta, cu, h0v, snap_every=every,
                                                                       workspace=ws, out=o_v)

        for _ in range(10):   # (it follows other kernels: let the clock settle)
            run_varlen()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_k):
            run_varlen()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_v = e0.elapsed_time(e1) / n_k
        v_parity = None
        if not args.no_cpu_baseline:
            from oracle import seq

            heads, si = [0, 17], 2          # the 8192-token sequence: its output and its snapshot at 4096
            a_, b_ = cu[si], cu[si + 1]
            f = lambda t: t.float().cpu().numpy()
            sel = lambda t, hi=None: f(t[:, a_:(b_ if hi is None else a_ + hi)][:, :, heads])
            o_ref, _ = seq.kda_seq(sel(q), sel(k), sel(v), sel(g), sel(beta), None, nthreads=seq.threads_default())
            _, s_ref = seq.kda_seq(sel(q, 4096), sel(k, 4096), sel(v, 4096), sel(g, 4096), sel(beta, 4096), None,
                                   nthreads=seq.threads_default())
            sidx = sum((((L_ + 63) // 64) - 1) // every for L_ in lengths[:si])
            o_gpu = res["o"][:, a_:b_][:, :, heads].cpu().double().numpy()
            s_gpu = res["snaps"][sidx][heads].cpu().double().numpy()[None]
            rms = lambda x: math.sqrt(float(np.mean(x * x)))
            v_parity = {"sample": f"sequence {si} ({lengths[si]} tokens), heads {heads}: output and the snapshot "
                                  f"after 4096 tokens vs fp64 oracle",
                        "max_err_over_rms_o": float(np.max(np.abs(o_gpu - o_ref)) / rms(o_ref)),
                        "max_err_over_rms_snapshot": float(np.max(np.abs(s_gpu - s_ref)) / rms(s_ref)),
                        "tolerance": 2e-2}
        varlen = {"workload": f"{len(lengths)} packed sequences of {lengths} tokens (sum {T}), H={H}, "
                              f"dk=dv={DK}, zero initial states, a state snapshot every {every} chunks",
                  "ms_per_call": round(ms_v, 4), "tokens_per_s": round(T / (ms_v * 1e-3), 1),
                  "snapshots": int(res["snaps"].shape[0]) if res["snaps"] is not None else 0,
                  "single_sequence_ms": round(ms_step, 4), "parity": v_parity}
        log(f"varlen: {ms_v:.3f} ms per call ({varlen['snapshots']} snapshots)"
            + (f"; parity o {v_parity['max_err_over_rms_o']:.2e}, snapshot "
               f"{v_parity['max_err_over_rms_snapshot']:.2e}" if v_parity else ""))
        del o_v, h0v, res

    # ---------------- the layer's steps fused in: gate of z in the scan, q/k
    # row normalisation in the kernel, sigmoid output gate on o; against the
    # same steps as separate passes (decay kernel, torch normalisation and gate)
    layer_res = None
    if not args.no_layer:
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        og = (2.0 * torch.randn((B, T, H, DV), generator=gen, device=dev)).to(torch.bfloat16)
        o_l = torch.empty_like(o)
        ht_l = torch.empty_like(ht)

        def fused_layer():
            kda.fwd_chunked_layer(q, k, v, z, A, beta, h0, og=og, qk_l2norm=True, ht=ht_l, workspace=ws, out=o_l)

        def separate_steps():
            gg, _ = kda.prepare_decay(z, A, want_gcum=False)
            nrm = lambda x: (x.float() * torch.rsqrt((x.float() ** 2).sum(-1, keepdim=True) + 1e-6)).to(x.dtype)
            oo, _ = kda.fwd_chunked(nrm(q), nrm(k), v, gg, beta, h0, ht=ht_l, workspace=ws)
            return oo * torch.sigmoid(og.float())

        def timed(fn, n):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        ms_fused_l = timed(fused_layer, n_k)
        ms_sep = timed(separate_steps, n_k)
        o_sep = separate_steps()
        fused_layer()
        torch.cuda.synchronize()
        agree = float((o_l - o_sep).abs().max() / o_sep.pow(2).mean().sqrt())
        l_parity = None
        if not args.no_cpu_baseline:
            from oracle import gate as ogate
            from oracle import layer as olayer
            from oracle import seq

            heads = [6, 25]
            f = lambda t: t[:, :, heads].float().cpu().numpy()
            bfr = lambda x: torch.from_numpy(x).to(torch.bfloat16).float().numpy()
            qn, kn = bfr(olayer.l2norm_rows(f(q))), bfr(olayer.l2norm_rows(f(k)))
            o_ref, _ = seq.kda_seq(qn, kn, f(v), ogate.gate(f(z), d["A"][heads]), f(beta), d["h0"][:, heads],
                                   nthreads=seq.threads_default())
            o_ref = olayer.output_gate(o_ref, f(og))
            err = lambda o, ref: float(np.max(np.abs(o[:, :, heads].cpu().double().numpy() - ref))
                                       / math.sqrt(float(np.mean(ref ** 2))))
            # the separate steps hand the recurrence g rounded to bf16 (the
            # decay pass's output type); their oracle takes that g
            gsep, _ = kda.prepare_decay(z, A, want_gcum=False)
            o_ref_s, _ = seq.kda_seq(qn, kn, f(v), f(gsep), f(beta), d["h0"][:, heads], nthreads=seq.threads_default())
            o_ref_s = olayer.output_gate(o_ref_s, f(og))
            l_parity = {"sample": f"o of heads {heads}, all {T} tokens, vs fp64 oracle (gate of z, row "
                                  "normalisation rounded to bf16, output gate)",
                        "max_err_over_rms": err(o_l, o_ref), "tolerance": 2e-2,
                        "separate_steps_max_err_over_rms": err(o_sep, o_ref_s)}
        layer_res = {"workload": "same prefill with z + A (decay gate in the scan), q/k row L2 normalisation in "
                                 "the kernel and a sigmoid output gate og [B,T,H,dv] bf16",
                     "fused_ms": round(ms_fused_l, 4), "separate_steps_ms": round(ms_sep, 4),
                     "fused_vs_separate_max_err_over_rms": agree,
                     "fused_vs_separate_note": "each path is held to 2e-2 of its own fp64 oracle (the fused kernel "
                                               "keeps g in fp32, the separate steps round it to bf16), so the two "
                                               "may differ by up to 4e-2",
                     "parity": l_parity}
        log(f"layer: fused {ms_fused_l:.3f} ms vs separate steps {ms_sep:.3f} ms; agreement {agree:.2e}"
            + (f"; parity {l_parity['max_err_over_rms']:.2e} (separate steps "
               f"{l_parity['separate_steps_max_err_over_rms']:.2e})" if l_parity else ""))
        del og, o_l, ht_l, o_sep

    # ---------------- backward of the same prefill (forward recompute included)
    bwd = None
    if not args.no_backward:
        do_h, dht_h = synth.output_grads(4, B, T, H, DK, DV)
        do_d, dht_d = torch.from_numpy(do_h).to(dev), torch.from_numpy(dht_h).to(dev)
        ws_b = torch.empty(kda.bwd_workspace_bytes(B, T, H, DK, DV, torch.bfloat16), dtype=torch.uint8, device=dev)
        grads = kda.bwd_chunked(q, k, v, g, beta, h0, do_d, dht_d, workspace=ws_b)

        def bwd_call():
            kda.bwd_chunked(q, k, v, g, beta, h0, do_d, dht_d, workspace=ws_b, out=grads)

        bwd_call()
        torch.cuda.synchronize()
        nb = max(3, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(nb):
            bwd_call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_b = e0.elapsed_time(e1) / nb
        bflop, bbytes = bwd_alg_counts(B, T, H, DK, DV)
        fflop, _ = prefill_alg_counts(B, T, H, DK, DV)
        b_tf = bflop / (ms_b * 1e-3) / 1e12
        # lower bound of the call: backward flops on fp32 MFMA, the recompute on bf16 MFMA
        b_bound = max(bflop / (FP32_PEAK_TFLOPS * 1e12) + fflop / (BF16_PEAK_TFLOPS * 1e12),
                      bbytes / (HBM_PEAK_GBS * 1e9)) * 1e3
        b_parity = None
        if not args.no_cpu_baseline:
            from oracle import seq

            heads = [3, 28]
            f = lambda t: t[:, :, heads].float().cpu().numpy()
            gb = g[:, :, heads].float().cpu().numpy()
            ref = seq.kda_seq_bwd(f(q), f(k), f(v), gb, f(beta), d["h0"][:, heads], do_h[:, :, heads],
                                  dht_h[:, heads], nthreads=2)
            worst = {}
            for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
                x = (grads[n][:, heads] if n == "dh0" else grads[n][:, :, heads]).double().cpu().numpy()
                r = ref[n]
                rms = math.sqrt(float(np.mean(r * r)))
                worst[n] = float(np.max(np.abs(x - r) / (rms + np.abs(r))))
            b_parity = {"sample": f"gradients of heads {heads}, all {T} tokens, vs the fp64 oracle gradient",
                        "max_elementwise_err": worst, "rule": "|x - ref| <= tau (rms(ref) + |ref|)",
                        "tolerance": 2e-2}
        bwd = {"workload": f"gradients of the same prefill (dq, dk, dv, dg, dbeta, dh0; fp32 out) given seeded "
                           f"do [B,T,H,dv] and dht, kda_bwd_chunked (recomputes the forward)",
               "ms_per_call": round(ms_b, 4), "tokens_per_s": round(B * T / (ms_b * 1e-3), 1),
               "alg_flop_per_call": int(bflop), "recompute_flop_per_call": int(fflop),
               "roofline": {"bound": "mfma", "achieved": round(b_tf, 2), "peak": FP32_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(b_tf / FP32_PEAK_TFLOPS, 4), "traffic": None,
                            "note": "backward flops (fp32 MFMA) over the whole call's time"},
               "binding_roofline_frac": round(b_bound / ms_b, 4),
               "parity": b_parity}
        log(f"backward: {ms_b:.3f} ms per call, {b_tf:.1f} TFLOP/s fp32 ({b_tf / FP32_PEAK_TFLOPS:.1%})"
            + (f"; parity {max(b_parity['max_elementwise_err'].values()):.2e}" if b_parity else ""))
        del ws_b, grads, do_d, dht_d

    tok_s = B * T / (ms_step * 1e-3)
    gbs = abytes / (ms_step * 1e-3) / 1e9
    gbs32 = abytes32 / (ms_step * 1e-3) / 1e9
    tflops = flop / (ms_step * 1e-3) / 1e12
    bind_ms = max(flop / (BF16_PEAK_TFLOPS * 1e12), abytes / (HBM_PEAK_GBS * 1e9)) * 1e3

    # ---------------- decode (B=256, H=32, fp32 state 512 MiB, 1000 steps)
    decode = None
    if not args.no_decode:
        log(f"decode B={DB} H={DH} steps={args.decode_steps}")
        st = torch.from_numpy(synth.initial_state(3, DB, DH, DK, DV)).to(dev)
        pool, lpool = [], []
        for s in range(DPOOL):
            tk = synth.decode_tokens(DB, DH, DK, DV, seed=3, step=s)
            tq, tkk, tv, tb, tz = (bf(tk[n]).to(dev) for n in ("q", "k", "v", "beta", "z"))
            tg, _ = kda.prepare_decay(tz[:, None].contiguous(), torch.from_numpy(tk["A"]).to(dev), want_gcum=False)
            pool.append((tq, tkk, tv, tg[:, 0].contiguous(), tb))
            tog = bf(2.0 * tk["v"]).to(dev)   # an output-gate pre-activation of the same shape as v
            lpool.append((tq, tkk, tv, tz, tb, tog))
        A_dec = torch.from_numpy(synth.decode_tokens(DB, DH, DK, DV, seed=3, step=0)["A"]).to(dev)
        od = torch.empty((DB, DH, DV), dtype=torch.float32, device=dev)
        for s in range(5):
            kda.decode_step(*pool[s % DPOOL], st, out=od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.decode_steps):
            kda.decode_step(*pool[s % DPOOL], st, out=od)
        e1.record(stream)
        torch.cuda.synchronize()
        d_ms = e0.elapsed_time(e1) / args.decode_steps
        d_bytes = decode_alg_bytes(DB, DH, DK, DV)
        d_gbs = d_bytes / (d_ms * 1e-3) / 1e9
        # the same steps with the layer's steps fused in (gate of z, q/k
        # normalisation, output gate): z replaces g, og adds 2 dv bytes
        def layer_step(s):
            q_, k_, v_, z_, b_, og_ = lpool[s % DPOOL]
            kda.decode_step_layer(q_, k_, v_, z_, A_dec, b_, st, og=og_, qk_l2norm=True, out=od)
        for s in range(5):
            layer_step(s)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(args.decode_steps):
            layer_step(s)
        e1.record(stream)
        torch.cuda.synchronize()
        dl_ms = e0.elapsed_time(e1) / args.decode_steps
        dl_bytes = d_bytes + DB * DH * 2 * DV
        dl_gbs = dl_bytes / (dl_ms * 1e-3) / 1e9
        decode = {
            "workload": f"KDA decode step B={DB} H={DH} dk=dv={DK}, fp32 state, {args.decode_steps} consecutive steps "
                        f"(token inputs cycle through {DPOOL} seeded steps)",
            "us_per_step": round(d_ms * 1e3, 2),
            "tokens_per_s": round(DB / (d_ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(d_gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "alg_bytes_per_step": d_bytes,
            "layer_steps": {"what": "kda_decode_step_layer: gate of z, q/k L2 normalisation, sigmoid output gate",
                            "us_per_step": round(dl_ms * 1e3, 2), "alg_bytes_per_step": dl_bytes,
                            "hbm_frac": round(dl_gbs / HBM_PEAK_GBS, 4)},
        }
        log(f"decode: {d_ms * 1e3:.1f} us/step, {d_gbs:.0f} GB/s; with the layer steps "
            f"{dl_ms * 1e3:.1f} us/step, {dl_gbs:.0f} GB/s")
        del st, pool, lpool

    # ---------------- parity of the timed output on a sample + CPU oracle baseline
    parity = None
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gate as ogate
        from oracle import seq

        Ts = T       # sample: the whole sequence, all heads
        f = lambda t: t.float().numpy()
        nthreads = seq.threads_default()
        # whole passes of the oracle until about 10 s of CPU work (at most 6)
        passes, t_c0 = 0, time.perf_counter()
        while passes < 6 and (passes == 0 or time.perf_counter() - t_c0 < 10.0):
            gs = ogate.gate(f(host["z"][:, :Ts]), d["A"]).astype(np.float32)
            g_ref = f(torch.from_numpy(gs).to(torch.bfloat16))
            o_ref, _ = seq.kda_seq(f(host["q"][:, :Ts]), f(host["k"][:, :Ts]), f(host["v"][:, :Ts]), g_ref,
                                   f(host["beta"][:, :Ts]), d["h0"], nthreads=nthreads)
            passes += 1
        cpu_s = time.perf_counter() - t_c0
        cpu = {"value": round(passes * B * Ts / cpu_s, 1), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
               "sample": f"fp64 sequential recurrence (+ fp64 gate) on the whole B={B} H={H} T={Ts} workload, "
                         f"all heads, {passes} passes in {cpu_s:.1f} s"}
        o_gpu = o[:, :Ts].cpu().double().numpy()
        rms = math.sqrt(float(np.mean(o_ref * o_ref)))
        parity = {"sample": f"o[:, :{Ts}] all heads vs fp64 oracle (oracle gate of the same z, rounded to bf16)",
                  "max_err_over_rms": float(np.max(np.abs(o_gpu - o_ref)) / rms), "tolerance": 2e-2}
        log(f"cpu oracle {cpu['value']} tokens/s on {nthreads} threads; parity {parity['max_err_over_rms']:.2e}")

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta=sigmoid(N(0,1)), "
                "g=-5*sigmoid(exp(A) z), z N(0,1), A U(-1,1), h0 N(0,0.02))",
        "config": {"workload": f"KDA chunked prefill B={B} H={H} T={T} dk=dv={DK} chunk {CHUNK}, bf16 "
                               f"q/k/v/beta/g inputs, fp32 state and output",
                   "B": B, "H": H, "T": T, "dk": DK, "dv": DV, "chunk": CHUNK},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "fused_fwd_kernel (one launch per call, after two 64-thread flag-clearing kernels; "
                               "HIP events bracket the whole call)",
                     "alg_bytes_per_call": int(abytes),
                     "alg_bytes_basis": "1282 B per token-head (bf16 q, k, g, v read, o counted at 2 B, beta) "
                                        "+ fp32 h0 read and ht written per head",
                     "frac_with_fp32_output": round(gbs32 / HBM_PEAK_GBS, 4),
                     "alg_bytes_per_call_fp32_output": int(abytes32)},
        "mfma": {"achieved_tflops": round(tflops, 2), "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "alg_flop_per_call": int(flop)},
        "binding_roofline_frac": round(bind_ms / ms_step, 4),
        "kernels_ms": {"fused_fwd_kernel (per call)": round(ms_step, 4),
                       "prepare_decay_kernel (gate z -> g, same shape)": round(ms_gate, 4),
                       "prepare_decay_gbs": round(gate_bytes / (ms_gate * 1e-3) / 1e9, 1),
                       "two_kernel_schedule": {"intra_chunk_kernel": round(ms_intra, 4),
                                               "state_pass_kernel": round(ms_state, 4),
                                               "bitwise_equal_output": same}},
        "other_prefill_configs": extra,
        "decode": decode,
        "unbounded_decay_ablation": ablation,
        "varlen_snapshots": varlen,
        "layer_prologue_epilogue": layer_res,
        "backward": bwd,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
