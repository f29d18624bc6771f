"""Driver for hardware-counter runs (rocprofv3 --pmc) of the prefill kernels.

Runs a few calls of one schedule on the long-prefill workload (B=1, H=32,
T=65536, dk=dv=128, bf16 inputs, seeded synthetic data) and, for scaling
the memory counters, a plain device copy of a known size:

  python -m gated_delta_rule_96_amd.pmc_probe --what fused  --calls 3
  python -m gated_delta_rule_96_amd.pmc_probe --what stages --calls 3
  python -m gated_delta_rule_96_amd.pmc_probe --what copy   --calls 3

Under `rocprofv3 --pmc FETCH_SIZE --kernel-trace -- python -m ...` each
dispatch gets its counter values; the copy moves exactly COPY_BYTES in each
direction per call, which calibrates FETCH_SIZE / WRITE_SIZE (KiB per
dispatch) into bytes.
"""
from __future__ import annotations

import argparse
import sys

B, H, T, DK, DV = 1, 32, 65536, 128, 128
COPY_BYTES = 1 << 30


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--what", choices=("fused", "stages", "copy"), required=True)
    ap.add_argument("--calls", type=int, default=3)
    args = ap.parse_args()

    import torch

    from gated_delta_rule_96_amd import kda, synth

    dev = torch.device("cuda:0")
    if args.what == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.calls):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[pmc_probe] copy of {COPY_BYTES} bytes x {args.calls}", file=sys.stderr)
        return

    d = synth.make_inputs(B, T, H, DK, DV, seed=2)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
    q, k, v, beta, z = (bf(d[n]) for n in ("q", "k", "v", "beta", "z"))
    A = torch.from_numpy(d["A"].copy()).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    g, _ = kda.prepare_decay(z, A, want_gcum=False)
    stages = args.what == "stages"
    ws = kda.alloc_workspace(B, T, H, DK, DV, torch.bfloat16, dev, stages=stages)
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=dev)
    ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    for _ in range(args.calls):
        kda.fwd_chunked(q, k, v, g, beta, h0, ht=ht, workspace=ws, out=o, stages=3 if stages else None)
    torch.cuda.synchronize()
    print(f"[pmc_probe] {args.what} x {args.calls} done", file=sys.stderr)


if __name__ == "__main__":
    main()
