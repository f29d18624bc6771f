"""Build libkda.so (gfx950) in-tree with hipcc.

Every HIP translation unit is compiled with packed fp32 instructions
disabled (-packed-fp32-ops) and linked with the C-ABI layer into
gated_delta_rule_96_amd/libkda.so.  The same objects, with the prefill
kernels compiled once more with KDA_CYCLE_STAMPS, make the profiling build
libkda_stamps.so (include/kda_stamps.h).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libkda.so"
OUT_STAMPS = PKG / "libkda_stamps.so"
BUILD = PKG / "_build"
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["kda_api.cpp", "kda_decay.hip", "kda_chunk.hip", "kda_decode.hip", "kda_bwd.hip", "kda_noalloc.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{ROOT / 'include'}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


STAMPED = "kda_chunk.hip"   # the source whose kernels carry the cycle stamps


def _compile(src: Path, obj: Path, extra=()) -> str:
    lang = ["-x", "hip"] if src.suffix == ".cpp" else []
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def _link(objs, out: Path) -> None:
    tmp = out.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    objs = []
    stamped = BUILD / (Path(STAMPED).stem + "_stamps.o")
    with cf.ThreadPoolExecutor(max_workers=min(6, len(SOURCES) + 1)) as ex:
        futs = {ex.submit(_compile, CSRC / STAMPED, stamped, ("-DKDA_CYCLE_STAMPS",)): STAMPED + " (stamps)"}
        for s in SOURCES:
            src = CSRC / s
            obj = BUILD / (src.stem + ".o")
            objs.append(obj)
            futs[ex.submit(_compile, src, obj)] = s
        for f in cf.as_completed(futs):
            msg = f.result()
            if verbose and msg.strip():
                print(f"[{futs[f]}]\n{msg}", file=sys.stderr)
    _link(objs, OUT)
    _link([stamped if o.name == Path(STAMPED).stem + ".o" else o for o in objs], OUT_STAMPS)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
