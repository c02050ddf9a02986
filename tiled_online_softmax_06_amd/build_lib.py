"""Builds libfa.so in-tree with hipcc for gfx950 (no GPU needed to compile).

    python -m tiled_online_softmax_06_amd.build_lib [--asm DIR]

``--asm DIR`` also writes the AMD assembly of the device code to DIR (for
register, LDS and spill checks of this library's own kernels).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("flash_fwd.hip", "flash_fwd_fp8.hip", "flash_bwd.hip", "fa_api.hip")]
OUTPUT = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code never tests for NaN: max/min need no quieting of their
    # inputs (the host side keeps its isfinite checks of the arguments)
    "-Xarch_device", "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = [hipcc()] + FLAGS + SOURCES + ["-o", tmp]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=asm_dir or HERE, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None)
    args = ap.parse_args()
    print(build(args.asm, verbose=True))
