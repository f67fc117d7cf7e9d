"""Build ``libhipdecode.so`` in-tree with hipcc for gfx950.

Run ``python -m paged_kv_decode_gqa_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles.  ``--save-temps DIR`` keeps the device assembly for
inspection of register counts and instruction selection.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhipdecode.so")
SOURCES = ["api.hip", "paged_decode.hip", "kv_append.hip", "prefill_attn.hip", "step_runner.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    # keep the compiler away from packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(out: str = LIB, save_temps: str | None = None, extra_flags: list[str] | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp, *srcs]
    cwd = None
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps")
        cwd = save_temps
    with tempfile.TemporaryDirectory() as td:
        env = dict(os.environ, TMPDIR=td)
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd, env=env)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    args = ap.parse_args()
    print(build(save_temps=args.save_temps))
