"""Build the stage library (HIP for gfx950) in-tree: pipeline_stage_decoder_amd/libpsd_stage.so."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpsd_stage.so")
SOURCES = ["capi.hip", "pipeline.hip", "placement.hip", "kernels_misc.hip", "kernels_gemv.hip", "kernels_gemm.hip", "kernels_attn.hip"]
# Packed FP32 instructions are disabled for all device code; hipcc's host pass warns that it does
# not know the feature, which is harmless.
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(force: bool = True, jobs: int = 8, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ["hipcc", *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
        if verbose and lines:
            print("\n".join(lines), file=sys.stderr)
    tmp = LIB + ".tmp"
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
