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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer: each -fsanitize= applies to the host
# pass only (-Xarch_host); device code is built as usual and never runs under them.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(force: bool = True, jobs: int = 8, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    return _build(os.path.join(PKG, "_build"), LIB, HIPFLAGS, ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"],
                  jobs, verbose)


def build_host_sanitized(outdir: str, jobs: int = 8) -> str:
    """The same library with its host code built under AddressSanitizer and UBSan, into outdir, for
    running the host-side logic (argument checks, planning, placement) on a machine without a GPU.
    Load it with the clang ASan runtime preloaded (asan_runtime())."""
    flags = [f for f in HIPFLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE
    lib = os.path.join(outdir, "libpsd_stage_san.so")
    # linked like the plain library: the sanitizer symbols resolve against the preloaded runtime
    return _build(os.path.join(outdir, "obj"), lib, flags, ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"],
                  jobs, False)


def asan_runtime() -> str:
    """Path of the clang ASan runtime that a host-sanitized library needs preloaded (or '')."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def _build(objdir: str, lib: str, flags, link, jobs: int, verbose: bool) -> str:
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ["hipcc", *flags, "-c", os.path.join(CSRC, src), "-o", obj]
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
    tmp = lib + ".tmp"
    subprocess.check_call([*link, *objs, "-o", tmp], stderr=subprocess.DEVNULL)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
