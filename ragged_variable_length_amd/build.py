"""Build librattn.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import sysconfig

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librattn.so")
SOURCES = ["api.hip", "pack.hip", "attention.hip", "repack.hip"]
# host-side timing loops used by bench.py (links librattn.so; not product ABI)
BENCH_LIB = os.path.join(HERE, "librattn_bench.so")
BENCH_SOURCES = ["bench_host.hip", "bench_peaks.hip"]
# CPython extension the Python binding calls (argument marshalling, links librattn.so)
EXT = os.path.join(HERE, "_rattn" + sysconfig.get_config_var("EXT_SUFFIX"))
EXT_SOURCE = "pymod.c"

# Device-code flags: gfx950 only; packed-fp32 instruction selection off (the
# compiler would otherwise form v_pk_* float ops on its own); kernel arguments
# preloaded into SGPRs at wave launch (the first 14 dwords, gfx950 code object
# v5), so a wavefront's first addresses do not wait for a scalar load of the
# argument segment.  Each kernel keeps a prologue that loads them itself when
# the firmware does not preload.  Measured on MI355X, rattn_fused at DeiT-S:
# 5.90 -> 5.65 us warm, 9.24 -> 8.9-9.0 us cold, bits unchanged.  Matrix
# instructions write ordinary VGPRs (-amdgpu-mfma-vgpr-form): without it the
# compiler gave the float32 kernels and the few-heads 16-bit kernels 16-36
# accumulation registers and 72-582 copies between them and the VGPRs that
# the softmax reads; the other kernels are unchanged by it.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-mllvm", "-amdgpu-kernarg-preload-count=16",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librattn.so)")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile librattn.so, librattn_bench.so and the _rattn extension next to
    this file (always rebuilds)."""
    _compile(LIB, SOURCES, [], verbose, extra_flags)
    _compile(BENCH_LIB, BENCH_SOURCES, ["-L", HERE, "-lrattn", "-Wl,-rpath,$ORIGIN"],
             verbose, extra_flags)
    _compile_ext(verbose)
    return LIB


def _compile_ext(verbose: bool) -> None:
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no C compiler found for the _rattn extension")
    tmp = EXT + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-I", sysconfig.get_paths()["include"], "-I", INCLUDE,
           "-o", tmp, os.path.join(CSRC, EXT_SOURCE), "-L", HERE, "-lrattn",
           "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the _rattn extension failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, EXT)


def _compile(out: str, sources, link_flags, verbose: bool, extra_flags) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), *DEVICE_FLAGS, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
           *extra_flags, "-o", tmp, *[os.path.join(CSRC, s) for s in sources], *link_flags]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose=True))
