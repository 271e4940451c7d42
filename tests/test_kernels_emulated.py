"""The HIP kernels' own source, run on the CPU.

api.hip, pack.hip and attention.hip are compiled for x86 by clang++ against the
emulation shim in tests/emu (one host thread per lane, wave intrinsics, MFMA,
global_load_lds and the transposing LDS read emulated from their documented or
measured lane layouts) with AddressSanitizer and UndefinedBehaviorSanitizer
(signed overflow, shifts, invalid loads, division; any report aborts), and driven through the Python
binding and the C ABI on host tensors.  Every entry point is checked:
rattn_pack, rattn_forward and rattn_unpack against the oracle (the scan and
the row movement bit-exact, attention within the per-dtype tolerances of
`_gpu_util`), rattn_fused bitwise against the three-call path,
rattn_fused_padded bitwise against rattn_fused, and rattn_repack bit-exact
against the oracle.  Any out-of-bounds global or
LDS access aborts the run.

These cases run the same kernels as the GPU parity tests, on the host, where
AddressSanitizer can see every access.  The emulation does not model timing, memory
ordering between workgroups or the wave scheduler, so it cannot show a hang or
a race; it shows indexing, bounds and arithmetic.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "ragged_variable_length_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def emu_lib(tmp_path_factory):
    rt = _asan_runtime()
    if not os.path.exists(CLANG) or rt is None:
        pytest.skip("clang++ with the AddressSanitizer runtime is not installed")
    out = str(tmp_path_factory.mktemp("emu") / "librattn_emu.so")
    # RATTN_LAUNCH_GGL: the emulated runtime runs a kernel as a function call
    # (hipLaunchKernelGGL), not through a device function handle
    cmd = [CLANG, "-std=c++20", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared-libasan", "-fno-omit-frame-pointer", "-w", "-DRATTN_LAUNCH_GGL",
           "-I", os.path.join(HERE, "emu"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "c++", os.path.join(HERE, "emu", "emu_runtime.cpp"),
           os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "pack.hip"),
           os.path.join(CSRC, "attention.hip"), os.path.join(CSRC, "repack.hip"), "-o", out,
           "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out, rt


def _run(emu_lib, *cases):
    lib, rt = emu_lib
    env = {**os.environ, "LD_PRELOAD": rt, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0"}
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "emu", "run_cases.py"), lib,
                        *cases], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout)
    assert r.returncode == 0 and "EMULATED CASES PASSED" in r.stdout, \
        (r.stdout[-3000:] + r.stderr[-6000:])


def test_emulated_tiny_fp32(emu_lib):
    _run(emu_lib, "tiny")


def test_emulated_16bit_sequential_cores(emu_lib):
    _run(emu_lib, "seq16")


def test_emulated_f32_sequential_core(emu_lib):
    _run(emu_lib, "f32_sequential")


def test_emulated_ragged_lengths_all_dtypes(emu_lib):
    _run(emu_lib, "ragged")


def test_emulated_max_seqlen_bounds(emu_lib):
    _run(emu_lib, "bounds")


def test_emulated_long_sequences(emu_lib):
    _run(emu_lib, "long")


def test_emulated_padded_comparator_matches_ragged(emu_lib):
    _run(emu_lib, "padded")


def test_emulated_repack(emu_lib):
    _run(emu_lib, "repack")


def test_emulated_scan_over_single_launch_limit(emu_lib):
    _run(emu_lib, "scan_large")


def test_emulated_small_rows_and_everything_pruned(emu_lib):
    _run(emu_lib, "small_rows", "everything_pruned")


def test_emulated_pack_subsets_and_unpack_modes(emu_lib):
    _run(emu_lib, "pack_subsets")
