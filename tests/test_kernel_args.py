"""The kernel-argument blocks the launchers build on the host (CPU only:
hipcc cross-compiles the device code for gfx950 and the test reads the
code-object metadata it prints).

Every launch writes the kernel's arguments itself into one block, each at its
natural alignment in parameter order (`launch` in csrc/internal.h), and hands
the block to hipModuleLaunchKernel.  That block is only right if the compiler
lays the kernel's explicit parameters out the same way.  This test reads each
kernel's parameter offsets and sizes from the metadata and fails if any
parameter is not at the offset natural-alignment packing gives, or if the
explicit parameters exceed the launcher's block.
"""
import os
import re
import shutil
import subprocess

import pytest
import yaml

from ragged_variable_length_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_variable_length_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# the product build's device flags, so the checked code is the shipped code
DEVICE_FLAGS = build.DEVICE_FLAGS
MAX_KERNARG_BYTES = 512  # kMaxKernArgBytes in csrc/internal.h

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return out.read_text()


def _metadata(src, tmp_path):
    asm = _asm(src, tmp_path)
    m = re.search(r"\.amdgpu_metadata\n(.*?)\n\s*\.end_amdgpu_metadata", asm, re.S)
    assert m, "no code-object metadata in the assembly"
    return yaml.safe_load(m.group(1))


@pytest.mark.parametrize("src", ["attention.hip", "pack.hip", "repack.hip"])
def test_explicit_parameters_follow_natural_alignment(src, tmp_path):
    meta = _metadata(os.path.join(CSRC, src), tmp_path)
    kernels = meta["amdhsa.kernels"]
    assert kernels, "no kernels"
    for k in kernels:
        off = 0
        for a in k[".args"]:
            if a[".value_kind"].startswith("hidden_"):
                continue
            size = a[".size"]
            # scalars and pointers align to their size; a struct passed by value
            # (the only larger parameter) to 8, its widest member
            align = min(size, 8) if size in (1, 2, 4, 8) else 8
            off = (off + align - 1) // align * align
            assert a[".offset"] == off, (k[".name"], a)
            off += size
        assert off <= MAX_KERNARG_BYTES, (k[".name"], off)


@pytest.mark.parametrize("src", ["attention.hip", "pack.hip", "repack.hip"])
def test_kernel_arguments_are_preloaded(src, tmp_path):
    # every kernel whose explicit arguments are scalars and pointers (all the
    # attention kernels) takes its first argument dwords in SGPRs at launch,
    # up to 14 next to the argument-segment pointer, behind a prologue that
    # loads them for firmware without preloading; a structure passed by value
    # (the copy kernels' descriptors) is not preloaded
    asm = _asm(os.path.join(CSRC, src), tmp_path)
    m = re.search(r"\.amdgpu_metadata\n(.*?)\n\s*\.end_amdgpu_metadata", asm, re.S)
    meta = {k[".name"]: k for k in yaml.safe_load(m.group(1))["amdhsa.kernels"]}
    blocks = re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S)
    assert blocks, "no kernel descriptors"
    checked = 0
    for name, body in blocks:
        explicit = [a for a in meta[name][".args"] if not a[".value_kind"].startswith("hidden_")]
        if any(a[".size"] > 8 for a in explicit):
            continue
        n = re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length (\d+)", body)
        assert n and 1 <= int(n.group(1)) <= 14, (name, n and n.group(1))
        checked += 1
    if src == "attention.hip":
        assert checked >= 8, checked
