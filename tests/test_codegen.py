"""Code-generation check of the copy kernels (CPU only: hipcc cross-compiles
the device code for gfx950 and the test reads the assembly it prints).

With a run-time branch on the tensor count (1, 2 or 3 tensors moved per
launch), ROCm 7.2's gfx950 back end structurized the three cases so that on
the three-tensor path the SGPR pair holding the second destination's base
address was left undefined (marked `implicit-def` in the assembly) and the
store went to an unrelated address: an illegal memory access at run time.  The
kernels now take the tensor count as a template parameter.  This test fails if
any 16-byte store of a pack / re-pack kernel takes its base address from an
SGPR pair that the compiler marks as undefined anywhere in that kernel.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_variable_length_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return out.read_text()


def _kernels(asm):
    for m in re.finditer(r"\n(_Z[^\s:]+):[^\n]*\n([\s\S]*?s_endpgm)", asm):
        yield m.group(1), [l.strip() for l in m.group(2).split("\n")]


def _store_bases(lines):
    """(line index, 's[a:b]') for every 16-byte global store whose address is
    formed from an SGPR pair, directly or by the v_lshl_add_u64 that last wrote
    its VGPR address."""
    out = []
    for i, l in enumerate(lines):
        if not l.startswith("global_store_dwordx4"):
            continue
        ops = [o.strip() for o in l.split(None, 1)[1].split(",")]
        if ops[2].startswith("s["):
            out.append((i, ops[2].split()[0]))
            continue
        for j in range(i - 1, -1, -1):
            if lines[j].startswith("v_") and lines[j].split(None, 1)[1].startswith(ops[0] + ","):
                m = re.search(r"s\[\d+:\d+\]", lines[j])
                if m:
                    out.append((i, m.group(0)))
                break
    return out


def _undefined_store_bases(asm, name_filter):
    bad, checked = [], 0
    for name, lines in _kernels(asm):
        if not name_filter(name):
            continue
        undefined = set()
        for l in lines:
            for a, b in re.findall(r"implicit-def: \$sgpr(\d+)_sgpr(\d+)", l):
                undefined.add(f"s[{a}:{b}]")
        for i, base in _store_bases(lines):
            checked += 1
            if base in undefined:
                bad.append((name, i, lines[i], base))
    return bad, checked


@pytest.mark.parametrize("src,kernel", [("pack.hip", "pack_kernel"),
                                        ("repack.hip", "repack_kernel")])
def test_copy_kernel_store_bases_are_defined(src, kernel, tmp_path):
    asm = _device_asm(os.path.join(CSRC, src), tmp_path)
    bad, checked = _undefined_store_bases(asm, lambda n: kernel in n)
    assert checked >= 4, f"found only {checked} 16-byte stores in the {kernel} instantiations"
    assert not bad, f"stores with an undefined SGPR base: {bad}"


def test_checker_flags_a_runtime_tensor_count_branch(tmp_path):
    """The shape of source that was miscompiled (a run-time 1/2/3 branch around
    the stores) is recognised by the checker, so the test above can fail."""
    src = tmp_path / "branchy.hip"
    src.write_text(r"""
#include <hip/hip_runtime.h>
#include <stdint.h>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct Args { const u32x4 *src[3]; u32x4 *dst[3]; const int *list; int n, rv, count; };
__global__ __launch_bounds__(256) void branchy_kernel(Args a) {
    for (int idx = threadIdx.x; idx < a.count * a.rv; idx += 256) {
        const int j = idx / a.rv, p = idx - j * a.rv;
        const int64_t so = (int64_t)a.list[j] * a.rv + p, d = (int64_t)(blockIdx.x + j) * a.rv + p;
        const u32x4 x0 = a.src[0][so];
        if (a.n == 1) { a.dst[0][d] = x0; }
        else if (a.n == 2) { const u32x4 x1 = a.src[1][so]; a.dst[0][d] = x0; a.dst[1][d] = x1; }
        else { const u32x4 x1 = a.src[1][so], x2 = a.src[2][so];
               a.dst[0][d] = x0; a.dst[1][d] = x1; a.dst[2][d] = x2; }
    }
}
""")
    asm = _device_asm(str(src), tmp_path)
    bad, checked = _undefined_store_bases(asm, lambda n: "branchy_kernel" in n)
    assert checked >= 3
    if not bad:
        pytest.skip("this compiler does not miscompile the run-time branch form")
