"""Code-generation check of the copy kernels (CPU only: hipcc cross-compiles
the device code for gfx950 and the test reads the assembly it prints).

With a run-time branch on the tensor count (1, 2 or 3 tensors moved per
launch), ROCm 7.2's gfx950 back end structurized the three cases so that on
the three-tensor path the SGPR pair holding the second destination's base
address was left undefined (marked `implicit-def` in the assembly) and the
store went to an unrelated address: an illegal memory access at run time.  The
kernels now take the tensor count as a template parameter.  This test fails if
any 16-byte store of a pack / re-pack kernel takes its base address from an
SGPR pair that, on some control-flow path to it, holds no value the program
wrote (the compiler marks such a pair `implicit-def`).
"""
import os
import re
import shutil
import subprocess

import pytest

from ragged_variable_length_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_variable_length_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# the product build's device flags, so the checked code is the shipped code
DEVICE_FLAGS = build.DEVICE_FLAGS

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return out.read_text()


def _kernels(asm):
    for m in re.finditer(r"\n(_Z[^\s:]+):[^\n]*\n([\s\S]*?s_endpgm)", asm):
        yield m.group(1), [l.strip() for l in m.group(2).split("\n")]


_LABEL = re.compile(r"^(\.LBB\d+_\d+|; %bb\.\d+):")
_UNDEF = re.compile(r"implicit-def: ((?:\$sgpr\d+_?)+)")
# VOP3b forms: the second operand is a scalar destination (carry / condition)
_SDST2 = ("v_mad_u64_u32", "v_mad_i64_i32", "v_add_co_u32", "v_sub_co_u32", "v_subrev_co_u32",
          "v_addc_co_u32", "v_subb_co_u32", "v_subbrev_co_u32", "v_div_scale")
_NO_DST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_barrier", "s_nop",
           "s_endpgm", "s_setprio", "s_sleep", "s_sendmsg", "s_trap", "s_dcache", "s_store",
           "s_buffer_store", "s_set_gpr_idx", "s_setpc")


def _sregs(op):
    """Scalar registers named by one operand ('s7', 's[4:7]'), else empty."""
    m = re.fullmatch(r"s(\d+)", op) or re.fullmatch(r"s\[(\d+):(\d+)\]", op)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def _defs(line):
    """(registers written, written-as-undefined) by one assembly line."""
    u = _UNDEF.search(line)
    if u:
        return {int(r) for r in re.findall(r"sgpr(\d+)", u.group(1))}, True
    if not line or line.startswith((";", ".")):
        return set(), False
    parts = line.split(None, 1)
    op = parts[0]
    if op.startswith(_NO_DST) or len(parts) < 2:
        return set(), False
    ops = [o.strip() for o in parts[1].split(",")]
    regs = _sregs(ops[0].split()[0])
    if op.startswith(_SDST2) and len(ops) > 1:
        regs |= _sregs(ops[1].split()[0])
    return regs, False


def _cfg(lines):
    """Basic blocks (start, end) of a kernel and each block's predecessors."""
    starts = [0] + [i for i, l in enumerate(lines) if _LABEL.match(l)]
    starts = sorted(set(starts))
    blocks = [(s_, e_) for s_, e_ in zip(starts, starts[1:] + [len(lines)])]
    name_of = {}
    for bi, (s_, _) in enumerate(blocks):
        m = _LABEL.match(lines[s_])
        if m:
            name_of[m.group(1)] = bi
    preds = {bi: set() for bi in range(len(blocks))}
    for bi, (s_, e_) in enumerate(blocks):
        body = [l for l in lines[s_:e_] if l and not l.startswith((";", "."))]
        falls = True
        for l in body:
            op = l.split()[0]
            if op.startswith(("s_cbranch", "s_branch")):
                tgt = l.split()[1]
                if tgt in name_of:
                    preds[name_of[tgt]].add(bi)
                if op == "s_branch":
                    falls = False
            if op in ("s_endpgm", "s_setpc_b64"):
                falls = False
        if falls and bi + 1 < len(blocks):
            preds[bi + 1].add(bi)
    return blocks, preds


def _undefined_on_some_path(lines, blocks, preds, store_line, regs):
    """True if, on some path into `store_line`, the nearest earlier write of
    any register in `regs` is an implicit-def or there is none (kernel entry)."""
    bi = next(b for b, (s_, e_) in enumerate(blocks) if s_ <= store_line < e_)
    work, seen = [(bi, store_line)], set()
    while work:
        b, end = work.pop()
        s_ = blocks[b][0]
        hit = None
        for i in range(end - 1, s_ - 1, -1):
            w, undef = _defs(lines[i])
            if w & regs:
                hit = undef
                break
        if hit is None:
            if b == 0 or not preds[b]:
                return True
            for pb in preds[b]:
                if pb not in seen:
                    seen.add(pb)
                    work.append((pb, blocks[pb][1]))
        elif hit:
            return True
    return False


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
                    out.append((j, m.group(0)))
                break
    return out


def _undefined_store_bases(asm, name_filter):
    """Stores of the selected kernels whose SGPR base pair may hold no value
    written by the program on some control-flow path to the address."""
    bad, checked = [], 0
    for name, lines in _kernels(asm):
        if not name_filter(name):
            continue
        blocks, preds = _cfg(lines)
        for i, base in _store_bases(lines):
            checked += 1
            if _undefined_on_some_path(lines, blocks, preds, i, _sregs(base)):
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
