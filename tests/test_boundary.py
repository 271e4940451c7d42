"""The C ABI boundary on the host (no GPU needed, no kernel launched).

Checks that librattn.so loads, exports every entry point include/rattn.h
declares, and rejects invalid arguments on the host before any HIP call, with
the documented status codes.  Fake device addresses are only passed where the
argument check must fail first, so nothing is ever dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

import ragged_variable_length_amd as rv
from ragged_variable_length_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rattn.h")

OK, INVALID, UNSUPPORTED, NO_DEVICE, HIP = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2
A = 0x10000  # a 16-byte-aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rattn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return rv.load()


def test_header_declares_the_three_path_calls():
    names = declared_functions()
    for n in ("rattn_pack", "rattn_forward", "rattn_unpack", "rattn_init",
              "rattn_status_string", "rattn_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.rattn_version() >> 16 == 1
    for code in (OK, INVALID, UNSUPPORTED, NO_DEVICE, HIP, 99):
        s = rv.status_string(code)
        assert isinstance(s, str) and s


def _fwd(lib, q=A, k=A, v=A, o=A, cu=A, B=2, ms=10, H=2, D=64, scale=0.125, dt=BF16):
    return lib.rattn_forward(q, k, v, o, cu, B, ms, H, D, ctypes.c_float(scale), dt, None)


def test_forward_argument_checks(lib):
    assert _fwd(lib, D=32) == UNSUPPORTED
    assert _fwd(lib, D=128) == UNSUPPORTED
    assert _fwd(lib, dt=7) == INVALID
    assert _fwd(lib, B=-1) == INVALID
    assert _fwd(lib, H=0) == INVALID
    assert _fwd(lib, ms=-3) == INVALID
    assert _fwd(lib, scale=float("nan")) == INVALID
    assert _fwd(lib, scale=float("inf")) == INVALID
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, o=None) == INVALID
    assert _fwd(lib, cu=None) == INVALID
    assert _fwd(lib, k=A + 8) == INVALID  # not 16-byte aligned
    assert _fwd(lib, cu=A + 2) == INVALID  # not 4-byte aligned
    # nothing to do: succeeds without touching the device or the pointers
    assert _fwd(lib, B=0, q=None, k=None, v=None, o=None, cu=None) == OK
    assert _fwd(lib, ms=0, q=None, k=None, v=None, o=None, cu=None) == OK


def _pack(lib, n=3, src=(A, A, A), dst=(A, A, A), keep=A, B=2, N=197, row=384, dt=BF16, cu=A,
          mx=None, tot=None):
    sa = (ctypes.c_void_p * 3)(*src) if src is not None else None
    da = (ctypes.c_void_p * 3)(*dst) if dst is not None else None
    return lib.rattn_pack(sa, da, n, keep, B, N, row, dt, cu, mx, tot, None)


def test_pack_argument_checks(lib):
    assert _pack(lib, n=0) == INVALID
    assert _pack(lib, n=4) == INVALID
    assert _pack(lib, src=None) == INVALID
    assert _pack(lib, dst=None) == INVALID
    assert _pack(lib, src=(A, None, A)) == INVALID
    assert _pack(lib, dst=(A, A, A + 4)) == INVALID
    assert _pack(lib, keep=None) == INVALID
    assert _pack(lib, keep=A + 1) == INVALID
    assert _pack(lib, cu=None) == INVALID
    assert _pack(lib, cu=A + 1) == INVALID
    assert _pack(lib, mx=A + 2) == INVALID
    assert _pack(lib, tot=A + 2) == INVALID
    assert _pack(lib, B=-1) == INVALID
    assert _pack(lib, N=0) == INVALID
    assert _pack(lib, B=1 << 20, N=1 << 12) == INVALID  # B*N beyond int32
    assert _pack(lib, row=0) == INVALID
    assert _pack(lib, row=3, dt=F16) == INVALID  # 6-byte rows are not 16-byte multiples
    assert _pack(lib, dt=9) == INVALID


def _unpack(lib, src=A, dst=A, cls=A, keep=A, cu=A, B=2, N=197, row=384, dt=BF16):
    return lib.rattn_unpack(src, dst, cls, keep, cu, B, N, row, dt, None)


def test_unpack_argument_checks(lib):
    assert _unpack(lib, dst=None, cls=None) == INVALID
    assert _unpack(lib, src=None) == INVALID
    assert _unpack(lib, keep=None) == INVALID
    assert _unpack(lib, cu=None) == INVALID
    assert _unpack(lib, src=A + 8) == INVALID
    assert _unpack(lib, dst=A + 8) == INVALID
    assert _unpack(lib, cls=A + 8) == INVALID
    assert _unpack(lib, N=0) == INVALID
    assert _unpack(lib, row=5, dt=F32) == INVALID
    assert _unpack(lib, B=0, src=None, keep=None, cu=None) == OK


def test_valid_call_without_device_reports_no_device(lib):
    if lib.rattn_init() == OK:
        pytest.skip("a gfx950 device is present; this checks the device-less path")
    assert lib.rattn_init() == NO_DEVICE
    assert _fwd(lib) == NO_DEVICE
    assert _pack(lib) == NO_DEVICE
    assert _unpack(lib) == NO_DEVICE


def test_binding_refuses_host_tensors():
    x = torch.zeros((2, 4, 2, 64), dtype=torch.bfloat16)
    keep = torch.ones((2, 4), dtype=torch.uint8)
    cu = torch.zeros(3, dtype=torch.int32)
    flat = torch.zeros((8, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rv.rattn_pack([x], [flat], keep, cu)
    with pytest.raises(TypeError):
        rv.rattn_forward(flat, flat, flat, flat, cu, 4, 0.125)
    with pytest.raises(TypeError):
        rv.rattn_unpack(flat, keep, cu, dst_padded=x)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _binding.load()


def test_extension_wraps_every_entry_point(lib):
    ext = _binding.ext()
    for name in declared_functions():
        assert hasattr(ext, name[len("rattn_"):]), name
    assert ext.version() == lib.rattn_version()
    assert ext.status_string(INVALID) == rv.status_string(INVALID)
    # the same host-side checks as through ctypes, same codes
    assert ext.forward(A, A, A, A, A, 2, 10, 2, 63, 0.125, BF16, None) == UNSUPPORTED
    assert ext.forward(None, A, A, A, A, 2, 10, 2, 64, 0.125, BF16, None) == INVALID
    assert ext.fused(A, A, A, A, None, None, 2, 10, 2, 64, 10, 0.125, BF16, None) == INVALID
    assert ext.unpack(A, A, A, A, A, 2, 10, 5, F32, None) == INVALID
    assert ext.pack([A], [A], A, 2, 10, 128, 7, A, None, None, None) == INVALID
    with pytest.raises(ValueError):
        ext.pack([A] * 4, [A] * 4, A, 2, 10, 128, BF16, A, None, None, None)
    with pytest.raises(TypeError):
        ext.fused(A, A, A)
    with pytest.raises(OverflowError):
        ext.forward(A, A, A, A, A, 2 ** 40, 10, 2, 64, 0.125, BF16, None)


def test_extension_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "_ext_mod", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _binding.ext()


def test_padded_comparator_argument_checks(lib):
    f = lib.rattn_fused_padded
    # pad_len outside [1, N]
    assert f(A, A, A, A, A, None, 2, 10, 2, 64, 0, ctypes.c_float(0.125), BF16, None) == INVALID
    assert f(A, A, A, A, A, None, 2, 10, 2, 64, 11, ctypes.c_float(0.125), BF16, None) == INVALID
    # the fused checks apply too
    assert f(A, A, A, A, A, None, 2, 10, 2, 63, 5, ctypes.c_float(0.125), BF16, None) == UNSUPPORTED
    assert f(A, A, A, A, None, None, 2, 10, 2, 64, 5, ctypes.c_float(0.125), BF16, None) == INVALID


def test_fused_row_stride_limit(lib):
    """Row strides (H * head_dim elements) must stay below 2^24: the fused
    kernels form padded row offsets with a 24-bit multiply."""
    H = (1 << 24) // 64
    for f, last in ((lib.rattn_fused, 1), (lib.rattn_fused_padded, 1)):
        assert f(A, A, A, A, A, None, 1, 1, H, 64, last, ctypes.c_float(0.125), BF16,
                 None) == INVALID
    # one head less passes the checks and reaches the device query
    st = lib.rattn_fused(A, A, A, A, A, None, 1, 1, H - 1, 64, 1, ctypes.c_float(0.125), BF16,
                         None)
    assert st not in (INVALID, UNSUPPORTED)


def test_repack_argument_checks(lib):
    P2 = ctypes.c_void_p * 1
    src, dst = P2(A), P2(A + 0x1000)
    f = lib.rattn_repack
    assert f(src, dst, 1, A, A, 0, 128, BF16, A + 64, None, None) == OK      # B = 0: nothing
    assert f(src, dst, 0, A, A, 2, 128, BF16, A + 64, None, None) == INVALID  # no tensors
    assert f(src, dst, 4, A, A, 2, 128, BF16, A + 64, None, None) == INVALID  # too many
    assert f(src, dst, 1, A + 1, A, 2, 128, BF16, A + 64, None, None) == INVALID  # keep2 misaligned
    assert f(src, dst, 1, A, A, 2, 128, BF16, A, None, None) == INVALID       # cu_out aliases cu
    assert f(src, P2(A), 1, A, A, 2, 128, BF16, A + 64, None, None) == INVALID  # dst == src
    assert f(src, dst, 1, A, A, 2, 5, F32, A + 64, None, None) == INVALID     # row not 16 B


def test_validate_mode_switch(lib):
    """The debug-validate switch is a process-wide flag: set returns the
    previous setting; no device is needed to flip it."""
    prev = lib.rattn_get_validate()
    try:
        assert lib.rattn_set_validate(1) == prev
        assert lib.rattn_get_validate() == 1
        assert lib.rattn_set_validate(7) == 1      # any nonzero value means on
        assert rv.rattn_get_validate() is True
        assert rv.rattn_set_validate(False) is True
        assert lib.rattn_get_validate() == 0
        # host-side checks still come first in the mode: nothing is read back
        lib.rattn_set_validate(1)
        assert _fwd(lib, D=32) == UNSUPPORTED
        assert _fwd(lib, q=None) == INVALID
    finally:
        lib.rattn_set_validate(prev)
