"""CPU oracle for the token-pruned ViT pack -> attend -> unpack path.

TEST INFRASTRUCTURE ONLY.  `tests/`, the smoke check in `__graft_entry__` and
the CPU-baseline leg of `bench.py` may import it; the product package never
does.  The arithmetic lives in `oracle.c` (plain C, fp64, per-sequence loops);
this module builds it with gcc, loads it with ctypes and converts arrays.  It
shares nothing with the HIP library.

Parity pins: every function here is pinned by `tests/test_oracle.py` (library
SDPA per image in float64, brute-force padded masked attention, closed forms,
invariants, hand-derived fixtures in `tests/golden/`).  Nothing is parity
unpinned except the pages' logit-level accuracy claims, which need trained
weights and ImageNet and are outside this oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc -O2 (no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # another build of oracle.c (the sanitizer test runs the pins on one)
    other = os.environ.get("RATTN_ORACLE_LIB")
    if other:
        _lib = _configure(ctypes.CDLL(other))
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _configure(lib):
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_scan.argtypes = [P, i32, i32, P, P, P]
    lib.oracle_scan.restype = i32
    lib.oracle_pack.argtypes = [P, P, P, i32, i32, i64]
    lib.oracle_pack.restype = i64
    lib.oracle_attention.argtypes = [P, P, P, P, i32, i32, i32, dbl, P, i64, P, P]
    lib.oracle_attention.restype = i32
    lib.oracle_unpack.argtypes = [P, P, P, P, P, i32, i32, i64]
    lib.oracle_unpack.restype = i32
    lib.oracle_repack.argtypes = [P, P, P, P, i32, i64, P]
    lib.oracle_repack.restype = i64
    return lib


class use_library:
    """Context manager swapping in another build of oracle.c (used only by the
    mutation test, which checks that the pins catch planted slips)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    """Any array/tensor -> contiguous numpy array viewed as raw bytes."""
    a = _np(a)
    return np.ascontiguousarray(a).view(np.uint8)


def _np(a) -> np.ndarray:
    if isinstance(a, np.ndarray):
        return a
    # torch tensor (CPU); bfloat16 has no numpy dtype, so move its bits as int16
    import torch
    t = a.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy()


# --------------------------------------------------------------------------
# exact widening of storage types to float64 (no rounding is possible here)
# --------------------------------------------------------------------------
def widen(a, dtype: str) -> np.ndarray:
    """Storage bits of an f32/f16/bf16 array -> float64, exactly."""
    x = np.ascontiguousarray(_np(a))
    if dtype == "f32":
        return x.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = x.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# the four steps
# --------------------------------------------------------------------------
def scan(keep):
    """-> (cu int32 [B+1], max_seqlen, total)."""
    k = np.ascontiguousarray(_u8(keep))
    B, N = (k.shape[0], k.shape[1]) if k.ndim == 2 else (1, k.size)
    cu = np.zeros(B + 1, dtype=np.int32)
    mx = np.zeros(1, dtype=np.int32)
    tot = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_scan(_ptr(k), B, N, _ptr(cu), _ptr(mx), _ptr(tot))
    if rc != 0:
        raise ValueError("oracle_scan: bad argument")
    return cu, int(mx[0]), int(tot[0])


def pack(src, keep) -> np.ndarray:
    """Padded [B, N, ...] -> flat [T, ...] with the same dtype bits (uint8 view
    of each row is copied)."""
    s = np.ascontiguousarray(_np(src))
    k = np.ascontiguousarray(_u8(keep))
    B, N = k.shape
    row_bytes = s.nbytes // (B * N) if B * N else 0
    T = int((k != 0).sum())
    out = _poisoned((T,) + s.shape[2:], s.dtype)
    sb = s.view(np.uint8).reshape(-1)
    ob = out.view(np.uint8).reshape(-1) if out.size else np.zeros(1, np.uint8)
    n = _load().oracle_pack(_ptr(sb), _ptr(ob), _ptr(k), B, N, row_bytes)
    assert n == T
    return out


def attention(q, k, v, cu, scale: float, rows=None, want_absw: bool = False):
    """q, k, v: float64 [T, H, D] (already widened).  Returns o (float64) for
    all rows or for the listed flat rows; with want_absw also sum p|v| / sum p."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    B = cu.shape[0] - 1
    T, H, D = q.shape
    assert k.shape == q.shape == v.shape and T >= cu[-1]
    rr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = T if rr is None else rr.shape[0]
    o = _poisoned((n, H, D), np.float64)
    a = _poisoned((n, H, D), np.float64) if want_absw else None
    if n:
        rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), B, H, D,
                                      float(scale), _ptr(rr), n if rr is not None else 0,
                                      _ptr(o), _ptr(a))
        if rc != 0:
            raise ValueError("oracle_attention: bad argument")
    return (o, a) if want_absw else o


def _poisoned(shape, dtype) -> np.ndarray:
    a = np.empty(shape, dtype=dtype)
    a.view(np.uint8).reshape(-1)[:] = 0xA5
    return a


def unpack(src, keep, cu, want_padded: bool = True, want_cls: bool = True):
    """Flat [T, ...] -> (padded [B, N, ...] with zero pruned rows, cls [B, ...])."""
    s = np.ascontiguousarray(_np(src))
    k = np.ascontiguousarray(_u8(keep))
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    B, N = k.shape
    row_shape = s.shape[1:]
    row_bytes = int(np.prod(row_shape)) * s.dtype.itemsize
    # outputs start as poison bytes: the C code must write every byte itself
    dst = _poisoned((B, N) + row_shape, s.dtype) if want_padded else None
    cls = _poisoned((B,) + row_shape, s.dtype) if want_cls else None
    sb = s.view(np.uint8).reshape(-1) if s.size else np.zeros(1, np.uint8)
    rc = _load().oracle_unpack(_ptr(sb), _ptr(dst), _ptr(cls), _ptr(k), _ptr(cu),
                               B, N, row_bytes)
    if rc != 0:
        raise ValueError("oracle_unpack: cu_seqlens disagrees with the keep mask")
    return dst, cls


def repack(src, keep2, cu):
    """Flat [T, ...] rows of images cu, second keep flag per row [T] ->
    (flat [T2, ...] of the rows kept again, cu2 int32 [B+1])."""
    s = np.ascontiguousarray(_np(src))
    k2 = np.ascontiguousarray(_u8(keep2)).reshape(-1)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    B = cu.shape[0] - 1
    T = int(cu[-1])
    assert s.shape[0] >= T and k2.shape[0] >= T
    row_shape = s.shape[1:]
    row_bytes = int(np.prod(row_shape)) * s.dtype.itemsize
    T2 = int((k2[:T] != 0).sum())
    # room for every row, so that the C code can never write past the buffer
    out = _poisoned((max(T, 1),) + row_shape, s.dtype)
    cu2 = np.full(B + 1, -1, dtype=np.int32)
    sb = s.view(np.uint8).reshape(-1) if s.size else np.zeros(1, np.uint8)
    ob = out.view(np.uint8).reshape(-1)
    n = _load().oracle_repack(_ptr(sb), _ptr(ob), _ptr(k2), _ptr(cu), B, row_bytes, _ptr(cu2))
    if n < 0:
        raise ValueError("oracle_repack: cu_seqlens decreases")
    assert n == T2, "oracle_repack wrote an unexpected number of rows"
    return out[:n].copy(), cu2


def pipeline(w, rows=None, want_absw: bool = False):
    """Whole path on a `workloads.Workload`: scan, pack q/k/v, attend (fp64).
    Returns a dict with cu, max_seqlen, total, packed q/k/v (storage bits),
    o64 (float64) and, with want_absw, absw."""
    cu, mx, tot = scan(w.keep)
    pq, pk, pv = (pack(t, w.keep) for t in (w.q, w.k, w.v))
    T = pq.shape[0]
    shp = (T, w.H, w.D)
    q64, k64, v64 = (widen(t, w.dtype).reshape(shp) for t in (pq, pk, pv))
    res = attention(q64, k64, v64, cu, w.scale, rows=rows, want_absw=want_absw)
    out = {"cu": cu, "max_seqlen": mx, "total": tot, "q": pq, "k": pk, "v": pv}
    if want_absw:
        out["o64"], out["absw"] = res
    else:
        out["o64"] = res
    return out
