"""ctypes binding of librattn.so -- argument marshalling only.

Every function has the name of the C entry point it calls and does no compute:
it reads shapes, dtypes, device pointers and the current HIP stream off torch
tensors and passes them through.  All work runs in the library's HIP kernels.
There is no fallback: if librattn.so is missing, or the call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librattn.so")

RATTN_OK = 0
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_lib = None


class RattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load librattn.so (torch is imported first so the HIP runtime is shared)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -c \"import __graft_entry__ as g; g.build()\"` "
            "(or python ragged_variable_length_amd/build.py) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.rattn_init.argtypes = []
    lib.rattn_init.restype = i32
    lib.rattn_status_string.argtypes = [i32]
    lib.rattn_status_string.restype = ctypes.c_char_p
    lib.rattn_version.argtypes = []
    lib.rattn_version.restype = i32
    lib.rattn_pack.argtypes = [P, P, i32, P, i32, i32, i32, i32, P, P, P, P]
    lib.rattn_pack.restype = i32
    lib.rattn_forward.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f32, i32, P]
    lib.rattn_forward.restype = i32
    lib.rattn_unpack.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
    lib.rattn_unpack.restype = i32
    lib.rattn_fused.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, f32, i32, P]
    lib.rattn_fused.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().rattn_status_string(int(status)).decode()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _check(fn: str, status: int) -> None:
    if status != RATTN_OK:
        raise RattnError(fn, status)


def rattn_init() -> None:
    _check("rattn_init", load().rattn_init())


def rattn_pack(srcs, dsts, keep: torch.Tensor, cu_seqlens: torch.Tensor,
               max_seqlen: torch.Tensor | None = None, total: torch.Tensor | None = None,
               stream=None) -> None:
    """Pack 1-3 padded [B, N, ...] tensors into flat [T, ...] tensors (C: rattn_pack)."""
    srcs, dsts = list(srcs), list(dsts)
    if not 1 <= len(srcs) == len(dsts) <= 3:
        raise ValueError("rattn_pack takes 1-3 (src, dst) pairs")
    B, N = keep.shape
    dt = srcs[0].dtype
    row = srcs[0].shape[2:]
    for s, d in zip(srcs, dsts):
        if s.dtype != dt or d.dtype != dt or s.shape[:2] != (B, N) or s.shape[2:] != row \
                or d.shape[1:] != row:
            raise ValueError("rattn_pack: inconsistent shapes or dtypes")
    row_elems = 1
    for x in row:
        row_elems *= int(x)
    n = len(srcs)
    src_arr = (ctypes.c_void_p * n)(*[_dev(s, "src") for s in srcs])
    dst_arr = (ctypes.c_void_p * n)(*[_dev(d, "dst") for d in dsts])
    st = load().rattn_pack(src_arr, dst_arr, n, _dev(keep, "keep"), B, N, row_elems,
                           _DTYPE_CODE[dt], _dev(cu_seqlens, "cu_seqlens"),
                           _opt(max_seqlen, "max_seqlen"), _opt(total, "total"), _stream(stream))
    _check("rattn_pack", st)


def rattn_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                  cu_seqlens: torch.Tensor, max_seqlen: int, scale: float,
                  stream=None) -> None:
    """Ragged bidirectional attention on [T, H, 64] buffers (C: rattn_forward)."""
    if not (q.shape == k.shape == v.shape == o.shape) or q.dim() != 3:
        raise ValueError("rattn_forward: q, k, v, o must share one [T, H, head_dim] shape")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise ValueError("rattn_forward: dtype mismatch")
    _, H, D = q.shape
    B = cu_seqlens.shape[0] - 1
    st = load().rattn_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                              _dev(cu_seqlens, "cu_seqlens"), B, int(max_seqlen), H, D,
                              float(scale), _DTYPE_CODE[q.dtype], _stream(stream))
    _check("rattn_forward", st)


def rattn_unpack(src: torch.Tensor, keep: torch.Tensor, cu_seqlens: torch.Tensor,
                 dst_padded: torch.Tensor | None = None, cls: torch.Tensor | None = None,
                 stream=None) -> None:
    """Scatter flat [T, ...] rows back to [B, N, ...] and/or CLS rows [B, ...]
    (C: rattn_unpack)."""
    B, N = keep.shape
    row_elems = 1
    for x in src.shape[1:]:
        row_elems *= int(x)
    for t, name in ((dst_padded, "dst_padded"), (cls, "cls")):
        if t is not None and t.dtype != src.dtype:
            raise ValueError(f"rattn_unpack: {name} dtype mismatch")
    if dst_padded is not None and tuple(dst_padded.shape) != (B, N) + tuple(src.shape[1:]):
        raise ValueError("rattn_unpack: dst_padded must be [B, N, *row]")
    if cls is not None and tuple(cls.shape) != (B,) + tuple(src.shape[1:]):
        raise ValueError("rattn_unpack: cls must be [B, *row]")
    st = load().rattn_unpack(_dev(src, "src"), _opt(dst_padded, "dst_padded"), _opt(cls, "cls"),
                             _dev(keep, "keep"), _dev(cu_seqlens, "cu_seqlens"), B, N, row_elems,
                             _DTYPE_CODE[src.dtype], _stream(stream))
    _check("rattn_unpack", st)


def rattn_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: torch.Tensor,
                scale: float, out_padded: torch.Tensor | None = None,
                cls: torch.Tensor | None = None, max_seqlen: int | None = None,
                stream=None) -> None:
    """Pack, attend and unpack in one launch, padded [B, N, H, 64] in and out
    (C: rattn_fused)."""
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("rattn_fused: q, k, v must share one [B, N, H, head_dim] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("rattn_fused: dtype mismatch")
    B, N, H, D = q.shape
    if tuple(keep.shape) != (B, N):
        raise ValueError("rattn_fused: keep must be [B, N]")
    if out_padded is not None and (out_padded.shape != q.shape or out_padded.dtype != q.dtype):
        raise ValueError("rattn_fused: out_padded must match q")
    if cls is not None and (tuple(cls.shape) != (B, H, D) or cls.dtype != q.dtype):
        raise ValueError("rattn_fused: cls must be [B, H, head_dim] of q's dtype")
    ms = N if max_seqlen is None else int(max_seqlen)
    st = load().rattn_fused(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(keep, "keep"),
                            _opt(out_padded, "out_padded"), _opt(cls, "cls"), B, N, H, D, ms,
                            float(scale), _DTYPE_CODE[q.dtype], _stream(stream))
    _check("rattn_fused", st)
