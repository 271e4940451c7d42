"""Python binding of librattn.so -- argument marshalling only.

Every function has the name of the C entry point it calls and does no compute:
it reads shapes, dtypes, device pointers and the current HIP stream off torch
tensors and passes them through the CPython extension `_rattn` (one
METH_FASTCALL function per entry point, linked against librattn.so).  All work
runs in the library's HIP kernels.  There is no fallback: if librattn.so or the
extension is missing, or a call fails, an exception is raised.

`load()` returns librattn.so itself through ctypes, with prototypes, for
callers that want the raw C ABI.
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
_ext_mod = None
_NOT_BUILT = ("is not built: run `python -c \"import __graft_entry__ as g; g.build()\"` "
              "(or python ragged_variable_length_amd/build.py) first")


class RattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """librattn.so through ctypes, with the C prototypes set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} {_NOT_BUILT}")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.rattn_init.argtypes = []
    lib.rattn_init.restype = i32
    lib.rattn_status_string.argtypes = [i32]
    lib.rattn_status_string.restype = ctypes.c_char_p
    lib.rattn_version.argtypes = []
    lib.rattn_version.restype = i32
    lib.rattn_set_validate.argtypes = [i32]
    lib.rattn_set_validate.restype = i32
    lib.rattn_get_validate.argtypes = []
    lib.rattn_get_validate.restype = i32
    lib.rattn_pack.argtypes = [P, P, i32, P, i32, i32, i32, i32, P, P, P, P]
    lib.rattn_pack.restype = i32
    lib.rattn_forward.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f32, i32, P]
    lib.rattn_forward.restype = i32
    lib.rattn_unpack.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
    lib.rattn_unpack.restype = i32
    lib.rattn_fused.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, f32, i32, P]
    lib.rattn_fused.restype = i32
    lib.rattn_fused_padded.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, f32, i32, P]
    lib.rattn_fused_padded.restype = i32
    lib.rattn_repack.argtypes = [P, P, i32, P, P, i32, i32, i32, P, P, P]
    lib.rattn_repack.restype = i32
    _lib = lib
    return lib


def ext():
    """The `_rattn` extension module the entry-point wrappers call."""
    global _ext_mod
    if _ext_mod is not None:
        return _ext_mod
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} {_NOT_BUILT}")
    try:
        from . import _rattn
    except ImportError as e:
        raise RuntimeError(f"the _rattn extension {_NOT_BUILT} ({e})") from e
    _ext_mod = _rattn
    return _ext_mod


def status_string(status: int) -> str:
    return ext().status_string(int(status))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, t: torch.Tensor) -> int:
    """HIP stream handle: `stream` if given, else torch's current stream on t's
    device."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.get_device())
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _typed(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    """_dev for the index and mask arguments, whose element type the kernels
    assume (int32 counts and offsets, uint8 flags)."""
    if isinstance(t, torch.Tensor) and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return _dev(t, name)


def _opt_typed(t, name, dtype):
    return None if t is None else _typed(t, name, dtype)


def _check(fn: str, status: int) -> None:
    if status != RATTN_OK:
        raise RattnError(fn, status)


def rattn_init() -> None:
    _check("rattn_init", ext().init())


def rattn_set_validate(on: bool) -> bool:
    """Switch the library's debug-validate mode on or off for the process;
    returns the previous setting (C: rattn_set_validate)."""
    return bool(ext().set_validate(1 if on else 0))


def rattn_get_validate() -> bool:
    """Whether debug-validate mode is on (C: rattn_get_validate)."""
    return bool(ext().get_validate())


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
    st = ext().pack([_dev(s, "src") for s in srcs], [_dev(d, "dst") for d in dsts],
                    _typed(keep, "keep", torch.uint8), B, N, row_elems, _DTYPE_CODE[dt],
                    _typed(cu_seqlens, "cu_seqlens", torch.int32), _opt_typed(max_seqlen, "max_seqlen", torch.int32),
                    _opt_typed(total, "total", torch.int32), _stream(stream, keep))
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
    st = ext().forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                       _typed(cu_seqlens, "cu_seqlens", torch.int32), B, int(max_seqlen), H, D, float(scale),
                       _DTYPE_CODE[q.dtype], _stream(stream, q))
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
    st = ext().unpack(_dev(src, "src"), _opt(dst_padded, "dst_padded"), _opt(cls, "cls"),
                      _typed(keep, "keep", torch.uint8), _typed(cu_seqlens, "cu_seqlens", torch.int32), B, N, row_elems,
                      _DTYPE_CODE[src.dtype], _stream(stream, src))
    _check("rattn_unpack", st)


def fused_args(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: torch.Tensor,
               scale: float, out_padded: torch.Tensor | None = None,
               cls: torch.Tensor | None = None, max_seqlen: int | None = None,
               stream=None) -> tuple:
    """Checked, marshalled argument tuple of one rattn_fused call."""
    qs = q.shape
    if len(qs) != 4 or k.shape != qs or v.shape != qs:
        raise ValueError("rattn_fused: q, k, v must share one [B, N, H, head_dim] shape")
    dt = q.dtype
    if k.dtype != dt or v.dtype != dt:
        raise ValueError("rattn_fused: dtype mismatch")
    B, N, H, D = qs
    if tuple(keep.shape) != (B, N):
        raise ValueError("rattn_fused: keep must be [B, N]")
    if out_padded is not None and (out_padded.shape != qs or out_padded.dtype != dt):
        raise ValueError("rattn_fused: out_padded must match q")
    if cls is not None and (tuple(cls.shape) != (B, H, D) or cls.dtype != dt):
        raise ValueError("rattn_fused: cls must be [B, H, head_dim] of q's dtype")
    ms = N if max_seqlen is None else int(max_seqlen)
    return (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _typed(keep, "keep", torch.uint8),
            _opt(out_padded, "out_padded"), _opt(cls, "cls"), B, N, H, D, ms, float(scale),
            _DTYPE_CODE[dt], _stream(stream, q))


def rattn_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: torch.Tensor,
                scale: float, out_padded: torch.Tensor | None = None,
                cls: torch.Tensor | None = None, max_seqlen: int | None = None,
                stream=None) -> None:
    """Pack, attend and unpack in one launch, padded [B, N, H, 64] in and out
    (C: rattn_fused)."""
    st = ext().fused(*fused_args(q, k, v, keep, scale, out_padded, cls, max_seqlen, stream))
    _check("rattn_fused", st)


def rattn_fused_padded(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: torch.Tensor,
                       scale: float, pad_len: int, out_padded: torch.Tensor | None = None,
                       cls: torch.Tensor | None = None, stream=None) -> None:
    """The dense comparator of rattn_fused: every image processed at pad_len
    tokens, padding masked; same outputs (C: rattn_fused_padded)."""
    args = fused_args(q, k, v, keep, scale, out_padded, cls, int(pad_len), stream)
    st = ext().fused_padded(*args)
    _check("rattn_fused_padded", st)


def rattn_repack(srcs, dsts, keep2: torch.Tensor, cu_seqlens: torch.Tensor,
                 cu_seqlens_out: torch.Tensor, total: torch.Tensor | None = None,
                 stream=None) -> None:
    """Compact 1-3 flat [T, ...] buffers under a second keep flag per row into
    flat [T2, ...] buffers, writing the new cu_seqlens (C: rattn_repack)."""
    srcs, dsts = list(srcs), list(dsts)
    if not 1 <= len(srcs) == len(dsts) <= 3:
        raise ValueError("rattn_repack takes 1-3 (src, dst) pairs")
    dt = srcs[0].dtype
    row = srcs[0].shape[1:]
    for s_, d_ in zip(srcs, dsts):
        if s_.dtype != dt or d_.dtype != dt or s_.shape[1:] != row or d_.shape[1:] != row:
            raise ValueError("rattn_repack: inconsistent shapes or dtypes")
    row_elems = 1
    for x in row:
        row_elems *= int(x)
    B = cu_seqlens.shape[0] - 1
    if tuple(cu_seqlens_out.shape) != (B + 1,):
        raise ValueError("rattn_repack: cu_seqlens_out must be [B+1]")
    st = ext().repack([_dev(s_, "src") for s_ in srcs], [_dev(d_, "dst") for d_ in dsts],
                      _typed(keep2, "keep2", torch.uint8), _typed(cu_seqlens, "cu_seqlens", torch.int32), B, row_elems,
                      _DTYPE_CODE[dt], _typed(cu_seqlens_out, "cu_seqlens_out", torch.int32),
                      _opt_typed(total, "total", torch.int32), _stream(stream, keep2))
    _check("rattn_repack", st)
