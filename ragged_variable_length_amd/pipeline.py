"""Device buffers and prepared calls for repeated pack -> attend -> unpack.

Pages on "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
(arXiv 2604.15408), radpulse.milrad-way.com write-up, section on the
integrated packing pipeline: cu_seqlens, pack, attend, CLS extract.

Buffers are sized from (B, N, H) once, with capacity B*N rows for the flat
tensors, so no call needs the kept-token count on the host: there is no
device-to-host copy and no allocation inside `run`.  Every step is one of the
three C entry points; nothing here computes.

`FusedPlan` is the serving form of rattn_fused: its arguments are checked and
marshalled once, so each `run()` is one extension call and one launch.  The
same write-up (sections on FlashAttention-2's dispatch ceiling and on the
Triton kernel) puts most of a small call's cost in per-call validation and
binding crossings rather than in the kernel; a plan removes them from the
repeated path.
"""
from __future__ import annotations

import torch

from . import _binding
from ._binding import RattnError, rattn_forward, rattn_pack, rattn_unpack


class RaggedPipeline:
    def __init__(self, B: int, N: int, H: int, dtype: torch.dtype, device="cuda",
                 head_dim: int = 64, want_padded: bool = True, want_cls: bool = True):
        self.B, self.N, self.H, self.D = B, N, H, head_dim
        self.dtype = dtype
        dev = torch.device(device)
        cap = max(1, B * N)
        shape = (cap, H, head_dim)
        self.pq = torch.empty(shape, dtype=dtype, device=dev)
        self.pk = torch.empty(shape, dtype=dtype, device=dev)
        self.pv = torch.empty(shape, dtype=dtype, device=dev)
        self.po = torch.empty(shape, dtype=dtype, device=dev)
        self.cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.max_seqlen_dev = torch.empty(1, dtype=torch.int32, device=dev)
        self.total_dev = torch.empty(1, dtype=torch.int32, device=dev)
        self.out = (torch.empty((B, N, H, head_dim), dtype=dtype, device=dev)
                    if want_padded else None)
        self.cls = torch.empty((B, H, head_dim), dtype=dtype, device=dev) if want_cls else None

    def pack(self, q, k, v, keep, stream=None):
        rattn_pack((q, k, v), (self.pq, self.pk, self.pv), keep, self.cu,
                   self.max_seqlen_dev, self.total_dev, stream=stream)

    def attend(self, scale: float, max_seqlen: int | None = None, stream=None):
        ms = self.N if max_seqlen is None else max_seqlen
        rattn_forward(self.pq, self.pk, self.pv, self.po, self.cu, ms, scale, stream=stream)

    def unpack(self, keep, stream=None):
        rattn_unpack(self.po, keep, self.cu, dst_padded=self.out, cls=self.cls, stream=stream)

    def run(self, q, k, v, keep, scale: float, max_seqlen: int | None = None, stream=None):
        """q, k, v: padded [B, N, H, 64] device tensors; keep: uint8 [B, N]."""
        self.pack(q, k, v, keep, stream)
        self.attend(scale, max_seqlen, stream)
        self.unpack(keep, stream)
        return self.out, self.cls


class FusedPlan:
    """rattn_fused on fixed buffers: checked once, launched by `run()`.

    q, k, v: padded [B, N, H, 64] device tensors; keep: uint8 [B, N]; at least
    one of out_padded ([B, N, H, 64]) and cls ([B, H, 64]).  The stream is
    fixed when the plan is made (None = torch's current stream then).  The
    plan holds references to the tensors; their contents may change between
    runs, their storage may not.

    With `pad_len` the plan runs the dense comparator rattn_fused_padded
    instead (every image processed at pad_len tokens; same outputs).
    """

    def __init__(self, q, k, v, keep, scale: float, out_padded=None, cls=None,
                 max_seqlen: int | None = None, stream=None, pad_len: int | None = None):
        bound = pad_len if pad_len is not None else max_seqlen
        self._args = _binding.fused_args(q, k, v, keep, scale, out_padded, cls, bound, stream)
        self._tensors = (q, k, v, keep, out_padded, cls)
        self._name = "rattn_fused" if pad_len is None else "rattn_fused_padded"
        self._fn = _binding.ext().fused if pad_len is None else _binding.ext().fused_padded

    def run(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            raise RattnError(self._name, st)
