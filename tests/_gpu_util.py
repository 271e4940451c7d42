"""Helpers for the GPU parity tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from ragged_variable_length_amd import RaggedPipeline

# Attention tolerances, max |gpu - oracle| over kept rows (unit-normal inputs).
FLAT_TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 1e-2}
# Unit round-off of the 16-bit types: the kernel rounds the probabilities and
# the output once each, so the rounding error of an element is at most
# u * (sum_j p_j |v_j| / sum_j p_j + |o|); the bound below allows twice that.
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
CANARY = 0x5A


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t) -> np.ndarray:
    """Storage bits of a tensor or array as an integer numpy array (CPU copy)."""
    if isinstance(t, np.ndarray):
        a = np.ascontiguousarray(t)
        return a.view({1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[a.dtype.itemsize])
    t = t.detach().cpu().contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy()
    if t.element_size() == 4:
        return t.view(torch.int32).numpy()
    return t.view(torch.uint8).numpy()


def run_hip(w, max_seqlen=None, poison_pruned=False, canary=True, stream=None):
    """Run pack -> forward -> unpack through the C ABI; return CPU copies."""
    dev = torch.device("cuda")
    q, k, v = (t.clone() for t in (w.q, w.k, w.v))
    if poison_pruned:
        pruned = w.keep == 0
        for t in (q, k, v):
            t[pruned] = float("nan")
    q, k, v = (t.to(dev) for t in (q, k, v))
    keep = w.keep.to(dev)
    pipe = RaggedPipeline(w.B, w.N, w.H, q.dtype, device=dev)
    if canary:
        for t in (pipe.pq, pipe.pk, pipe.pv, pipe.po):
            t.view(torch.uint8).fill_(CANARY)
    pipe.cu.fill_(-7)
    pipe.run(q, k, v, keep, w.scale, max_seqlen=max_seqlen, stream=stream)
    torch.cuda.synchronize()
    return {
        "cu": pipe.cu.cpu().numpy(),
        "max_seqlen": int(pipe.max_seqlen_dev.item()),
        "total": int(pipe.total_dev.item()),
        "pq": pipe.pq.cpu(), "pk": pipe.pk.cpu(), "pv": pipe.pv.cpu(), "po": pipe.po.cpu(),
        "out": pipe.out.cpu(), "cls": pipe.cls.cpu(),
    }


def check_indexing(w, got, ref):
    """cu_seqlens, max, total, packed q/k/v: bit-exact; capacity rows untouched;
    unpack / CLS bit-exact against the oracle's unpack of the GPU's own o."""
    T = ref["total"]
    assert got["cu"].tolist() == ref["cu"].tolist(), "cu_seqlens"
    assert got["max_seqlen"] == ref["max_seqlen"], "max_seqlen"
    assert got["total"] == T, "total"
    for name, key in (("q", "pq"), ("k", "pk"), ("v", "pv")):
        g = bits(got[key])
        assert np.array_equal(g[:T], ref[name].view(g.dtype)), f"packed {name}"
        assert np.all(got[key].view(torch.uint8).numpy()[T:] == CANARY), f"{name} rows past T written"
    assert np.all(got["po"].view(torch.uint8).numpy()[T:] == CANARY), "o rows past T written"
    po = got["po"][:T]
    dst, cls = oracle.unpack(po, w.keep, ref["cu"])
    assert np.array_equal(bits(got["out"]), dst.view(bits(got["out"]).dtype)), "unpack"
    assert np.array_equal(bits(got["cls"]), cls.view(bits(got["cls"]).dtype)), "cls"


def attention_error(w, got, ref_o, ref_absw, rows=None):
    """Returns (max abs error, max of error / derived bound) over the rows."""
    T = got["total"]
    o = oracle.widen(got["po"][:T], w.dtype).reshape(T, w.H, w.D)
    if rows is not None:
        o = o[rows]
    assert np.all(np.isfinite(o)), "non-finite attention output"
    err = np.abs(o - ref_o)
    bound = 2.0 * UNIT_ROUNDOFF[w.dtype] * (np.abs(ref_o) + ref_absw) + FLAT_TOL[w.dtype]
    return float(err.max()), float((err / bound).max())


def sample_rows(cu: np.ndarray, n: int, seed: int = 0) -> np.ndarray:
    """Flat rows to check one by one: first and last row of every image plus a
    seeded uniform sample, sorted and unique."""
    rng = np.random.default_rng(seed)
    T = int(cu[-1])
    firsts = cu[:-1][np.diff(cu) > 0]
    lasts = cu[1:][np.diff(cu) > 0] - 1
    extra = rng.choice(T, size=min(n, T), replace=False) if T else np.zeros(0, np.int64)
    return np.unique(np.concatenate([firsts, lasts, extra]).astype(np.int64))
