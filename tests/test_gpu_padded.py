"""The dense comparator rattn_fused_padded on MI355X: every image processed at
a padded length (the longest survivor, or N), padding keys masked and padding
query rows computed and discarded.  Masked keys contribute exactly zero, so
its outputs must be bit-for-bit those of rattn_fused, whose parity with the
oracle is checked in test_gpu_fused.py; only the amount of work differs.
"""
import numpy as np
import pytest
import torch

import workloads
from tests._gpu_util import bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def _run(w, pad=None, want_out=True):
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
    out = torch.empty_like(q) if want_out else None
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev)
    for t in (out, cls):
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)
    if pad is None:
        rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out, cls=cls)
    else:
        rv.rattn_fused_padded(q, k, v, keep, w.scale, pad, out_padded=out, cls=cls)
    torch.cuda.synchronize()
    return (None if out is None else bits(out.cpu())), bits(cls.cpu())


def _same_bits(w):
    ref = _run(w)
    for pad in (max(max(w.kept_counts), 1), w.N):
        say(f"{w.name}: padded to {pad} (ragged max {max(w.kept_counts)}, N {w.N})")
        got = _run(w, pad)
        assert np.array_equal(got[0], ref[0]), "padded output differs from ragged"
        assert np.array_equal(got[1], ref[1]), "padded CLS differs from ragged"


def test_padded_deit_s_fp16():
    _same_bits(workloads.deit_s())


@pytest.mark.parametrize("B,p", [(1, 0.8), (4, 0.5), (2, 0.0)])
def test_padded_deit_b_sweep_bf16(B, p):
    _same_bits(workloads.deit_b_sweep(B, p))


def test_padded_deit_b_384_bf16():
    _same_bits(workloads.deit_b_384())


def test_padded_large_batch_bf16():
    _same_bits(workloads.large_batch(B=128))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_padded_ragged_tails(dtype):
    g = torch.Generator().manual_seed(19)
    lengths = [1, 0, 16, 17, 63, 64, 65, 129, 200]
    keep = torch.zeros((len(lengths), 200), dtype=torch.uint8)
    for b, L in enumerate(lengths):
        keep[b, torch.randperm(200, generator=g)[:L]] = 1
    _same_bits(workloads.custom(len(lengths), 200, 2, dtype, keep=keep, seed=19,
                                name=f"padded_tails_{dtype}"))


def test_padded_cls_only():
    w = workloads.deit_b_sweep(4, 0.8)
    say("padded comparator, CLS rows only")
    _, ref = _run(w, want_out=False)
    _, got = _run(w, pad=w.N, want_out=False)
    assert np.array_equal(got, ref)
