"""The two float32 attention cores against the CPU oracle, on MI355X.

Float32 batches of at most 64 heads split each 16-row query tile's key chunks
over the workgroup's four wavefronts and merge their partial softmax states;
larger batches give each wavefront 16 query rows and all key chunks.  The rule
reads the head count only, so every entry point takes the same core for the
same batch.  Checked for 64 heads (split) and 65 heads (one wavefront per row
block), on lengths at every tile and chunk edge: the three calls against the
oracle (indexing bit-exact, attention within 1e-4), rattn_fused against the
oracle and bitwise equal to the three calls, the padded comparator and the
CLS-only mode bitwise equal to rattn_fused, and the max_seqlen bound (exact,
N, 4N) leaving the bits unchanged.  Long sequences (577 and 2048 positions)
give every wavefront of the split core several chunks.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import (FLAT_TOL, attention_error, bits, check_indexing, check_padded,
                             run_hip, say)

pytestmark = pytest.mark.gpu
POISON = 0xA5
EDGE_LENGTHS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 300]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def _keep(lengths, N, seed):
    g = torch.Generator().manual_seed(seed)
    keep = torch.zeros((len(lengths), N), dtype=torch.uint8)
    for b, L in enumerate(lengths):
        keep[b, torch.randperm(N, generator=g)[:L]] = 1
    return keep


def _fused(w, pad=None, want_out=True, max_seqlen=None):
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
    out = torch.empty_like(q) if want_out else None
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev)
    for t in (out, cls):
        if t is not None:
            t.view(torch.uint8).fill_(POISON)
    if pad is None:
        rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out, cls=cls, max_seqlen=max_seqlen)
    else:
        rv.rattn_fused_padded(q, k, v, keep, w.scale, pad, out_padded=out, cls=cls)
    torch.cuda.synchronize()
    return (None if out is None else out.cpu()), cls.cpu()


def _all_paths(w):
    ref = oracle.pipeline(w, want_absw=True)
    got = run_hip(w)
    check_indexing(w, got, ref)
    err, ratio = attention_error(w, got, ref["o64"], ref["absw"])
    say(f"{w.name}: three calls max|err|={err:.3e} err/bound={ratio:.3f}")
    assert err <= FLAT_TOL["f32"] and ratio <= 1.0, (err, ratio)
    out, cls = _fused(w)
    check_padded(w, out, cls, ref["o64"], ref["absw"])
    assert np.array_equal(bits(out), bits(got["out"])), "fused output differs from three calls"
    assert np.array_equal(bits(cls), bits(got["cls"])), "fused CLS differs from three calls"
    for pad in (max(w.kept_counts), w.N):
        po, pc = _fused(w, pad=pad)
        assert np.array_equal(bits(po), bits(out)), f"padded to {pad}: output"
        assert np.array_equal(bits(pc), bits(cls)), f"padded to {pad}: CLS"
    _, cc = _fused(w, want_out=False)
    assert np.array_equal(bits(cc), bits(cls)), "CLS-only mode"
    return got, out


@pytest.mark.parametrize("B,H", [(16, 4), (13, 5)], ids=["64_heads_split", "65_heads_rows"])
def test_f32_cores_at_the_head_threshold(B, H):
    lengths = (EDGE_LENGTHS * 2)[:B]
    w = workloads.custom(B, 300, H, "f32", keep=_keep(lengths, 300, seed=80 + H), seed=81 + H,
                         name=f"f32_cores_{B}x{H}")
    got, out = _all_paths(w)
    # the bound selects the tile groups per head, never the arithmetic
    for bound in (max(w.kept_counts), 4 * w.N):
        again = run_hip(w, max_seqlen=bound)
        assert np.array_equal(bits(again["po"]), bits(got["po"])), f"max_seqlen {bound}"
        fo, _ = _fused(w, max_seqlen=bound)
        assert np.array_equal(bits(fo), bits(out)), f"fused max_seqlen {bound}"


@pytest.mark.parametrize("N", [577, 2048])
def test_f32_split_core_long_sequences(N):
    keep = torch.ones((2, N), dtype=torch.uint8)
    keep[1, N // 3:] = 0
    _all_paths(workloads.custom(2, N, 2, "f32", keep=keep, seed=82, name=f"f32_long_{N}"))
