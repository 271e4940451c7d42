"""The dense comparator rattn_fused_padded on MI355X: every image processed at
a padded length (the longest survivor, or N), padding keys masked and padding
query rows computed and discarded.

Each padded run is checked against the CPU oracle element by element (kept
rows within the tolerances of `_gpu_util`, pruned rows all-zero bytes, CLS
rows the output rows (b, 0)).  Masked keys contribute exactly zero and a row's
softmax reference depends on its own scores only, so the outputs must also be
bit for bit those of rattn_fused; only the amount of work differs.  Where the
padded length and the ragged bound fall on different sides of 256, the two
runs use different tile shapes (64-row and 128-row tiles), which the bitwise
check then compares as well.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import (bits, check_padded, check_rows, keep_length_range,
                             late_outlier_keys, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def _run(w, pad=None, want_out=True, bound=None):
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
    out = torch.empty_like(q) if want_out else None
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev)
    for t in (out, cls):
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)
    if pad is None:
        rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out, cls=cls, max_seqlen=bound)
    else:
        rv.rattn_fused_padded(q, k, v, keep, w.scale, pad, out_padded=out, cls=cls)
    torch.cuda.synchronize()
    return (None if out is None else out.cpu()), cls.cpu()


def _oracle_ref(w, rows):
    if rows is None:
        ref = oracle.pipeline(w, want_absw=True)
        return ref["o64"], ref["absw"]
    cu, _, T = oracle.scan(w.keep)
    packed = (oracle.widen(oracle.pack(t, w.keep), w.dtype).reshape(T, w.H, w.D)
              for t in (w.q, w.k, w.v))
    return oracle.attention(*packed, cu, w.scale, rows=rows, want_absw=True)


def _against_oracle_and_ragged(w, flat=True, rows=None, pads=None):
    """Each padded run against the oracle, and bitwise against rattn_fused."""
    o64, absw = _oracle_ref(w, rows)
    ref = _run(w)
    for pad in pads or (max(max(w.kept_counts), 1), w.N):
        say(f"{w.name}: padded to {pad} (ragged max {max(w.kept_counts)}, N {w.N})")
        got = _run(w, pad)
        check_padded(w, got[0], got[1], o64, absw, rows=rows, flat=flat)
        assert np.array_equal(bits(got[0]), bits(ref[0])), "padded output differs from ragged"
        assert np.array_equal(bits(got[1]), bits(ref[1])), "padded CLS differs from ragged"


def test_padded_deit_s_fp16():
    _against_oracle_and_ragged(workloads.deit_s())


@pytest.mark.parametrize("B,p", [(1, 0.8), (4, 0.5), (2, 0.0)])
def test_padded_deit_b_sweep_bf16(B, p):
    _against_oracle_and_ragged(workloads.deit_b_sweep(B, p))


def test_padded_deit_b_384_bf16():
    # not unit normal (std 0.5 plus x8 outlier rows): the derived bound; whole
    # images and every kept outlier row, besides a sample
    w = workloads.deit_b_384()
    cu = oracle.scan(w.keep)[0]
    rows = check_rows(w, cu, 160, n_whole_extra=2, min_long=256, n_long=4)
    _against_oracle_and_ragged(w, flat=False, rows=rows)


def test_padded_large_batch_bf16():
    _against_oracle_and_ragged(workloads.large_batch(B=128))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_padded_ragged_tails(dtype):
    g = torch.Generator().manual_seed(19)
    lengths = [1, 0, 16, 17, 63, 64, 65, 129, 200]
    keep = torch.zeros((len(lengths), 200), dtype=torch.uint8)
    for b, L in enumerate(lengths):
        keep[b, torch.randperm(200, generator=g)[:L]] = 1
    _against_oracle_and_ragged(workloads.custom(len(lengths), 200, 2, dtype, keep=keep, seed=19,
                                                name=f"padded_tails_{dtype}"))


def test_padded_shape_differs_from_ragged_shape():
    """Kept counts 130..250 of N = 300: the ragged call with the bound N runs
    128-row tiles; padding to the longest survivor (at most 250) runs 64-row
    tiles.  Unit-normal inputs: the flat tolerance."""
    w = workloads.custom(32, 300, 8, "bf16", keep=keep_length_range(32, 300, 130, 250, 60),
                         seed=64, name="padded_vs_ragged_shapes")
    _against_oracle_and_ragged(w, pads=(max(w.kept_counts),))


def test_padded_shape_differs_late_rescale():
    """As above, with strong keys late in each image, so that some rows move
    their softmax reference after the first chunk and others do not."""
    w = late_outlier_keys(seed=81, name="padded_late_outlier_keys")
    _against_oracle_and_ragged(w, flat=False, pads=(max(w.kept_counts), w.N))


def test_padded_cls_only():
    w = workloads.deit_b_sweep(4, 0.8)
    say("padded comparator, CLS rows only")
    ref = oracle.pipeline(w)
    _, cls_ref = _run(w, want_out=False)
    _, cls = _run(w, pad=w.N, want_out=False)
    assert np.array_equal(bits(cls), bits(cls_ref))
    # against the oracle: the CLS row of each image is its flat row cu[b]
    cu = ref["cu"]
    o = oracle.widen(bits(cls), w.dtype).reshape(w.B, w.H, w.D)
    err = max(float(np.abs(o[b] - ref["o64"][cu[b]]).max()) for b in range(w.B))
    say(f"CLS rows max|err|={err:.3e}")
    assert err <= 1e-2
