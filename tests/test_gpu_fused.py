"""Parity of the one-launch path (rattn_fused, through the C ABI) with the CPU
oracle, on MI355X.

rattn_fused reads padded q/k/v and the keep mask and writes the padded output
and the CLS rows directly.  Checked: pruned output rows are exactly zero; the
kept rows, gathered in (b, n) order, match the oracle's attention within the
tolerances of `_gpu_util` (fp32 1e-4, fp16 2e-3, bf16 1e-2 max-abs on
unit-normal inputs; the 384 px workload against the derived rounding bound);
CLS rows are bitwise the output rows (b, 0); results do not depend on the
max_seqlen bound, on the contents of pruned input rows, on other images'
contents, or on the run (the batch's head count picks the core: up to 24
heads, images longer than one chunk split their keys over the wavefronts, and
a batch and its images alone agree bitwise on either side of that line).  The
five named workloads run at full size in the launch
configuration the benchmark times (max_seqlen = N); at the two largest the
oracle computes sampled rows one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import bits, check_padded, check_rows, late_outlier_keys, say

pytestmark = pytest.mark.gpu
POISON = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def run_fused(w, max_seqlen=None, poison_pruned=False, want_out=True, want_cls=True,
              stream=None):
    """One rattn_fused call; returns CPU copies of (out, cls)."""
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    q, k, v = (t.clone() for t in (w.q, w.k, w.v))
    if poison_pruned:
        pruned = w.keep == 0
        for t in (q, k, v):
            t[pruned] = float("nan")
    q, k, v = (t.to(dev) for t in (q, k, v))
    keep = w.keep.to(dev)
    out = torch.empty_like(q) if want_out else None
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev) if want_cls else None
    for t in (out, cls):
        if t is not None:
            t.view(torch.uint8).fill_(POISON)
    rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out, cls=cls, max_seqlen=max_seqlen,
                   stream=stream)
    torch.cuda.synchronize()
    return (None if out is None else out.cpu()), (None if cls is None else cls.cpu())


def kept_rows(out, keep):
    """Kept rows of a padded output, in (b, n) order (bitwise gather)."""
    return oracle.pack(out, keep)


def check(w, out, cls, o64, absw, rows=None, flat=True):
    check_padded(w, out, cls, o64, absw, rows=rows, flat=flat)


def full(w, flat=True, **kw):
    say(f"{w.name}: B={w.B} N={w.N} H={w.H} {w.dtype} T={w.total_kept}")
    ref = oracle.pipeline(w, want_absw=True)
    out, cls = run_fused(w, **kw)
    check(w, out, cls, ref["o64"], ref["absw"], flat=flat)
    return out, cls, ref


# ---------------------------------------------------------------------------
# the named workloads, full size, max_seqlen = N
# ---------------------------------------------------------------------------
def test_fused_tiny_fp32():
    full(workloads.tiny())


def test_fused_deit_s_80pct_fp16():
    full(workloads.deit_s())


@pytest.mark.parametrize("B,p,exact", workloads.sweep_points())
def test_fused_deit_b_sweep_bf16(B, p, exact):
    full(workloads.deit_b_sweep(B, p, exact_unpruned=exact))


def _sampled(w, nrows, flat, **pick):
    out, cls = run_fused(w)
    cu, _, T = oracle.scan(w.keep)
    pq, pk, pv = (oracle.pack(t, w.keep) for t in (w.q, w.k, w.v))
    rows = check_rows(w, cu, nrows, **pick)
    say(f"{w.name}: B={w.B} N={w.N} H={w.H} {w.dtype} T={T}: {len(rows)} rows checked")
    o64, absw = oracle.attention(*(oracle.widen(t, w.dtype).reshape(T, w.H, w.D)
                                   for t in (pq, pk, pv)), cu, w.scale, rows=rows,
                                 want_absw=True)
    check(w, out, cls, o64, absw, rows=rows, flat=flat)


def test_fused_deit_b_384_50pct_outliers_bf16():
    # whole images: the longest, the shortest, four longer than 256 (their
    # rows past 256 take the key chunks in reverse) and two more; every kept
    # outlier row (they move the softmax reference after the first chunk)
    _sampled(workloads.deit_b_384(), nrows=160, flat=False, n_whole_extra=2, min_long=256,
             n_long=4)


def test_fused_large_batch_threshold_bf16():
    _sampled(workloads.large_batch(), nrows=400, flat=True, n_whole_extra=6)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def _keep_with_lengths(lengths, N, seed):
    g = torch.Generator().manual_seed(seed)
    keep = torch.zeros((len(lengths), N), dtype=torch.uint8)
    for b, L in enumerate(lengths):
        keep[b, torch.randperm(N, generator=g)[:L]] = 1
    return keep


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fused_ragged_tails(dtype):
    lengths = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]
    keep = _keep_with_lengths(lengths, 200, seed=3)
    full(workloads.custom(len(lengths), 200, 2, dtype, keep=keep, seed=11,
                          name=f"tails_{dtype}"), flat=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fused_length_one_returns_v_row(dtype):
    B, N = 6, 197
    keep = torch.zeros((B, N), dtype=torch.uint8)
    keep[:, 0] = 1
    keep[3, 0] = 0
    keep[3, 77] = 1  # one kept patch, CLS pruned
    w = workloads.custom(B, N, 3, dtype, keep=keep, seed=12, name=f"len1_{dtype}")
    out, cls, ref = full(w, flat=True)
    assert np.array_equal(bits(kept_rows(out, w.keep)), ref["v"].view(bits(out).dtype))


def test_fused_empty_images_and_pruned_cls():
    B, N = 5, 40
    keep = torch.zeros((B, N), dtype=torch.uint8)
    keep[1, [3, 9, 10]] = 1
    keep[3, :] = 1
    out, cls, _ = full(workloads.custom(B, N, 2, "bf16", keep=keep, seed=13, name="empty"),
                       flat=True)
    assert not cls[[0, 1, 2, 4]].view(torch.int16).any()


def test_fused_everything_pruned():
    B, N = 3, 50
    w = workloads.custom(B, N, 2, "bf16", keep=torch.zeros((B, N), dtype=torch.uint8), seed=14)
    say("every token pruned")
    out, cls = run_fused(w)
    assert not out.view(torch.int16).any() and not cls.view(torch.int16).any()
    out0, cls0 = run_fused(w, max_seqlen=0)
    assert not out0.view(torch.int16).any() and not cls0.view(torch.int16).any()


@pytest.mark.parametrize("N", [577, 1100, 2048])
def test_fused_long_sequences(N):
    keep = torch.ones((2, N), dtype=torch.uint8)
    keep[1, N // 3:] = 0
    full(workloads.custom(2, N, 2, "bf16", keep=keep, seed=15, name=f"long_{N}"), flat=True)


@pytest.mark.parametrize("N", [256, 257, 1024, 1025])
def test_fused_rank_tiers(N):
    # the mask is ranked by every wavefront up to 4 and up to 16 chunks of 64
    # positions, through an LDS exchange past that: each side of both edges,
    # with an image that keeps only its last position and one that keeps all
    keep = _keep_length_range(4, N, 1, N // 3, seed=17 + N)
    keep[1] = 0
    keep[1, N - 1] = 1
    keep[2] = 1
    full(workloads.custom(4, N, 2, "bf16", keep=keep, seed=18 + N, name=f"rank_tier_{N}"))


@pytest.mark.parametrize("B,N", [(1, 1), (3, 5), (700, 7)])
def test_fused_small_rows(B, N):
    full(workloads.custom(B, N, 1, "bf16", p_keep=0.6, seed=16 + N, name=f"small_{B}x{N}"),
         flat=True)


def test_fused_max_seqlen_bound_does_not_change_bits():
    w = workloads.deit_s()
    say("max_seqlen exact vs N vs 4N")
    a = run_fused(w, max_seqlen=max(w.kept_counts))
    b = run_fused(w, max_seqlen=w.N)
    c = run_fused(w, max_seqlen=4 * w.N)
    for x, y in ((a, b), (a, c)):
        assert np.array_equal(bits(x[0]), bits(y[0])) and np.array_equal(bits(x[1]), bits(y[1]))


def _keep_length_range(B, N, lo, hi, seed):
    """Keep mask whose image b keeps a random subset of lo..hi positions."""
    g = torch.Generator().manual_seed(seed)
    keep = torch.zeros((B, N), dtype=torch.uint8)
    for b in range(B):
        L = int(torch.randint(lo, hi + 1, (1,), generator=g))
        keep[b, torch.randperm(N, generator=g)[:L]] = 1
    return keep


def test_fused_bound_across_tile_shapes_does_not_change_bits():
    # N = 300 selects 128-row tiles; the exact bound (at most 250) selects
    # 64-row tiles
    w = workloads.custom(32, 300, 8, "bf16", keep=_keep_length_range(32, 300, 130, 250, 60),
                         seed=61, name="bound_shapes")
    say("max_seqlen exact (64-row tiles) vs N (128-row tiles)")
    a = run_fused(w, max_seqlen=max(w.kept_counts))
    b = run_fused(w, max_seqlen=w.N)
    assert np.array_equal(bits(a[0]), bits(b[0])) and np.array_equal(bits(a[1]), bits(b[1]))


@pytest.mark.parametrize("B,H,picks", [(8, 32, (0, 3, 7)), (3, 8, (0, 1, 2))],
                         ids=["many_heads", "few_heads"])
def test_fused_batch_equals_images_one_by_one(B, H, picks):
    # The core depends on the batch's head count: up to 24 heads an image
    # longer than one 64-key chunk has its keys split over a workgroup's
    # wavefronts.  A batch and its images alone on the same side of that line
    # give the same bits.  Many heads (256 in the batch): one workgroup per
    # head, whose later tiles take the key chunks of rows past 256 in reverse
    # and reuse the double buffer's chunks; an image alone: a workgroup per
    # tile, no reuse.  Few heads: different numbers of workgroups per head.
    w = workloads.custom(B, 400, H, "bf16", keep=_keep_length_range(B, 400, 260, 380, 62),
                         seed=63, name=f"batch_vs_single_{B}x{H}")
    say(f"{B * H}-head batch vs images one by one, N=400, kept 260..380")
    out, cls = run_fused(w)
    for b in picks:
        one = workloads.custom(1, 400, H, "bf16", keep=w.keep[b:b + 1].clone(), seed=63,
                               name=f"single_{b}")
        one.q, one.k, one.v = (t[b:b + 1].clone() for t in (w.q, w.k, w.v))
        o1, c1 = run_fused(one)
        assert np.array_equal(bits(o1[0]), bits(out[b])), b
        assert np.array_equal(bits(c1[0]), bits(cls[b])), b


def test_fused_one_chunk_images_same_bits_at_any_head_count():
    # images of at most 64 kept tokens run the same core in a batch of many
    # heads (256) and alone (8 heads, a batch of few)
    w = workloads.custom(32, 197, 8, "bf16", keep=_keep_length_range(32, 197, 1, 64, 64),
                         seed=65, name="one_chunk_batch")
    say("256-head batch of one-chunk images vs images one by one")
    out, cls = run_fused(w)
    for b in (0, 13, 31):
        one = workloads.custom(1, 197, 8, "bf16", keep=w.keep[b:b + 1].clone(), seed=65,
                               name=f"one_chunk_{b}")
        one.q, one.k, one.v = (t[b:b + 1].clone() for t in (w.q, w.k, w.v))
        o1, c1 = run_fused(one)
        assert np.array_equal(bits(o1[0]), bits(out[b])), b
        assert np.array_equal(bits(c1[0]), bits(cls[b])), b


def test_fused_poisoned_pruned_rows_do_not_leak():
    w = workloads.deit_b_sweep(4, 0.5)
    say("NaN-poisoned pruned rows")
    a = run_fused(w)
    b = run_fused(w, poison_pruned=True)
    assert np.array_equal(bits(a[0]), bits(b[0])) and np.array_equal(bits(a[1]), bits(b[1]))


def test_fused_run_to_run_determinism():
    w = workloads.large_batch(B=64)
    say("determinism")
    a, b = run_fused(w), run_fused(w)
    assert np.array_equal(bits(a[0]), bits(b[0])) and np.array_equal(bits(a[1]), bits(b[1]))


def test_fused_cross_image_isolation():
    w = workloads.deit_b_sweep(4, 0.25)
    say("isolation")
    a = run_fused(w)
    w.k[2] = -w.k[2]
    w.v[2] = w.v[2] * 2
    b = run_fused(w)
    others = [0, 1, 3]
    assert np.array_equal(bits(a[0])[others], bits(b[0])[others])
    assert not np.array_equal(bits(a[0])[2], bits(b[0])[2])


def test_fused_cls_only_matches_full():
    w = workloads.deit_b_sweep(4, 0.8)
    say("CLS rows only")
    _, cls_full = run_fused(w)
    out_none, cls_only = run_fused(w, want_out=False)
    assert out_none is None
    assert np.array_equal(bits(cls_only), bits(cls_full))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fused_cls_only_several_tiles(dtype):
    """CLS rows only, with two to three 64-row query tiles per head: only the
    tile holding row 0 is computed, and it gives the full run's bits."""
    keep = torch.zeros((4, 197), dtype=torch.uint8)
    g = torch.Generator().manual_seed(31)
    for b, L in enumerate((150, 197, 65, 129)):
        keep[b, torch.randperm(197, generator=g)[:L]] = 1
    keep[1:, 0] = 1  # image 0 may have lost its CLS row; the others keep it
    w = workloads.custom(4, 197, 3, dtype, keep=keep, seed=32, name=f"cls_only_{dtype}")
    say(f"CLS rows only, several tiles, {dtype}")
    _, cls_full = run_fused(w)
    _, cls_only = run_fused(w, want_out=False)
    assert np.array_equal(bits(cls_only), bits(cls_full))


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_fused_unusual_scales(scale):
    full(workloads.custom(4, 90, 2, "bf16", p_keep=0.7, seed=17, scale=scale,
                          name=f"scale_{scale}"), flat=scale != 0.5)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_fused_unusual_scales_two_block_tiles(scale):
    # 300 positions select the 128-row tiles whose Q rows are staged in LDS;
    # 32 x 8 = 256 heads give one workgroup per head, so each copies the next
    # tile's Q rows while its current tile finishes
    full(workloads.custom(32, 300, 8, "bf16", p_keep=0.9, seed=19, scale=scale,
                          name=f"scale_{scale}_128_row_tiles"), flat=scale != 0.5)


def test_fused_side_stream():
    w = workloads.deit_b_sweep(2, 0.8)
    s = torch.cuda.Stream()
    say("non-default stream")
    ref = oracle.pipeline(w, want_absw=True)
    with torch.cuda.stream(s):
        out, cls = run_fused(w, stream=s)
    check(w, out, cls, ref["o64"], ref["absw"])


def test_fused_late_rescale_is_per_row_across_shapes_and_modes():
    """Rows whose softmax reference moves after the first chunk (strong keys
    late in the image) next to rows whose reference does not: the bound N
    (128-row tiles), the exact bound (64-row tiles) and the CLS-only mode
    (64-row tiles) give the same bits, within the rounding bound of the oracle
    (these keys are not unit normal)."""
    w = late_outlier_keys()
    say(f"{w.name}: late outlier keys, bound N vs exact vs CLS only")
    ref = oracle.pipeline(w, want_absw=True)
    out_n, cls_n = run_fused(w, max_seqlen=w.N)
    check(w, out_n, cls_n, ref["o64"], ref["absw"], flat=False)
    out_e, cls_e = run_fused(w, max_seqlen=max(w.kept_counts))
    assert np.array_equal(bits(out_e), bits(out_n)) and np.array_equal(bits(cls_e), bits(cls_n))
    _, cls_only = run_fused(w, want_out=False)
    assert np.array_equal(bits(cls_only), bits(cls_n))


def test_fused_cls_only_matches_full_at_384px():
    """At 577 positions the full call runs 128-row tiles and the CLS-only call
    64-row tiles; the outlier rows of this workload move the softmax reference
    after the first chunk."""
    w = workloads.deit_b_384()
    say(f"{w.name}: CLS rows only vs full")
    _, cls_full = run_fused(w)
    _, cls_only = run_fused(w, want_out=False)
    assert np.array_equal(bits(cls_only), bits(cls_full))


@pytest.mark.parametrize("N", [90, 300])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fused_tiny_positive_scale(dtype, N):
    """scale 1e-39: 8 / (scale log2 e) overflows float32; the output is the
    mean of the image's V rows."""
    full(workloads.custom(4, N, 2, dtype, p_keep=0.7, seed=23, scale=1e-39,
                          name=f"scale_1e-39_{dtype}_{N}"), flat=True)
