"""Parity of rattn_forward (flat ragged attention through the C ABI) with the
CPU oracle, on MI355X.

The flat q/k/v buffers and cu_seqlens are prepared on the host: the kept rows
of the padded tensors in (image, position) order, and the prefix sum of the
kept counts.  rattn_pack does not run here.  Checked:

* every kept row's output against the oracle, within the per-dtype tolerances
  of `_gpu_util` (fp32 1e-4, fp16 2e-3, bf16 1e-2 max-abs on unit-normal
  inputs; the 384 px workload against the rounding bound derived there);
* rows past T are left untouched;
* the output is bitwise the fused kernel's output gathered at the kept
  positions, since both run the same attention core;
* the bits do not depend on the max_seqlen bound, the run, or the other
  images' contents; the batch's head count picks the core (up to 24 heads,
  images longer than one chunk split their keys over the wavefronts);
* an image longer than max_seqlen breaks the contract and is left unwritten.

The five named workloads run at full size with max_seqlen = N, the launch
configuration of the fused benchmark; at the two largest the oracle computes
sampled rows one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import (FLAT_TOL, UNIT_ROUNDOFF, bits, check_rows, late_outlier_keys,
                             say)

pytestmark = pytest.mark.gpu
CANARY = 0x5A
EXTRA_ROWS = 37


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def host_flat(w):
    """Kept rows of q, k, v in (image, position) order, and cu_seqlens."""
    keep = w.keep != 0
    flat = [t[keep].contiguous() for t in (w.q, w.k, w.v)]
    counts = keep.sum(dim=1).to(torch.int64)
    cu = torch.zeros(w.B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return flat, cu


def run_forward(w, max_seqlen=None, stream=None, flat_cu=None):
    """rattn_forward on capacity T + EXTRA_ROWS buffers; returns (o[:T+extra] on
    CPU, T)."""
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    flat, cu = flat_cu if flat_cu is not None else host_flat(w)
    T = flat[0].shape[0]
    cap = T + EXTRA_ROWS
    bufs = []
    for t in flat:
        b = torch.empty((cap, w.H, w.D), dtype=t.dtype, device=dev)
        b.view(torch.uint8).fill_(CANARY)
        b[:T].copy_(t.to(dev))
        bufs.append(b)
    o = torch.empty((cap, w.H, w.D), dtype=flat[0].dtype, device=dev)
    o.view(torch.uint8).fill_(CANARY)
    ms = w.N if max_seqlen is None else max_seqlen
    rv.rattn_forward(*bufs, o, cu.to(dev), ms, w.scale, stream=stream)
    torch.cuda.synchronize()
    return o.cpu(), T


def check(w, o, T, o64, absw, rows=None, flat=True):
    assert np.all(o[T:].view(torch.uint8).numpy() == CANARY), "rows past T written"
    got = oracle.widen(o[:T], w.dtype).reshape(T, w.H, w.D)
    if rows is not None:
        got = got[rows]
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - o64)
    bound = FLAT_TOL[w.dtype] + 2.0 * UNIT_ROUNDOFF[w.dtype] * (np.abs(o64) + absw)
    e = float(err.max()) if err.size else 0.0
    r = float((err / bound).max()) if err.size else 0.0
    say(f"{w.name}: T={T} max|err|={e:.3e} err/bound={r:.3f}")
    if flat:
        assert e <= FLAT_TOL[w.dtype], e
    assert r <= 1.0, r


def full(w, flat=True, **kw):
    say(f"{w.name}: B={w.B} N={w.N} H={w.H} {w.dtype} T={w.total_kept}")
    ref = oracle.pipeline(w, want_absw=True)
    o, T = run_forward(w, **kw)
    check(w, o, T, ref["o64"], ref["absw"], flat=flat)
    return o, T


def fused_kept_rows(w):
    """rattn_fused's padded output, gathered at the kept positions (bits)."""
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
    out = torch.empty_like(q)
    rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out)
    torch.cuda.synchronize()
    return bits(out.cpu()[w.keep != 0])


# ---------------------------------------------------------------------------
# the named workloads, full size, max_seqlen = N
# ---------------------------------------------------------------------------
def test_forward_tiny_fp32():
    full(workloads.tiny())


def test_forward_deit_s_80pct_fp16():
    full(workloads.deit_s())


@pytest.mark.parametrize("B,p,exact", workloads.sweep_points())
def test_forward_deit_b_sweep_bf16(B, p, exact):
    full(workloads.deit_b_sweep(B, p, exact_unpruned=exact))


def _sampled(w, nrows, flat, **pick):
    o, T = run_forward(w)
    cu, _, T2 = oracle.scan(w.keep)
    assert T2 == T
    pq, pk, pv = (oracle.pack(t, w.keep) for t in (w.q, w.k, w.v))
    rows = check_rows(w, cu, nrows, **pick)
    say(f"{w.name}: B={w.B} N={w.N} H={w.H} {w.dtype} T={T}: {len(rows)} rows checked")
    o64, absw = oracle.attention(*(oracle.widen(t, w.dtype).reshape(T, w.H, w.D)
                                   for t in (pq, pk, pv)), cu, w.scale, rows=rows,
                                 want_absw=True)
    check(w, o, T, o64, absw, rows=rows, flat=flat)
    return o, T


def test_forward_deit_b_384_50pct_outliers_bf16():
    # whole images (the longest, the shortest, four longer than 256 and two
    # more) and every kept outlier row, besides the sample
    w = workloads.deit_b_384()
    o, T = _sampled(w, nrows=160, flat=False, n_whole_extra=2, min_long=256, n_long=4)
    assert np.array_equal(bits(o[:T]), fused_kept_rows(w)), "forward != fused"


def test_forward_large_batch_threshold_bf16():
    w = workloads.large_batch()
    o, T = _sampled(w, nrows=400, flat=True, n_whole_extra=6)
    assert np.array_equal(bits(o[:T]), fused_kept_rows(w)), "forward != fused"


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
def test_forward_ragged_tails(dtype):
    lengths = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]
    keep = _keep_with_lengths(lengths, 200, seed=3)
    w = workloads.custom(len(lengths), 200, 2, dtype, keep=keep, seed=11, name=f"fwd_tails_{dtype}")
    o, T = full(w, flat=True)
    assert np.array_equal(bits(o[:T]), fused_kept_rows(w)), "forward != fused"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forward_length_one_returns_v_row(dtype):
    B, N = 6, 197
    keep = torch.zeros((B, N), dtype=torch.uint8)
    keep[:, 0] = 1
    w = workloads.custom(B, N, 3, dtype, keep=keep, seed=12, name=f"fwd_len1_{dtype}")
    o, T = full(w, flat=True)
    assert np.array_equal(bits(o[:T]), bits(w.v[:, 0]))


def test_forward_empty_images():
    B, N = 5, 40
    keep = torch.zeros((B, N), dtype=torch.uint8)
    keep[1, [3, 9, 10]] = 1
    keep[3, :] = 1
    full(workloads.custom(B, N, 2, "bf16", keep=keep, seed=13, name="fwd_empty"), flat=True)


def test_forward_nothing_to_do_writes_nothing():
    w = workloads.custom(3, 50, 2, "bf16", keep=torch.zeros((3, 50), dtype=torch.uint8), seed=14)
    say("every token pruned; max_seqlen 0")
    o, T = run_forward(w)
    assert T == 0 and np.all(o.view(torch.uint8).numpy() == CANARY)
    o0, _ = run_forward(w, max_seqlen=0)
    assert np.all(o0.view(torch.uint8).numpy() == CANARY)


@pytest.mark.parametrize("N", [577, 1100, 2048])
def test_forward_long_sequences(N):
    keep = torch.ones((2, N), dtype=torch.uint8)
    keep[1, N // 3:] = 0
    w = workloads.custom(2, N, 2, "bf16", keep=keep, seed=15, name=f"fwd_long_{N}")
    o, T = full(w, flat=True)
    assert np.array_equal(bits(o[:T]), fused_kept_rows(w)), "forward != fused"


def test_forward_max_seqlen_bound_does_not_change_bits():
    w = workloads.deit_s()
    flat_cu = host_flat(w)
    say("max_seqlen exact vs N vs 4N")
    a, T = run_forward(w, max_seqlen=max(w.kept_counts), flat_cu=flat_cu)
    b, _ = run_forward(w, max_seqlen=w.N, flat_cu=flat_cu)
    c, _ = run_forward(w, max_seqlen=4 * w.N, flat_cu=flat_cu)
    assert np.array_equal(bits(a), bits(b)) and np.array_equal(bits(a), bits(c))


def _keep_length_range(B, N, lo, hi, seed):
    """Keep mask whose image b keeps a random subset of lo..hi positions."""
    g = torch.Generator().manual_seed(seed)
    keep = torch.zeros((B, N), dtype=torch.uint8)
    for b in range(B):
        L = int(torch.randint(lo, hi + 1, (1,), generator=g))
        keep[b, torch.randperm(N, generator=g)[:L]] = 1
    return keep


def test_forward_bound_across_tile_shapes_does_not_change_bits():
    # N = 300 selects 128-row tiles (up to three workgroups per head); the
    # exact bound (at most 250) selects 64-row tiles
    w = workloads.custom(32, 300, 8, "bf16", keep=_keep_length_range(32, 300, 130, 250, 60),
                         seed=61, name="fwd_bound_shapes")
    flat_cu = host_flat(w)
    say("max_seqlen exact (64-row tiles) vs N (128-row tiles)")
    a, _ = run_forward(w, max_seqlen=max(w.kept_counts), flat_cu=flat_cu)
    b, _ = run_forward(w, max_seqlen=w.N, flat_cu=flat_cu)
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("B,H,picks", [(8, 32, (0, 3, 7)), (3, 8, (0, 1, 2))],
                         ids=["many_heads", "few_heads"])
def test_forward_batch_equals_images_one_by_one(B, H, picks):
    # the core depends on the batch's head count (up to 24 heads, images
    # longer than one chunk split their keys over the wavefronts); on the
    # same side of that line a batch and its images alone split the heads over
    # workgroups differently and give the same bits (rows past 256 take the
    # key chunks in reverse)
    w = workloads.custom(B, 400, H, "bf16", keep=_keep_length_range(B, 400, 260, 380, 62),
                         seed=63, name=f"fwd_batch_vs_single_{B}x{H}")
    flat, cu = host_flat(w)
    say(f"{B * H}-head batch vs images one by one, N=400, kept 260..380")
    o, T = run_forward(w, flat_cu=(flat, cu))
    for b in picks:
        s, e = int(cu[b]), int(cu[b + 1])
        one = workloads.custom(1, 400, H, "bf16", keep=w.keep[b:b + 1].clone(), seed=63,
                               name=f"fwd_single_{b}")
        one.q, one.k, one.v = (t[b:b + 1].clone() for t in (w.q, w.k, w.v))
        o1, T1 = run_forward(one)
        assert T1 == e - s
        assert np.array_equal(bits(o1[:T1]), bits(o[s:e])), b


def test_forward_one_chunk_images_same_bits_at_any_head_count():
    # images of at most 64 kept tokens run the same core in a batch of many
    # heads (256) and alone (8 heads)
    w = workloads.custom(32, 197, 8, "bf16", keep=_keep_length_range(32, 197, 1, 64, 64),
                         seed=65, name="fwd_one_chunk_batch")
    flat, cu = host_flat(w)
    say("256-head batch of one-chunk images vs images one by one")
    o, T = run_forward(w, flat_cu=(flat, cu))
    for b in (0, 13, 31):
        s, e = int(cu[b]), int(cu[b + 1])
        one = workloads.custom(1, 197, 8, "bf16", keep=w.keep[b:b + 1].clone(), seed=65,
                               name=f"fwd_one_chunk_{b}")
        one.q, one.k, one.v = (t[b:b + 1].clone() for t in (w.q, w.k, w.v))
        o1, T1 = run_forward(one)
        assert T1 == e - s
        assert np.array_equal(bits(o1[:T1]), bits(o[s:e])), b


def test_forward_image_longer_than_bound_is_left_unwritten():
    lengths = [10, 40, 12]
    keep = _keep_with_lengths(lengths, 64, seed=18)
    w = workloads.custom(3, 64, 2, "bf16", keep=keep, seed=18, name="fwd_over_bound")
    say("image 1 longer than max_seqlen")
    ref = oracle.pipeline(w)
    o, T = run_forward(w, max_seqlen=20)
    cu = ref["cu"]
    ob = o.view(torch.uint8).numpy()
    assert np.all(ob[cu[1]:cu[2]] == CANARY), "over-long image was written"
    for b in (0, 2):
        got = oracle.widen(o[cu[b]:cu[b + 1]], "bf16").reshape(-1, w.H, w.D)
        assert np.abs(got - ref["o64"][cu[b]:cu[b + 1]]).max() <= FLAT_TOL["bf16"]


def test_forward_run_to_run_determinism():
    w = workloads.large_batch(B=64)
    flat_cu = host_flat(w)
    say("determinism")
    a, _ = run_forward(w, flat_cu=flat_cu)
    b, _ = run_forward(w, flat_cu=flat_cu)
    assert np.array_equal(bits(a), bits(b))


def test_forward_cross_image_isolation():
    w = workloads.deit_b_sweep(4, 0.25)
    say("isolation")
    a, T = run_forward(w)
    cu = oracle.scan(w.keep)[0]
    w.k[2] = -w.k[2]
    w.v[2] = w.v[2] * 2
    b, _ = run_forward(w)
    others = np.ones(T, bool)
    others[cu[2]:cu[3]] = False
    assert np.array_equal(bits(a[:T])[others], bits(b[:T])[others])
    assert not np.array_equal(bits(a[cu[2]:cu[3]]), bits(b[cu[2]:cu[3]]))


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_forward_unusual_scales(scale):
    full(workloads.custom(4, 90, 2, "bf16", p_keep=0.7, seed=17, scale=scale,
                          name=f"fwd_scale_{scale}"), flat=scale != 0.5)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_forward_unusual_scales_two_block_tiles(scale):
    # 300 positions select the 128-row tiles whose Q rows are staged in LDS;
    # 32 x 8 = 256 heads give one workgroup per head, so each copies the next
    # tile's Q rows while its current tile finishes
    full(workloads.custom(32, 300, 8, "bf16", p_keep=0.9, seed=19, scale=scale,
                          name=f"fwd_scale_{scale}_128_row_tiles"), flat=scale != 0.5)


def test_forward_side_stream():
    w = workloads.deit_b_sweep(2, 0.8)
    s = torch.cuda.Stream()
    say("non-default stream")
    ref = oracle.pipeline(w, want_absw=True)
    with torch.cuda.stream(s):
        o, T = run_forward(w, stream=s)
    check(w, o, T, ref["o64"], ref["absw"])


def test_forward_late_rescale_is_per_row_across_bounds():
    """Rows whose softmax reference moves after the first chunk next to rows
    whose reference does not: the bound N (128-row tiles) and the exact bound
    (64-row tiles) give the same bits, within the oracle's rounding bound, and
    the fused kernel's bits."""
    w = late_outlier_keys(name="fwd_late_outlier_keys")
    flat_cu = host_flat(w)
    say(f"{w.name}: late outlier keys, bound N vs exact")
    ref = oracle.pipeline(w, want_absw=True)
    a, T = run_forward(w, max_seqlen=w.N, flat_cu=flat_cu)
    check(w, a, T, ref["o64"], ref["absw"], flat=False)
    b, _ = run_forward(w, max_seqlen=max(w.kept_counts), flat_cu=flat_cu)
    assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(bits(a[:T]), fused_kept_rows(w)), "forward != fused"


@pytest.mark.parametrize("N", [90, 300])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forward_tiny_positive_scale(dtype, N):
    """scale 1e-39: 8 / (scale log2 e) overflows float32; the output is the
    mean of the image's V rows."""
    full(workloads.custom(4, N, 2, dtype, p_keep=0.7, seed=23, scale=1e-39,
                          name=f"fwd_scale_1e-39_{dtype}_{N}"), flat=True)
