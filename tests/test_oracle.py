"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in `oracle/oracle.c` fails at least
one of them: a wrong image boundary (library SDPA per image, brute force,
isolation), a dropped scale or a transposed operand (SDPA, closed forms), a
missing max-subtraction (large-logit one-hot case), a wrong value index (constant
and one-hot cases), a wrong pack order (hand-derived fixture, round trips).

Pages: "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
(arXiv 2604.15408): the abstract and the radpulse.milrad-way.com write-up's
sections on padding, on the Triton bidirectional kernel and on the integrated
packing pipeline.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_case(seed, B, N, H, D, p_keep=0.6, std=1.0, force_cls=True):
    rng = np.random.default_rng(seed)
    keep = (rng.random((B, N)) < p_keep).astype(np.uint8)
    if force_cls:
        keep[:, 0] = 1
    q = rng.normal(0, std, (B, N, H, D))
    k = rng.normal(0, std, (B, N, H, D))
    v = rng.normal(0, std, (B, N, H, D))
    return keep, q, k, v


def _oracle_padded_inputs(keep, q, k, v, scale, **kw):
    cu, mx, tot = oracle.scan(keep)
    pq, pk, pv = (oracle.pack(x, keep) for x in (q, k, v))
    o = oracle.attention(pq, pk, pv, cu, scale, **kw)
    return cu, pq, pk, pv, o


# --------------------------------------------------------------------------
# scan / pack / unpack
# --------------------------------------------------------------------------
def test_scan_pack_hand_fixture():
    g = _load("scan_pack_small.json")
    keep = np.array(g["keep"], dtype=np.uint8)
    cu, mx, tot = oracle.scan(keep)
    assert cu.tolist() == g["cu_seqlens"]
    assert mx == g["max_seqlen"] and tot == g["total"]
    assert np.diff(cu).tolist() == g["counts"]
    B, N = keep.shape
    # tag every padded row with its own (b, n) so the packed order is visible
    src = np.zeros((B, N, 2), dtype=np.int32)
    for b in range(B):
        for n in range(N):
            src[b, n] = (b, n)
    packed = oracle.pack(src, keep)
    assert packed.tolist() == g["packed_source_positions"]
    dst, cls = oracle.unpack(packed, keep, cu)
    for b in range(B):
        r = g["cls_from_packed_row"][b]
        want = np.zeros(2, np.int32) if r is None else packed[r]
        assert cls[b].tolist() == want.tolist()
        for n in range(N):
            want = src[b, n] if keep[b, n] else np.zeros(2, np.int32)
            assert dst[b, n].tolist() == want.tolist()


@pytest.mark.parametrize("seed", range(6))
def test_pack_unpack_identities(seed):
    rng = np.random.default_rng(100 + seed)
    B, N = int(rng.integers(1, 7)), int(rng.integers(1, 40))
    keep = (rng.random((B, N)) < rng.random()).astype(np.uint8)
    keep[rng.random((B, N)) < 0.05] = 7  # any nonzero byte means kept
    x = rng.integers(-2**15, 2**15, (B, N, 3, 5), dtype=np.int16)
    cu, mx, tot = oracle.scan(keep)
    counts = (keep != 0).sum(1)
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0)
    assert cu[-1] == tot == int((keep != 0).sum())
    assert mx == (counts.max() if B else 0)
    assert np.diff(cu).tolist() == counts.tolist()
    p = oracle.pack(x, keep)
    assert p.shape == (tot, 3, 5)
    dst, cls = oracle.unpack(p, keep, cu)
    # unpack(pack(x)) = x on kept rows, zero bytes elsewhere
    assert np.array_equal(dst, np.where((keep != 0)[:, :, None, None], x, 0))
    # pack(unpack(y)) = y
    y = rng.integers(-2**15, 2**15, (tot, 3, 5), dtype=np.int16)
    d2, c2 = oracle.unpack(y, keep, cu)
    assert np.array_equal(oracle.pack(d2, keep), y)
    for b in range(B):
        if keep[b, 0]:
            assert np.array_equal(c2[b], y[cu[b]])
        else:
            assert not c2[b].any()


def test_unpack_rejects_inconsistent_cu():
    keep = np.array([[1, 1, 0]], dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.unpack(np.zeros((3, 4), np.float32), keep, np.array([0, 3], np.int32))


def test_scan_all_empty_and_all_kept():
    cu, mx, tot = oracle.scan(np.zeros((3, 8), np.uint8))
    assert cu.tolist() == [0, 0, 0, 0] and mx == 0 and tot == 0
    cu, mx, tot = oracle.scan(np.ones((3, 8), np.uint8))
    assert cu.tolist() == [0, 8, 16, 24] and mx == 8 and tot == 24


# --------------------------------------------------------------------------
# attention: hand-derived fixtures and closed forms
# --------------------------------------------------------------------------
def test_attention_hand_fixture():
    g = _load("attention_closed_form.json")
    for case in g["cases"]:
        q = np.array(case["q"])[:, None, :]
        k = np.array(case["k"])[:, None, :]
        v = np.array(case["v"])[:, None, :]
        # one image holding all key rows; query rows are its first rows
        L = k.shape[0]
        qq = np.zeros_like(k)
        qq[: q.shape[0]] = q
        cu = np.array([0, L], np.int32)
        o = oracle.attention(qq, k, v, cu, case["scale"])
        want = np.array(case["expected_o"])
        assert np.max(np.abs(o[: q.shape[0], 0, :] - want)) < 1e-14, case["name"]


def test_two_token_logistic_closed_form():
    # o = sigma(d) v0 + (1 - sigma(d)) v1 with d = s0 - s1
    rng = np.random.default_rng(7)
    D = 64
    for _ in range(20):
        q, k, v = rng.normal(size=(3, 2, 1, D))
        scale = float(rng.uniform(0.05, 0.5))
        o = oracle.attention(q, k, v, np.array([0, 2], np.int32), scale)
        for i in range(2):
            s0 = scale * float(np.sum(q[i, 0] * k[0, 0]))
            s1 = scale * float(np.sum(q[i, 0] * k[1, 0]))
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            want = w0 * v[0, 0] + (1 - w0) * v[1, 0]
            assert np.max(np.abs(o[i, 0] - want)) < 1e-13


def test_length_one_returns_v_row_exactly():
    keep, q, k, v = _rand_case(1, B=3, N=6, H=2, D=64)
    keep[1] = 0
    keep[1, 3] = 1  # image 1 keeps one token (not CLS)
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, 0.125)
    r = cu[1]
    assert cu[2] - cu[1] == 1
    assert np.array_equal(o[r], pv[r])  # p = 1, l = 1: bit-exact


@pytest.mark.parametrize("zero", ["q", "scale"])
def test_uniform_weights_give_mean_of_v(zero):
    keep, q, k, v = _rand_case(2, B=3, N=9, H=2, D=64)
    if zero == "q":
        q[:] = 0.0
    scale = 0.0 if zero == "scale" else 0.125
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, scale)
    for b in range(3):
        mean = pv[cu[b]:cu[b + 1]].mean(axis=0)
        assert np.max(np.abs(o[cu[b]:cu[b + 1]] - mean[None])) < 1e-14


def test_constant_v_is_returned():
    keep, q, k, v = _rand_case(3, B=2, N=11, H=3, D=64)
    c = np.random.default_rng(3).normal(size=(3, 64))
    v[:] = c[None, None]
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, 0.125)
    assert np.max(np.abs(o - c[None])) < 1e-13


def test_dominant_logit_is_one_hot_and_finite():
    # logits of ~1e4: without subtracting the maximum exp() overflows
    rng = np.random.default_rng(4)
    L, D = 7, 64
    q = np.zeros((L, 1, D))
    k = np.zeros((L, 1, D))
    v = rng.normal(size=(L, 1, D))
    q[:, 0, 0] = 100.0
    k[:, 0, 0] = np.arange(L) * 10.0  # key L-1 wins by >= 1000 in logit
    o = oracle.attention(q, k, v, np.array([0, L], np.int32), 1.0)
    assert np.all(np.isfinite(o))
    assert np.array_equal(o[:, 0], np.repeat(v[L - 1], L, axis=0))


# --------------------------------------------------------------------------
# attention: library routine and brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,B,N,H,D", [(10, 1, 5, 1, 64), (11, 3, 9, 2, 64),
                                          (12, 4, 17, 3, 64), (13, 2, 30, 2, 8),
                                          (14, 5, 40, 4, 64)])
def test_matches_library_sdpa_per_image(seed, B, N, H, D):
    """Each image's ragged attention is textbook SDPA over its kept tokens:
    torch's CPU scaled_dot_product_attention in float64 is the reference."""
    keep, q, k, v = _rand_case(seed, B, N, H, D, p_keep=0.5)
    if B > 2:
        keep[2] = 0  # an empty image contributes nothing
    scale = 1.0 / math.sqrt(D)
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, scale)
    for b in range(B):
        a, z = cu[b], cu[b + 1]
        if z == a:
            continue
        t = [torch.from_numpy(x[a:z]).permute(1, 0, 2).contiguous() for x in (pq, pk, pv)]
        ref = torch.nn.functional.scaled_dot_product_attention(*t, scale=scale)
        ref = ref.permute(1, 0, 2).numpy()
        assert np.max(np.abs(o[a:z] - ref)) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_matches_brute_force_padded_masked(seed):
    """The padded form the pages compare against: every image padded to N rows,
    pruned keys masked with -inf, an N x N softmax per image and head."""
    rng = np.random.default_rng(20 + seed)
    B, N, H = int(rng.integers(1, 4)), int(rng.integers(1, 10)), int(rng.integers(1, 3))
    keep, q, k, v = _rand_case(30 + seed, B, N, H, 64, p_keep=0.6)
    scale = 0.125
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, scale)
    logits = np.einsum("bnhd,bmhd->bhnm", q, k) * scale
    logits = np.where((keep != 0)[:, None, None, :], logits, -np.inf)
    w = np.exp(logits - logits.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    dense = np.einsum("bhnm,bmhd->bnhd", w, v)
    r = 0
    for b in range(B):
        for n in range(N):
            if keep[b, n]:
                assert np.max(np.abs(o[r] - dense[b, n])) < 1e-12
                r += 1


# --------------------------------------------------------------------------
# attention: invariants
# --------------------------------------------------------------------------
def test_permutation_equivariance_within_image():
    keep, q, k, v = _rand_case(5, B=3, N=20, H=2, D=64)
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, 0.125)
    rng = np.random.default_rng(5)
    perm = np.arange(cu[-1])
    for b in range(3):
        seg = perm[cu[b]:cu[b + 1]]
        perm[cu[b]:cu[b + 1]] = rng.permutation(seg)
    o2 = oracle.attention(pq[perm], pk[perm], pv[perm], cu, 0.125)
    assert np.max(np.abs(o2 - o[perm])) < 1e-13


def test_key_shift_invariance():
    keep, q, k, v = _rand_case(6, B=2, N=15, H=2, D=64)
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, 0.125)
    pk2 = pk.copy()
    c = np.random.default_rng(6).normal(size=(2, 2, 64))
    for b in range(2):
        pk2[cu[b]:cu[b + 1]] += c[b][None]  # q.(k + c) = q.k + q.c: same shift for all keys
    o2 = oracle.attention(pq, pk2, pv, cu, 0.125)
    assert np.max(np.abs(o2 - o)) < 1e-12


def test_cross_image_isolation():
    keep, q, k, v = _rand_case(7, B=4, N=12, H=2, D=64)
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, 0.125)
    a, z = cu[2], cu[3]
    pq2, pk2, pv2 = pq.copy(), pk.copy(), pv.copy()
    pk2[a:z] *= -3.0
    pv2[a:z] += 100.0
    o2 = oracle.attention(pq2, pk2, pv2, cu, 0.125)
    mask = np.ones(cu[-1], bool)
    mask[a:z] = False
    assert np.array_equal(o2[mask], o[mask])
    assert not np.array_equal(o2[a:z], o[a:z])


def test_row_subset_bit_identical_and_absw():
    keep, q, k, v = _rand_case(8, B=3, N=25, H=3, D=64)
    cu, pq, pk, pv, o = _oracle_padded_inputs(keep, q, k, v, 0.125)
    rows = np.array([0, cu[1], cu[-1] - 1, 3], np.int64)
    o_sub, absw = oracle.attention(pq, pk, pv, cu, 0.125, rows=rows, want_absw=True)
    assert np.array_equal(o_sub, o[rows])
    assert np.all(absw >= np.abs(o_sub) - 1e-15)
    # with non-negative values the two sums coincide
    o_pos, absw_pos = oracle.attention(pq, pk, np.abs(pv), cu, 0.125, rows=rows, want_absw=True)
    assert np.max(np.abs(o_pos - absw_pos)) < 1e-14


# --------------------------------------------------------------------------
# widening, and the whole path on a named workload
# --------------------------------------------------------------------------
def test_widen_is_exact():
    x = torch.randn(1000, dtype=torch.float32)
    for dt, tdt in (("f32", torch.float32), ("f16", torch.float16), ("bf16", torch.bfloat16)):
        y = x.to(tdt)
        assert np.array_equal(oracle.widen(y, dt), y.to(torch.float64).numpy())


def test_pipeline_on_tiny_workload():
    w = workloads.tiny()
    res = oracle.pipeline(w)
    cu = res["cu"]
    assert cu[-1] == w.total_kept == res["total"]
    assert res["max_seqlen"] == max(w.kept_counts)
    # the packed q rows are bitwise the kept padded rows in order
    flat = w.q.reshape(w.B * w.N, w.H, w.D).numpy()
    idx = np.nonzero(w.keep.reshape(-1).numpy())[0]
    assert np.array_equal(res["q"], flat[idx])
    assert res["o64"].shape == (cu[-1], w.H, w.D)


# ---------------------------------------------------------------------------
# re-pack (a second pruning stage on the packed buffer)
# ---------------------------------------------------------------------------
def test_repack_hand_fixture():
    # two images of 3 and 2 rows; rows are single bytes equal to their index
    src = np.arange(5, dtype=np.uint8).reshape(5, 1)
    cu = np.array([0, 3, 5], np.int32)
    keep2 = np.array([1, 0, 1, 0, 0], np.uint8)
    out, cu2 = oracle.repack(src, keep2, cu)
    assert out.reshape(-1).tolist() == [0, 2]
    assert cu2.tolist() == [0, 2, 2]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_repack_composes_with_pack(seed):
    """Pruning in two stages equals pruning once with both masks:
    repack(pack(x, k1), k2 at the kept rows) == pack(x, k1 & k2), and the new
    cu_seqlens is the scan of k1 & k2."""
    rng = np.random.default_rng(seed)
    B, N, H, D = 5, 23, 2, 8
    x = rng.normal(size=(B, N, H, D)).astype(np.float32)
    k1 = (rng.random((B, N)) < 0.6).astype(np.uint8)
    k2 = (rng.random((B, N)) < 0.5).astype(np.uint8)
    k1[2] = 0                      # an image emptied by the first stage
    k2[3] = 0                      # and one by the second
    cu1, _, _ = oracle.scan(k1)
    flat = oracle.pack(x, k1)
    k2_flat = oracle.pack(k2[..., None], k1).reshape(-1)
    out, cu2 = oracle.repack(flat, k2_flat, cu1)
    both = (k1 & k2).astype(np.uint8)
    assert np.array_equal(out.view(np.uint8), oracle.pack(x, both).view(np.uint8))
    assert cu2.tolist() == oracle.scan(both)[0].tolist()


def test_repack_keep_all_is_identity_and_keep_none_empties():
    rng = np.random.default_rng(7)
    cu = np.array([0, 4, 4, 9], np.int32)
    src = rng.integers(0, 2 ** 16, size=(9, 3), dtype=np.uint16)
    out, cu2 = oracle.repack(src, np.ones(9, np.uint8), cu)
    assert np.array_equal(out, src) and cu2.tolist() == cu.tolist()
    out0, cu0 = oracle.repack(src, np.zeros(9, np.uint8), cu)
    assert out0.shape[0] == 0 and cu0.tolist() == [0, 0, 0, 0]
