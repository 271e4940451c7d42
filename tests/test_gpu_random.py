"""Seeded random cases on MI355X: every entry point of the path against the
CPU oracle, on shapes and masks drawn at random (the property-based layer of
the parity tests; the named workloads and the hand-picked edge cases are in
the other test_gpu_* modules).

Each case draws B, N, H, the dtype, a pruning rate (per image, so lengths
spread widely, empty images included), the scale and the max_seqlen bound
from its own seed, then checks:
  * rattn_pack: cu_seqlens, max, total and the packed rows bit-exact;
  * rattn_forward, rattn_fused, rattn_pack -> rattn_forward -> rattn_unpack:
    kept rows within the tolerances of `_gpu_util` against the fp64 oracle
    (the flat bound on unit-normal inputs at the ViT scale), pruned rows
    all-zero bytes, CLS rows the output rows (b, 0);
  * the three paths bitwise equal to each other (they run the same attention
    arithmetic), whatever bound was drawn.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import (CANARY, FLAT_TOL, UNIT_ROUNDOFF, bits, check_indexing,
                             check_padded, run_hip, say)

pytestmark = pytest.mark.gpu
N_CASES = 64


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def _draw(seed):
    g = np.random.default_rng(10_000 + seed)
    dtype = ["bf16", "f16", "f32"][int(g.integers(3))]
    N = int(g.choice([1, 7, 40, 64, 65, 130, 197, 257, 300, 577, 1100, 2048]))
    B = int(g.integers(1, 24 if N <= 300 else (8 if N <= 577 else 3)))
    H = int(g.integers(1, (9 if dtype != "f32" else 5) if N <= 577 else 3))
    scale = 0.125 if g.random() < 0.7 else float(g.choice([0.03, 0.2, -0.05, 0.0]))
    keep = torch.zeros((B, N), dtype=torch.uint8)
    tg = torch.Generator().manual_seed(20_000 + seed)
    for b in range(B):
        r = g.random()
        p_keep = 0.0 if r < 0.08 else (1.0 if r > 0.92 else float(g.random()))
        keep[b] = (torch.rand(N, generator=tg) < p_keep).to(torch.uint8)
        if g.random() < 0.8 and N > 0:
            keep[b, 0] = 1 if p_keep > 0 else 0
    w = workloads.custom(B, N, H, dtype, keep=keep, seed=30_000 + seed, scale=scale,
                         name=f"random_{seed}_{dtype}_B{B}_N{N}_H{H}_s{scale}")
    longest = max(w.kept_counts) if B else 0
    bound = int(g.choice([N, max(longest, 0), 4 * N])) if longest else N
    return w, max(bound, longest)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    import ragged_variable_length_amd as rv
    w, bound = _draw(seed)
    flat = w.scale == 0.125  # unit-normal inputs at the ViT scale
    say(f"{w.name}: bound {bound}, kept {w.total_kept}")
    ref = oracle.pipeline(w, want_absw=True)
    dev = torch.device("cuda")

    # three calls (pack, forward, unpack), through RaggedPipeline
    got = run_hip(w, max_seqlen=bound)
    check_indexing(w, got, ref)
    T = ref["total"]
    if T:
        o = oracle.widen(got["po"][:T], w.dtype).reshape(T, w.H, w.D)
        err = np.abs(o - ref["o64"])
        limit = FLAT_TOL[w.dtype] + 2.0 * UNIT_ROUNDOFF[w.dtype] * (np.abs(ref["o64"]) + ref["absw"])
        assert np.all(err <= limit), float((err / limit).max())
        if flat:
            assert float(err.max()) <= FLAT_TOL[w.dtype], float(err.max())

    # one launch
    q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
    out = torch.empty_like(q)
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev)
    for t in (out, cls):
        t.view(torch.uint8).fill_(CANARY)
    rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out, cls=cls, max_seqlen=bound)
    torch.cuda.synchronize()
    check_padded(w, out.cpu(), cls.cpu(), ref["o64"], ref["absw"], flat=flat)
    assert np.array_equal(bits(out.cpu()), bits(got["out"])), "fused != three calls"
    assert np.array_equal(bits(cls.cpu()), bits(got["cls"])), "fused CLS != three calls"
