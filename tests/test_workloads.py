"""The seeded synthetic workloads have the stated shapes and mask rules (CPU)."""
import json
import os

import pytest
import torch

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_shape_and_mask():
    w = workloads.tiny()
    assert (w.B, w.N, w.H, w.D, w.dtype) == (4, 197, 3, 64, "f32")
    assert w.q.dtype == torch.float32 and w.q.shape == (4, 197, 3, 64)
    assert torch.all(w.keep[:, 0] == 1)
    frac = w.keep[:, 1:].float().mean().item()
    assert 0.4 < frac < 0.6  # Bernoulli(0.5) over 784 patches


def test_deit_s_counts():
    w = workloads.deit_s()
    assert (w.B, w.N, w.H, w.dtype) == (32, 197, 6, "f16")
    assert w.q.dtype == torch.float16
    c = w.kept_counts
    assert all(30 <= x <= 48 for x in c)
    assert torch.all(w.keep[:, 0] == 1)


def test_sweep_points_and_counts():
    gold = json.load(open(os.path.join(GOLD, "pages_numbers.json")))
    item = gold["items"][0]
    # 80 % pruning of the 196 patches + CLS lands within one token of the pages' ~39
    assert abs(workloads.sweep_kept_count(item["prune_rate"]) - item["tokens_after_about"]) <= 1
    assert [workloads.sweep_kept_count(p) for p in workloads.SWEEP_P] == [197, 148, 99, 40]
    for B, p, exact in workloads.sweep_points():
        w = workloads.deit_b_sweep(B, p, exact_unpruned=exact)
        assert (w.B, w.N, w.H, w.dtype) == (B, 197, 12, "bf16")
        k0 = workloads.sweep_kept_count(p)
        for c in w.kept_counts:
            if exact:
                assert c == 197
            else:
                assert max(1, int(0.9 * k0) - 1) <= c <= min(197, int(1.1 * k0) + 1)


def test_deit_b_384_outliers():
    w = workloads.deit_b_384(B=4)  # small B keeps the CPU test quick
    assert (w.N, w.H, w.dtype) == (577, 12, "bf16")
    assert all(230 <= c <= 347 for c in w.kept_counts)
    norms = w.q.float().reshape(4 * 577, -1).norm(dim=1)
    big = (norms > 4 * norms.median()).sum().item()
    assert big == w.meta["outlier_rows"] == round(0.01 * 4 * 577)


def test_large_batch_threshold_mask():
    w = workloads.large_batch(B=16)
    assert (w.N, w.H, w.dtype) == (197, 6, "bf16")
    assert torch.all(w.keep[:, 0] == 1)
    frac = (w.keep[:, 1:].float().mean(dim=1))
    # per-image keep fraction is 1 - quantile level, level in [0.2, 0.8]
    assert torch.all(frac >= 0.19) and torch.all(frac <= 0.81)


@pytest.mark.parametrize("name", ["tiny", "deit_s"])
def test_seeded_determinism(name):
    a, b = workloads.by_name(name), workloads.by_name(name)
    assert torch.equal(a.keep, b.keep)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    c = workloads.by_name(name, seed=99)
    assert not torch.equal(a.q, c.q)
