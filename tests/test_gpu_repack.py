"""rattn_repack (a second pruning stage on the packed buffer) on MI355X,
against the CPU oracle: kept rows, the new cu_seqlens and the total
bit-exact, rows past the new total untouched.  The packed input buffers are
prepared on the host (the oracle's pack of a named workload), so the pack
kernel does not run here.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def _flat(w, t):
    p = oracle.pack(t, w.keep)
    if t.dtype == torch.bfloat16:
        return torch.from_numpy(p.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(p)


def _check(w, keep2, n_tensors=3, name=None):
    import ragged_variable_length_amd as rv
    name = name or w.name
    dev = torch.device("cuda")
    cu, _, T = oracle.scan(w.keep)
    flats = [_flat(w, t) for t in (w.q, w.k, w.v)[:n_tensors]]
    fill = torch.tensor(3.0, dtype=flats[0].dtype)
    srcs = [f.to(dev) for f in flats]
    dsts = [torch.full_like(f, 3.0) for f in srcs]
    k2 = torch.zeros(T + 16, dtype=torch.uint8)
    k2[:T] = keep2
    cu_d = torch.from_numpy(cu).to(dev)
    cu2 = torch.full_like(cu_d, -7)
    tot = torch.full((1,), -7, dtype=torch.int32, device=dev)
    say(f"{name}: B={w.B} T={T} kept again {int(keep2.sum())}, {n_tensors} tensor(s)")
    rv.rattn_repack(srcs, dsts, k2.to(dev), cu_d, cu2, tot)
    torch.cuda.synchronize()
    for f, d in zip(flats, dsts):
        ref, ref_cu = oracle.repack(f, keep2, cu)
        T2 = ref.shape[0]
        d = d.cpu()
        assert np.array_equal(bits(d[:T2]), bits(ref)), "re-packed rows"
        assert np.all(bits(d[T2:]) == bits(fill)), "rows past the new total written"
        assert cu2.cpu().numpy().tolist() == ref_cu.tolist(), "cu_seqlens"
        assert int(tot.item()) == T2, "total"


def _rand(T, p, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(T, generator=g) < p).to(torch.uint8)


def test_repack_deit_s_fp16():
    w = workloads.deit_s()
    _check(w, _rand(w.total_kept, 0.5, 1))


def test_repack_deit_b_384_bf16():
    w = workloads.deit_b_384()
    _check(w, _rand(w.total_kept, 0.6, 2), n_tensors=2)


def test_repack_large_batch_bf16():
    w = workloads.large_batch()
    _check(w, _rand(w.total_kept, 0.5, 3))


def test_repack_tiny_fp32():
    w = workloads.tiny()
    _check(w, _rand(w.total_kept, 0.3, 4), n_tensors=1)


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_repack_keep_none_and_all(p):
    w = workloads.deit_b_sweep(4, 0.25)
    _check(w, torch.full((w.total_kept,), int(p), dtype=torch.uint8), name=f"repack_p{p}")


def test_repack_empty_and_long_images():
    g = torch.Generator().manual_seed(5)
    lengths = [0, 1, 255, 256, 257, 0, 600, 33]
    keep = torch.zeros((len(lengths), 640), dtype=torch.uint8)
    for b, L in enumerate(lengths):
        keep[b, torch.randperm(640, generator=g)[:L]] = 1
    w = workloads.custom(len(lengths), 640, 2, "bf16", keep=keep, seed=6, name="repack_edges")
    _check(w, _rand(w.total_kept, 0.4, 7))


def test_repack_then_forward_matches_oracle_on_twice_pruned_tokens():
    """Two pruning stages then attention: rattn_repack's output fed to
    rattn_forward equals the oracle's attention on the tokens kept by both
    masks (within the bf16 tolerance)."""
    import ragged_variable_length_amd as rv
    w = workloads.deit_b_sweep(4, 0.25)
    dev = torch.device("cuda")
    cu, mx, T = oracle.scan(w.keep)
    keep2 = _rand(T, 0.5, 8)
    srcs = [_flat(w, t).to(dev) for t in (w.q, w.k, w.v)]
    dsts = [torch.empty_like(s_) for s_ in srcs]
    k2 = torch.zeros(T + 16, dtype=torch.uint8)
    k2[:T] = keep2
    cu2 = torch.empty(w.B + 1, dtype=torch.int32, device=dev)
    say("repack then forward")
    rv.rattn_repack(srcs, dsts, k2.to(dev), torch.from_numpy(cu).to(dev), cu2)
    o = torch.empty_like(dsts[0])
    rv.rattn_forward(*dsts, o, cu2, mx, w.scale)   # the old bound stays valid
    torch.cuda.synchronize()
    both = w.keep.clone()
    both[w.keep != 0] = keep2
    w2 = workloads.Workload("twice", w.B, w.N, w.H, w.D, w.dtype, both, w.q, w.k, w.v,
                            scale=w.scale)
    ref = oracle.pipeline(w2)
    T2 = ref["total"]
    assert cu2.cpu().numpy().tolist() == ref["cu"].tolist()
    got = oracle.widen(o.cpu()[:T2], "bf16").reshape(T2, w.H, w.D)
    err = float(np.abs(got - ref["o64"]).max())
    say(f"twice pruned: T2={T2} max|err|={err:.3e}")
    assert err <= 1e-2
