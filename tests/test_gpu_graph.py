"""The product path captured into a graph and replayed, on MI355X.

`FusedPlan.run()` (one launch) and `RaggedPipeline.run()` (pack -> forward ->
unpack) are captured once into a torch CUDA graph on a side stream and
replayed several times, on the DeiT-S, 384-px and tiny float32 workloads (the
last runs the float32 core that splits keys over wavefronts).  Between replays the outputs are overwritten with a
canary by ordinary eager kernels and the program synchronises, so a replay
that skipped or repeated part of its work would leave canary bytes or stale
values.  Every replay must give the bits of the eager call on the same
inputs (the eager call is itself checked against the oracle by the other
GPU tests).  A last replay after the inputs were overwritten in place must
give the eager result for the new inputs: the graph reads the live buffers,
not a copy taken at capture.
"""
import numpy as np
import pytest
import torch

import workloads
from tests._gpu_util import bits, say

pytestmark = pytest.mark.gpu
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()
    rv.rattn_set_validate(0)  # the validate mode synchronises, which a capture forbids


def _resident(w):
    dev = torch.device("cuda")
    return [t.to(dev).contiguous() for t in (w.q, w.k, w.v, w.keep)]


def _new_inputs(w, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(w.q.shape, generator=g).to(w.q.dtype) for _ in range(3)]


@pytest.mark.parametrize("name", ["deit_s", "tiny"])
def test_graph_replay_fused(name):
    import ragged_variable_length_amd as rv
    w = workloads.by_name(name)
    q, k, v, keep = _resident(w)
    out = torch.empty_like(q)
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=q.device)
    s = torch.cuda.Stream()
    plan = rv.FusedPlan(q, k, v, keep, w.scale, out_padded=out, cls=cls, stream=s)
    plan.run()
    s.synchronize()
    ref_out, ref_cls = out.clone(), cls.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        plan.run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        say(f"{name}: fused graph replay {rep}")
        out.view(torch.uint8).fill_(0xA5)
        cls.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(ref_out)), f"replay {rep}: output"
        assert np.array_equal(bits(cls), bits(ref_cls)), f"replay {rep}: CLS"

    # new inputs in the same buffers
    for t, n in zip((q, k, v), _new_inputs(w, 907)):
        t.copy_(n)
    out2 = torch.empty_like(q)
    cls2 = torch.empty_like(cls)
    rv.rattn_fused(q, k, v, keep, w.scale, out_padded=out2, cls=cls2)
    torch.cuda.synchronize()
    assert not np.array_equal(bits(out2), bits(ref_out))
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(out2)), "replay after new inputs: output"
    assert np.array_equal(bits(cls), bits(cls2)), "replay after new inputs: CLS"


@pytest.mark.parametrize("name", ["deit_s", "deit_b_384", "tiny"])
def test_graph_replay_three_calls(name):
    import ragged_variable_length_amd as rv
    w = workloads.by_name(name)
    q, k, v, keep = _resident(w)
    s = torch.cuda.Stream()
    pipe = rv.RaggedPipeline(w.B, w.N, w.H, q.dtype, device=q.device)
    with torch.cuda.stream(s):
        pipe.run(q, k, v, keep, w.scale)
    s.synchronize()
    ref = {n: getattr(pipe, n).clone() for n in ("cu", "po", "out", "cls")}
    T = int(ref["cu"][-1])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        pipe.run(q, k, v, keep, w.scale)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        say(f"{name}: three-call graph replay {rep}")
        for n in ("po", "out", "cls"):
            getattr(pipe, n).view(torch.uint8).fill_(0x5A)
        pipe.cu.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(pipe.cu), bits(ref["cu"])), f"replay {rep}: cu_seqlens"
        assert np.array_equal(bits(pipe.po[:T]), bits(ref["po"][:T])), f"replay {rep}: flat output"
        assert np.array_equal(bits(pipe.out), bits(ref["out"])), f"replay {rep}: output"
        assert np.array_equal(bits(pipe.cls), bits(ref["cls"])), f"replay {rep}: CLS"

    for t, n in zip((q, k, v), _new_inputs(w, 911)):
        t.copy_(n)
    fresh = rv.RaggedPipeline(w.B, w.N, w.H, q.dtype, device=q.device)
    fresh.run(q, k, v, keep, w.scale)
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(pipe.out), bits(fresh.out)), "replay after new inputs: output"
    assert np.array_equal(bits(pipe.cls), bits(fresh.cls)), "replay after new inputs: CLS"
