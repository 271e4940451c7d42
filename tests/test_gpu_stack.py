"""A stack of attention layers on one keep mask, on MI355X.

The integrated packing pipeline keeps the packed buffer across blocks: the
tokens are packed once, every layer attends on the flat buffers, and the
result is unpacked once.  Here each layer's output is the next layer's query
(k and v are those of the first layer), so the layers depend on each other.

* Every layer of the packed stack against the CPU oracle's attention on that
  layer's own inputs, read back from the GPU (the tolerances of `_gpu_util`),
  and the final unpack bit-exact against the oracle's unpack.
* The whole packed stack (rattn_pack once, rattn_forward per layer,
  rattn_unpack once) bitwise equal to rattn_fused applied per layer on the
  padded layout with the same chaining, at 12 layers, on the named workloads.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu_util import FLAT_TOL, UNIT_ROUNDOFF, bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def _resident(w):
    dev = torch.device("cuda")
    return [t.to(dev) for t in (w.q, w.k, w.v)] + [w.keep.to(dev)]


def packed_stack(w, layers, q, k, v, keep, readback=False):
    """rattn_pack once, `layers` rattn_forward calls (ping-pong between the
    flat q and o buffers), rattn_unpack of the last output.  With readback,
    also the flat (input q, output o) of every layer as CPU copies."""
    import ragged_variable_length_amd as rv
    pipe = rv.RaggedPipeline(w.B, w.N, w.H, q.dtype)
    pipe.pack(q, k, v, keep)
    T = w.total_kept
    qb, ob = pipe.pq, pipe.po
    per_layer = []
    for _ in range(layers):
        rv.rattn_forward(qb, pipe.pk, pipe.pv, ob, pipe.cu, w.N, w.scale)
        if readback:
            per_layer.append((qb[:T].cpu(), ob[:T].cpu()))
        qb, ob = ob, qb
    # qb now holds the last layer's output (pipe.po or pipe.pq, by parity)
    rv.rattn_unpack(qb, keep, pipe.cu, dst_padded=pipe.out, cls=pipe.cls)
    torch.cuda.synchronize()
    return pipe, qb[:T].cpu(), per_layer


def fused_stack(w, layers, q, k, v, keep):
    """rattn_fused per layer on the padded layout, each layer's padded output
    the next layer's query; the CLS rows from the last layer."""
    import ragged_variable_length_amd as rv
    a, b = torch.empty_like(q), torch.empty_like(q)
    cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=q.device)
    qb = q
    for layer in range(layers):
        rv.rattn_fused(qb, k, v, keep, w.scale, out_padded=a,
                       cls=cls if layer == layers - 1 else None)
        qb = a
        a, b = b, a
    torch.cuda.synchronize()
    return qb.cpu(), cls.cpu()


@pytest.mark.parametrize("name,layers", [("tiny", 3), ("deit_s", 3), ("deit_b_sweep", 4)])
def test_each_layer_matches_oracle(name, layers):
    w = {"tiny": workloads.tiny, "deit_s": workloads.deit_s,
         "deit_b_sweep": lambda: workloads.deit_b_sweep(4, 0.5)}[name]()
    say(f"stack {w.name}: {layers} layers, each against the oracle")
    q, k, v, keep = _resident(w)
    pipe, last, per_layer = packed_stack(w, layers, q, k, v, keep, readback=True)
    cu, _, T = oracle.scan(w.keep)
    assert pipe.cu.cpu().numpy().tolist() == cu.tolist()
    kf = oracle.widen(oracle.pack(w.k, w.keep), w.dtype)
    vf = oracle.widen(oracle.pack(w.v, w.keep), w.dtype)
    worst = 0.0
    for layer, (qin, o) in enumerate(per_layer):
        ref, absw = oracle.attention(oracle.widen(qin, w.dtype), kf, vf, cu, w.scale,
                                     want_absw=True)
        got = oracle.widen(o, w.dtype).reshape(ref.shape)
        assert np.all(np.isfinite(got)), f"layer {layer}: non-finite output"
        err = np.abs(got - ref)
        bound = 2.0 * UNIT_ROUNDOFF[w.dtype] * (np.abs(ref) + absw) + FLAT_TOL[w.dtype]
        assert float(err.max()) <= FLAT_TOL[w.dtype], (layer, float(err.max()))
        assert float((err / bound).max()) <= 1.0, layer
        worst = max(worst, float(err.max()))
    say(f"stack {w.name}: worst layer max|err|={worst:.3e}")
    dst, cls = oracle.unpack(last, w.keep, cu)
    assert np.array_equal(bits(pipe.out), dst.view(bits(pipe.out).dtype)), "unpack of the last layer"
    assert np.array_equal(bits(pipe.cls), cls.view(bits(pipe.cls).dtype)), "CLS of the last layer"


@pytest.mark.parametrize("maker", [workloads.tiny, workloads.deit_s, workloads.deit_b_384,
                                   workloads.large_batch],
                         ids=["tiny", "deit_s", "deit_b_384", "large_batch"])
def test_packed_stack_equals_fused_per_layer(maker):
    w = maker()
    layers = 12
    say(f"stack {w.name}: {layers} layers, packed once vs rattn_fused per layer")
    q, k, v, keep = _resident(w)
    pipe, _, _ = packed_stack(w, layers, q, k, v, keep)
    out_f, cls_f = fused_stack(w, layers, q, k, v, keep)
    assert np.array_equal(bits(pipe.out), bits(out_f)), "padded output"
    assert np.array_equal(bits(pipe.cls), bits(cls_f)), "CLS rows"
    assert np.all(np.isfinite(pipe.out.float().cpu().numpy()))
