"""Several host threads calling the library at once, each on its own stream,
on MI355X.  The library keeps no device state between calls, so calls on
different streams may overlap freely: every result must be bit for bit the
one the same call gives alone on one stream (that result is itself checked
against the oracle by the other GPU tests).
"""
import threading

import numpy as np
import pytest
import torch

import workloads
from tests._gpu_util import bits, say

pytestmark = pytest.mark.gpu
THREADS = 4
ITERS = 20


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


def test_threads_on_separate_streams():
    import ragged_variable_length_amd as rv
    dev = torch.device("cuda")
    jobs = []
    for i in range(THREADS):
        w = workloads.deit_s(seed=500 + i) if i % 2 == 0 else workloads.deit_b_sweep(4, 0.5, seed=600 + i)
        q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
        out = torch.empty_like(q)
        cls = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev)
        pipe = rv.RaggedPipeline(w.B, w.N, w.H, q.dtype, device=dev)
        jobs.append(dict(w=w, q=q, k=k, v=v, keep=keep, out=out, cls=cls, pipe=pipe,
                         stream=torch.cuda.Stream()))
    # each job alone, in turn, on the default stream
    for j in jobs:
        rv.rattn_fused(j["q"], j["k"], j["v"], j["keep"], j["w"].scale, out_padded=j["out"], cls=j["cls"])
        j["pipe"].run(j["q"], j["k"], j["v"], j["keep"], j["w"].scale)
        torch.cuda.synchronize()
        j["ref"] = [t.clone() for t in (j["out"], j["cls"], j["pipe"].out, j["pipe"].cls)]

    errors = []

    def worker(j):
        try:
            plan = rv.FusedPlan(j["q"], j["k"], j["v"], j["keep"], j["w"].scale,
                                out_padded=j["out"], cls=j["cls"], stream=j["stream"])
            for _ in range(ITERS):
                plan.run()
                j["pipe"].run(j["q"], j["k"], j["v"], j["keep"], j["w"].scale, stream=j["stream"])
            j["stream"].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    for j in jobs:
        for t in (j["out"], j["cls"], j["pipe"].out, j["pipe"].cls):
            t.view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    say(f"{THREADS} threads x {ITERS} fused + three-call steps on separate streams")
    threads = [threading.Thread(target=worker, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, j in enumerate(jobs):
        got = (j["out"], j["cls"], j["pipe"].out, j["pipe"].cls)
        for name, g, r in zip(("fused out", "fused CLS", "three-call out", "three-call CLS"), got, j["ref"]):
            assert np.array_equal(bits(g), bits(r)), f"job {i}: {name}"
