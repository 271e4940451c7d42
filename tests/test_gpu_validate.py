"""The opt-in debug-validate mode on MI355X: the contract a call cannot check
from its host arguments alone (a max_seqlen or pad_len bound below the true
longest image, a cu_seqlens that does not start at 0, decreases, or disagrees
with the keep mask) is caught by reading the device data back, and the call
returns RATTN_ERR_INVALID_ARG with nothing launched: the outputs keep their
canary bytes.  With valid arguments the mode changes no output bit.  The
flat buffers have 2N rows of spare capacity, so that even a call the mode
failed to reject would stay inside them.
"""
import numpy as np
import pytest
import torch

import workloads
from tests._gpu_util import bits, say

pytestmark = pytest.mark.gpu
INVALID = 1
CANARY = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_variable_length_amd as rv
    rv.rattn_init()


@pytest.fixture
def validating():
    import ragged_variable_length_amd as rv
    prev = rv.rattn_set_validate(True)
    try:
        yield rv
    finally:
        rv.rattn_set_validate(prev)


def _canary_like(t):
    x = torch.empty(tuple(t.shape), dtype=t.dtype, device=t.device)
    x.view(torch.uint8).fill_(CANARY)
    return x


def _flat(w, dev):
    """Flat q, k, v (kept rows, then 2N zero rows of spare capacity) and the
    true cu_seqlens."""
    keep = w.keep != 0
    spare = torch.zeros((2 * w.N, w.H, w.D), dtype=w.q.dtype)
    flat = [torch.cat([t[keep], spare]).contiguous().to(dev) for t in (w.q, w.k, w.v)]
    cu = torch.zeros(w.B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(keep.sum(dim=1), 0).to(torch.int32)
    return flat, cu.to(dev)


def _status(fn, *a, **kw):
    import ragged_variable_length_amd as rv
    try:
        fn(*a, **kw)
    except rv.RattnError as e:
        return e.status
    return 0


def test_forward_bound_below_longest_image_is_rejected(validating):
    rv = validating
    dev = torch.device("cuda")
    w = workloads.deit_b_sweep(4, 0.5)
    flat, cu = _flat(w, dev)
    longest = max(w.kept_counts)
    say(f"validate: rattn_forward bound {longest - 1} < longest {longest}")
    o = _canary_like(flat[0])
    assert _status(rv.rattn_forward, *flat, o, cu, longest - 1, w.scale) == INVALID
    torch.cuda.synchronize()
    assert np.all(o.cpu().view(torch.uint8).numpy() == CANARY), "rejected call wrote output"
    # the exact bound and N pass, with the bits of a call outside the mode
    o_exact, o_n, o_off = _canary_like(o), _canary_like(o), _canary_like(o)
    rv.rattn_forward(*flat, o_exact, cu, longest, w.scale)
    rv.rattn_forward(*flat, o_n, cu, w.N, w.scale)
    rv.rattn_set_validate(False)
    rv.rattn_forward(*flat, o_off, cu, w.N, w.scale)
    rv.rattn_set_validate(True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_exact), bits(o_off)) and np.array_equal(bits(o_n), bits(o_off))


def test_forward_malformed_cu_seqlens_is_rejected(validating):
    rv = validating
    dev = torch.device("cuda")
    w = workloads.deit_b_sweep(2, 0.8)
    flat, cu = _flat(w, dev)
    o = _canary_like(flat[0])
    say("validate: cu_seqlens not starting at 0 / decreasing")
    bad0 = cu.clone()
    bad0[0] = 1
    assert _status(rv.rattn_forward, *flat, o, bad0, w.N, w.scale) == INVALID
    dec = cu.clone()
    dec[1] = cu[2] + 1
    assert _status(rv.rattn_forward, *flat, o, dec, w.N, w.scale) == INVALID
    torch.cuda.synchronize()
    assert np.all(o.cpu().view(torch.uint8).numpy() == CANARY)


def test_fused_bound_below_longest_image_is_rejected(validating):
    rv = validating
    dev = torch.device("cuda")
    w = workloads.deit_s()
    q, k, v, keep = (t.to(dev) for t in (w.q, w.k, w.v, w.keep))
    longest = max(w.kept_counts)
    out, cls = _canary_like(q), _canary_like(q[:, 0])
    say(f"validate: rattn_fused / rattn_fused_padded bound {longest - 1} < longest {longest}")
    assert _status(rv.rattn_fused, q, k, v, keep, w.scale, out_padded=out, cls=cls,
                   max_seqlen=longest - 1) == INVALID
    assert _status(rv.rattn_fused_padded, q, k, v, keep, w.scale, longest - 1,
                   out_padded=out, cls=cls) == INVALID
    torch.cuda.synchronize()
    assert np.all(out.cpu().view(torch.uint8).numpy() == CANARY)
    assert np.all(cls.cpu().view(torch.uint8).numpy() == CANARY)
    # valid bounds run, with the bits of a call outside the mode
    a, ca = _canary_like(q), _canary_like(q[:, 0])
    rv.rattn_fused(q, k, v, keep, w.scale, out_padded=a, cls=ca, max_seqlen=longest)
    p, cp = _canary_like(q), _canary_like(q[:, 0])
    rv.rattn_fused_padded(q, k, v, keep, w.scale, longest, out_padded=p, cls=cp)
    rv.rattn_set_validate(False)
    r, cr = _canary_like(q), _canary_like(q[:, 0])
    rv.rattn_fused(q, k, v, keep, w.scale, out_padded=r, cls=cr)
    rv.rattn_set_validate(True)
    torch.cuda.synchronize()
    for x, y in ((a, r), (ca, cr), (p, r), (cp, cr)):
        assert np.array_equal(bits(x), bits(y))


def test_unpack_and_repack_malformed_cu_seqlens_are_rejected(validating):
    """unpack: cu_seqlens one row longer than the mask says from image 1 on;
    repack: cu_seqlens not starting at 0."""
    rv = validating
    dev = torch.device("cuda")
    w = workloads.deit_b_sweep(4, 0.8)
    flat, cu = _flat(w, dev)
    keep = w.keep.to(dev)
    out = _canary_like(w.q.to(dev))
    say("validate: rattn_unpack with cu_seqlens off by one; rattn_repack with cu[0] = 1")
    off = cu.clone()
    off[2:] += 1  # image 1 one row longer than its mask says
    assert _status(rv.rattn_unpack, flat[0], keep, off, dst_padded=out) == INVALID
    torch.cuda.synchronize()
    assert np.all(out.cpu().view(torch.uint8).numpy() == CANARY)
    rv.rattn_unpack(flat[0], keep, cu, dst_padded=out)  # the right cu_seqlens passes
    keep2 = torch.ones(flat[0].shape[0], dtype=torch.uint8, device=dev)
    dst = _canary_like(flat[0])
    cu2 = torch.full_like(cu, -7)
    bad0 = cu.clone()
    bad0[0] = 1
    assert _status(rv.rattn_repack, [flat[0]], [dst], keep2, bad0, cu2) == INVALID
    torch.cuda.synchronize()
    assert np.all(dst.cpu().view(torch.uint8).numpy() == CANARY)
    assert cu2.cpu().tolist() == [-7] * (w.B + 1)
