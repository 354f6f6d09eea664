"""The allocation-free prompt pass (gdn_prefill_chunked_noalloc, for callers
that cannot allocate) against gdn_prefill_chunked with a caller workspace:
bit for bit the same outputs, states and tails, on two calls in a row (the
second smaller, so it runs over what the first left in the fixed array), and
a pass larger than the fixed array refused with its outputs untouched."""
import pytest
import torch

from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import announce

pytestmark = pytest.mark.gpu


def _both(b: gi.Batch):
    dev = "cuda"
    params = gdn.LayerParams.from_host(b.params, dev)
    seq_start, qkv, a, bb = b.row_start.to(dev), b.qkv.to(dev), b.a.to(dev), b.b.to(dev)
    res = []
    for noalloc in (False, True):
        tail, state = b.tail.to(dev).clone(), b.state.to(dev).clone()
        out = torch.full((b.rows, b.shape.hv, b.shape.dv), float("nan"), device=dev)
        if noalloc:
            gdn.prefill_chunked_noalloc(b.shape, params, seq_start, qkv, a, bb, tail, state, out,
                                        max_len=max(b.lengths()))
        else:
            ws = torch.empty(gdn.prefill_workspace_bytes(b.shape, b.n, b.rows), dtype=torch.uint8, device=dev)
            gdn.prefill_chunked(b.shape, params, seq_start, qkv, a, bb, tail, state, out, ws,
                                max_len=max(b.lengths()))
        torch.cuda.synchronize()
        res.append((out, state, tail))
    return res


def test_noalloc_prompt_pass_equals_workspace_pass_twice():
    first = gi.make_batch(gi.QWEN_27B, [700, 64, 1, 600], seed=120)
    assert gdn.prefill_workspace_bytes(first.shape, first.n, first.rows) <= gdn.PREFILL_SCRATCH_BYTES
    announce(f"noalloc prompt pass, 27B-like {first.lengths()}")
    (o1, s1, t1), (o2, s2, t2) = _both(first)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(t1, t2)
    second = gi.make_batch(gi.Shape(hk=2, hv=6, dk=128, dv=128), [130, 5, 64], seed=121, long_memory=True)
    announce(f"noalloc prompt pass, smaller, after the first {second.lengths()}")
    (o1, s1, t1), (o2, s2, t2) = _both(second)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(t1, t2)


def over_the_fixed_array(shape):
    """The fewest rows (a multiple of 64) of one prompt whose pass needs more
    workspace than the fixed array holds."""
    rows = 64
    while gdn.prefill_workspace_bytes(shape, 1, rows) <= gdn.PREFILL_SCRATCH_BYTES:
        rows += 64
    return rows


def test_noalloc_refuses_a_pass_over_the_fixed_array():
    shape = gi.QWEN_27B
    rows = over_the_fixed_array(shape)
    dev = "cuda"
    b = gi.make_batch(shape, [rows], seed=122)
    params = gdn.LayerParams.from_host(b.params, dev)
    tail, state = b.tail.to(dev), b.state.to(dev)
    out = torch.full((rows, shape.hv, shape.dv), float("nan"), device=dev)
    announce("noalloc prompt pass over the fixed array: refused")
    with pytest.raises(gdn.GdnError) as e:
        gdn.prefill_chunked_noalloc(shape, params, b.row_start.to(dev), b.qkv.to(dev), b.a.to(dev), b.b.to(dev),
                                    tail, state, out, max_len=rows)
    assert e.value.status == gdn.GDN_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert torch.equal(state.cpu(), b.state) and torch.equal(tail.cpu(), b.tail)
