"""HIP-graph capture of the launch-bound calls (one-row steps, a 2B-like
verify window): captured launches replayed several times give, bit for bit,
what the same calls give run eagerly.  Every count the kernels need is read on
the device, so one captured graph serves any window layout of the same sizes
(captured forwards: page "perf(qwen3_5 cuda): deliver the first token before
drafting", commit note on captured forwards and device-read counts)."""
import pytest
import torch

from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import announce, device_batch

pytestmark = pytest.mark.gpu


def test_captured_steps_equal_eager_steps():
    shape = gi.SMALL
    n, nsteps, replays = 3, 4, 3
    b = gi.make_batch(shape, [nsteps] * n, seed=40)
    announce(f"graph capture: {nsteps} one-row steps of {n} streams, {replays} replays")
    params = gdn.LayerParams.from_host(b.params, "cuda")
    # rows[k] = the k-th row of every stream
    rows = [(b.qkv[k::nsteps].contiguous().cuda(), b.a[k::nsteps].contiguous().cuda(),
             b.b[k::nsteps].contiguous().cuda()) for k in range(nsteps)]
    tail_g, state_g = b.tail.cuda(), b.state.cuda()
    tail_e, state_e = b.tail.cuda(), b.state.cuda()
    outs_g = [torch.empty((n, shape.hv, shape.dv), device="cuda") for _ in range(nsteps)]
    out_e = torch.empty((n, shape.hv, shape.dv), device="cuda")

    def steps(tl, st, outs):
        for k in range(nsteps):
            q, a, bb = rows[k]
            gdn.conv_step(shape, params, q, a, bb, tl, st, outs[k])

    # warm-up outside the capture (first-call set-up happens here), on copies
    steps(tail_e.clone(), state_e.clone(), outs_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(tail_g, state_g, outs_g)
    torch.cuda.synchronize()
    # capture does not run the work: the state is still the initial one
    assert torch.equal(state_g, state_e)
    for rep in range(replays):
        g.replay()
        torch.cuda.synchronize()
        for k in range(nsteps):
            q, a, bb = rows[k]
            gdn.conv_step(shape, params, q, a, bb, tail_e, state_e, out_e)
            torch.cuda.synchronize()
            assert torch.equal(outs_g[k], out_e), f"replay {rep}, step {k}: outputs differ"
        assert torch.equal(state_g, state_e), f"replay {rep}: states differ"
        assert torch.equal(tail_g, tail_e), f"replay {rep}: tails differ"


def test_captured_window_equals_eager_window_for_new_layouts():
    shape = gi.QWEN_2B
    b = gi.make_batch(shape, [16], seed=41)
    announce("graph capture: 2B-like 16-row window, replayed with new row layouts")
    d = device_batch(b)
    R = b.rows
    out_g = torch.empty((R, shape.hv, shape.dv), device="cuda")
    ts_g = torch.empty((R, 3, shape.channels), dtype=torch.bfloat16, device="cuda")
    ss_g = torch.empty((R, shape.hv, shape.dk, shape.dv), device="cuda")
    out_e, ts_e, ss_e = torch.empty_like(out_g), torch.empty_like(ts_g), torch.empty_like(ss_g)
    row_start = d["row_start"].clone()

    def call(rs, out, ts, ss):
        gdn.recur_window(shape, d["params"], rs, d["qkv"], d["a"], d["b"], d["tail"], d["state"], out, ts, ss,
                         max_rows=16)

    call(row_start, out_e, ts_e, ss_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(row_start, out_g, ts_g, ss_g)
    # the captured graph reads the layout on the device: a shorter window
    # written into the same buffer is what the replays compute
    for length in (16, 9, 1):
        row_start.copy_(torch.tensor([0, length], dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(row_start, out_e, ts_e, ss_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g[:length], out_e[:length]), f"window of {length}: outputs differ"
        assert torch.equal(ss_g[:length], ss_e[:length]), f"window of {length}: snapshots differ"
        assert torch.equal(ts_g[:length], ts_e[:length]), f"window of {length}: tail snapshots differ"
