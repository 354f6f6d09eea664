"""HIP-graph capture of the launch-bound calls (one-row steps, a 2B-like
verify window, a logged verify round with its commit by replay, a prompt
pass): captured launches replayed several times give, bit for bit, what the
same calls give run eagerly, and every replay matches the oracle within the
row kernels' (or the prompt pass's) tolerance.  Every count the kernels need
is read on the device, so one captured graph serves any window layout of the
same sizes (captured forwards: page "perf(qwen3_5 cuda): deliver the first
token before drafting", commit note on captured forwards and device-read
counts)."""
import numpy as np
import pytest
import torch

import oracle
from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import (TOL_PREFILL, TOL_ROWS, announce, bits16, bound_err, device_batch, host_batch,
                      max_rel_err, oracle_rows)

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
    # the oracle: each stream's rows run `replays` times over, as one window
    rep_rows = [s * nsteps + k for s in range(n) for _ in range(replays) for k in range(nsteps)]
    seq = gi.Batch(shape=shape, params=b.params,
                   row_start=gi.starts_from_lengths([nsteps * replays] * n),
                   qkv=b.qkv[rep_rows], a=b.a[rep_rows], b=b.b[rep_rows], tail=b.tail, state=b.state)
    ref = oracle_rows(seq)
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
            r = [s * nsteps * replays + rep * nsteps + k for s in range(n)]
            assert bound_err(outs_g[k].cpu().numpy(), ref["o"][r], ref["o_mag"][r]) <= TOL_ROWS, (rep, k)
        assert torch.equal(state_g, state_e), f"replay {rep}: states differ"
        assert torch.equal(tail_g, tail_e), f"replay {rep}: tails differ"
        last = [s * nsteps * replays + (rep + 1) * nsteps - 1 for s in range(n)]
        assert max_rel_err(state_g.cpu().numpy(), ref["snap32"][last], 2) <= TOL_ROWS, rep
        assert np.array_equal(bits16(tail_g), ref["tail_snap"][last]), rep


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
        part = gi.Batch(shape=shape, params=b.params, row_start=torch.tensor([0, length], dtype=torch.int32),
                        qkv=b.qkv[:length], a=b.a[:length], b=b.b[:length], tail=b.tail, state=b.state)
        ref = oracle_rows(part)
        assert bound_err(out_g[:length].cpu().numpy(), ref["o"], ref["o_mag"]) <= TOL_ROWS, length
        assert max_rel_err(ss_g[:length].cpu().numpy(), ref["snap32"], 2) <= TOL_ROWS, length
        assert np.array_equal(bits16(ts_g[:length]), ref["tail_snap"]), length


def test_captured_logged_verify_round_equals_eager():
    """A logged verify pass followed by the commit by replay, captured as one
    graph: every replay (with new accepted rows written into the same device
    buffer between replays) equals the eager calls bit for bit."""
    shape = gi.Shape(hk=2, hv=6, dk=128, dv=128)
    lengths = [16, 7, 12]
    b = gi.make_batch(shape, lengths, seed=42)
    announce(f"graph capture: logged verify {lengths} + commit by replay")
    d = device_batch(b)
    R = b.rows
    rs = b.row_start.tolist()

    def bufs():
        return (torch.empty((R, shape.hv, shape.dv), device="cuda"),
                torch.empty((R, shape.hv), device="cuda"),
                torch.empty((R, shape.hv, shape.dv), device="cuda"),
                torch.empty((R, shape.hk, shape.dk), device="cuda"))

    out_g, la_g, ld_g, lk_g = bufs()
    out_e, la_e, ld_e, lk_e = bufs()
    accept = torch.tensor([rs[1] - 1, rs[1] + 3, -1], dtype=torch.int32, device="cuda")
    tail0, state0 = d["tail"].clone(), d["state"].clone()
    tail_g, state_g = tail0.clone(), state0.clone()

    def round_(tail, state, out, la, ld, lk):
        gdn.recur_log(shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"], tail, state, out, la, ld,
                      lk, max_rows=16)
        gdn.commit_replay(shape, d["row_start"], accept, d["qkv"], la, ld, lk, tail, state, max_rows=16)

    round_(tail0.clone(), state0.clone(), out_g, la_g, ld_g, lk_g)   # first-call set-up, outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_(tail_g, state_g, out_g, la_g, ld_g, lk_g)
    torch.cuda.synchronize()
    tail_e, state_e = tail0.clone(), state0.clone()
    h = host_batch(b)
    tail_o, state_o = h["tail"], h["state"]   # the oracle's stream, carried across rounds
    for rep, acc in enumerate(([rs[1] - 1, rs[1] + 3, -1], [rs[0] + 5, -1, rs[3] - 1], [rs[0], rs[2] - 1, rs[2]])):
        accept.copy_(torch.tensor(acc, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        round_(tail_e, state_e, out_e, la_e, ld_e, lk_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: o differs"
        assert torch.equal(ld_g, ld_e) and torch.equal(lk_g, lk_e) and torch.equal(la_g, la_e), f"replay {rep}: log"
        assert torch.equal(state_g, state_e), f"replay {rep}: states differ"
        assert torch.equal(tail_g, tail_e), f"replay {rep}: tails differ"
        ref = oracle.window(shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"], h["qkv"], h["a"],
                            h["b"], tail_o, state_o, snap64=False, tail_snap=False, log=True, mag=True)
        assert bound_err(out_g.cpu().numpy(), ref["o"], ref["o_mag"]) <= TOL_ROWS, rep
        assert bound_err(ld_g.cpu().numpy(), ref["log_delta"], ref["log_delta_mag"]) <= TOL_ROWS, rep
        assert max_rel_err(la_g.cpu().numpy(), ref["log_alpha"], 2) <= TOL_ROWS, rep
        assert max_rel_err(lk_g.cpu().numpy(), ref["log_key"], 2) <= TOL_ROWS, rep
        tail_o, state_o = oracle.commit_replay(shape, h["row_start"], None, np.array(acc, np.int32), h["qkv"],
                                               ref["log_alpha"], ref["log_delta"], ref["log_key"], tail_o,
                                               state_o)
        assert max_rel_err(state_g.cpu().numpy(), state_o, 2) <= TOL_ROWS, rep
        assert np.array_equal(bits16(tail_g), tail_o), rep


def test_captured_prompt_pass_equals_eager():
    """The chunked prompt pass (two launches, no host work between them)
    captured and replayed several times, each replay from the same initial
    state, equals the eager pass bit for bit."""
    shape = gi.Shape(hk=2, hv=6, dk=128, dv=128)
    lengths = [200, 64, 3, 130]
    b = gi.make_batch(shape, lengths, seed=43)
    announce(f"graph capture: prompt pass {lengths}")
    d = device_batch(b)
    ws = torch.empty(gdn.prefill_workspace_bytes(shape, b.n, b.rows), dtype=torch.uint8, device="cuda")
    out_g = torch.empty((b.rows, shape.hv, shape.dv), device="cuda")
    out_e = torch.empty_like(out_g)
    tail0, state0 = d["tail"].clone(), d["state"].clone()
    tail_g, state_g = tail0.clone(), state0.clone()

    def pass_(tail, state, out):
        gdn.prefill_chunked(shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"], tail, state, out, ws,
                            max_len=max(lengths))

    pass_(tail0.clone(), state0.clone(), out_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pass_(tail_g, state_g, out_g)
    torch.cuda.synchronize()
    tail_e, state_e = tail0.clone(), state0.clone()
    pass_(tail_e, state_e, out_e)
    torch.cuda.synchronize()
    h = host_batch(b)
    o_ref, st_ref, tl_ref, o_mag, _ = oracle.prefill(shape, h["conv_w"], h["a_log"], h["dt_bias"],
                                                     h["row_start"], h["qkv"], h["a"], h["b"], h["tail"],
                                                     h["state"], mag=True)
    for rep in range(3):
        tail_g.copy_(tail0)
        state_g.copy_(state0)
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: o differs"
        assert torch.equal(state_g, state_e), f"replay {rep}: states differ"
        assert torch.equal(tail_g, tail_e), f"replay {rep}: tails differ"
        assert bound_err(out_g.cpu().numpy(), o_ref, o_mag) <= TOL_PREFILL, rep
        assert max_rel_err(state_g.cpu().numpy(), st_ref, 2) <= TOL_PREFILL, rep
        assert np.array_equal(bits16(tail_g), tl_ref), rep
