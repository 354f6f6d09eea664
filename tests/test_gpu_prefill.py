"""GPU parity of the chunked prompt pass (bf16 matrix-core operands, fp32
state) against the oracle's row-by-row recurrence, within 2e-2."""
import numpy as np
import pytest
import torch

import oracle
from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import TOL_PREFILL, announce, bits16, bound_err, host_batch, max_rel_err, row_rel_err

pytestmark = pytest.mark.gpu

SMALL_27B_HEADS = gi.Shape(hk=2, hv=6, dk=128, dv=128)   # 3 value heads a key head


def run_prefill(b: gi.Batch, dev="cuda"):
    params = gdn.LayerParams.from_host(b.params, dev)
    seq_start = b.row_start.to(dev)
    qkv, a, bb = b.qkv.to(dev), b.a.to(dev), b.b.to(dev)
    tail, state = b.tail.to(dev).clone(), b.state.to(dev).clone()
    out = torch.full((b.rows, b.shape.hv, b.shape.dv), float("nan"), device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(b.shape, b.n, b.rows), dtype=torch.uint8, device=dev)
    gdn.prefill_chunked(b.shape, params, seq_start, qkv, a, bb, tail, state, out, ws,
                        max_len=max(b.lengths()))
    torch.cuda.synchronize()
    return out, tail, state


def oracle_prefill(b: gi.Batch):
    """(o, final state, final tail, o's magnitude, the final state's
    magnitude) of the row-by-row recurrence."""
    h = host_batch(b)
    return oracle.prefill(b.shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"], h["qkv"],
                          h["a"], h["b"], h["tail"], h["state"], mag=True)


def check(b: gi.Batch, out, tail, state, tol=TOL_PREFILL):
    """Every output element within tol of its magnitude (its row's step
    carried out on magnitudes); each final (prompt, head) state within tol of
    its largest element; conv tails bit for bit.  The final state's element-
    wise bound is printed only: bf16 operand errors accumulate over a
    prompt's chunks, while an element's magnitude covers only the last row's
    terms, so near-zero elements of a long-memory state have no meaningful
    element-wise bound at this precision."""
    o_ref, st_ref, tl_ref, o_mag, st_mag = oracle_prefill(b)
    o = out.cpu().numpy()
    st = state.cpu().numpy()
    e_o = bound_err(o, o_ref, o_mag)
    e_s = max_rel_err(st, st_ref, 2)
    e_se = bound_err(st, st_ref, st_mag)
    if b.rows:
        g = np.abs(o.astype(np.float64) - o_ref) / np.maximum(o_mag, 1e-30)
        per_row = g.reshape(b.rows, -1).max(1)
        print(f"o: bound err {e_o:.2e} (median row {np.median(per_row):.2e}, "
              f"per-row rel {row_rel_err(o, o_ref):.2e}); final state {e_s:.2e} "
              f"(element bound {e_se:.2e})")
    assert np.array_equal(bits16(tail), tl_ref), "conv tails must match bitwise"
    assert e_o <= tol, f"o: element-wise bound err {e_o:.3e}"
    assert e_s <= tol, f"final state: max rel err {e_s:.3e}"
    return e_o, e_s


@pytest.mark.parametrize("zero_state", [False, True])
def test_prefill_ragged_prompts(zero_state):
    lengths = [1, 2, 3, 63, 64, 65, 130, 200]
    b = gi.make_batch(SMALL_27B_HEADS, lengths, seed=31, zero_state=zero_state)
    announce(f"prefill ragged {lengths} zero_state={zero_state}")
    out, tail, state = run_prefill(b)
    e_o, e_s = check(b, out, tail, state)
    print(f"o err {e_o:.2e}, state err {e_s:.2e}")


def test_prefill_long_memory():
    lengths = [300, 17, 129]
    b = gi.make_batch(SMALL_27B_HEADS, lengths, seed=32, long_memory=True)
    announce(f"prefill long memory {lengths}")
    out, tail, state = run_prefill(b)
    e_o, e_s = check(b, out, tail, state)
    print(f"o err {e_o:.2e}, state err {e_s:.2e}")


def test_prefill_2b_layer():
    lengths = [96, 5, 160]
    b = gi.make_batch(gi.QWEN_2B, lengths, seed=33)
    announce(f"prefill 2B-like {lengths}")
    out, tail, state = run_prefill(b)
    check(b, out, tail, state)


@pytest.mark.parametrize("hk,hv", [(2, 4), (1, 4), (2, 12), (1, 5), (1, 8), (3, 24)])
def test_prefill_value_heads_per_key_head(hk, hv):
    """Two, four, five, six and eight value heads a key head (eight is the
    most the pass takes).  The per-chunk kernel places the r value heads of a
    (chunk, key head) as consecutive workgroups of one XCD, and the sweep the
    tile pairs of a (prompt, key head): odd r and r = 8 exercise both maps."""
    shape = gi.Shape(hk=hk, hv=hv, dk=128, dv=128)
    lengths = [70, 5, 130]
    b = gi.make_batch(shape, lengths, seed=35 + hv)
    announce(f"prefill hk={hk} hv={hv} {lengths}")
    out, tail, state = run_prefill(b)
    check(b, out, tail, state)


def test_prefill_many_prompts_with_equal_lengths():
    """40 prompts, several of equal length (the sweep orders prompts by length,
    ties by index) and some empty, so that the (prompt, key head) units fill
    the XCD slots unevenly."""
    rng = np.random.default_rng(41)
    lengths = [int(x) for x in rng.choice([0, 1, 7, 64, 65, 100, 150], size=40)]
    b = gi.make_batch(SMALL_27B_HEADS, lengths, seed=41)
    announce(f"prefill {len(lengths)} prompts {lengths}")
    out, tail, state = run_prefill(b)
    check(b, out, tail, state)


def test_prefill_more_than_256_prompts():
    """Past 256 prompts the sweep takes prompts in index order (no length
    ranking in LDS); short prompts, one key head, two value heads."""
    rng = np.random.default_rng(42)
    lengths = [int(x) for x in rng.integers(0, 9, size=260)]
    b = gi.make_batch(gi.Shape(hk=1, hv=2, dk=128, dv=128), lengths, seed=42)
    announce(f"prefill {len(lengths)} short prompts, {sum(lengths)} rows")
    out, tail, state = run_prefill(b)
    check(b, out, tail, state)


def test_prefill_with_empty_prompt():
    lengths = [70, 0, 33]
    b = gi.make_batch(SMALL_27B_HEADS, lengths, seed=34)
    announce(f"prefill with an empty prompt {lengths}")
    out, tail, state = run_prefill(b)
    check(b, out, tail, state)
    assert torch.equal(state[1].cpu(), b.state[1]) and torch.equal(tail[1].cpu(), b.tail[1])


def test_prefill_27b_four_prompts():
    shape, lengths, kw = gi.workload("prefill27b")
    b = gi.make_batch(shape, lengths, **kw)
    announce(f"prefill 27B-like {lengths} seed={kw['seed']}")
    out, tail, state = run_prefill(b)
    e_o, e_s = check(b, out, tail, state)
    print(f"27B prefill: o err {e_o:.2e}, state err {e_s:.2e}")


@pytest.mark.parametrize("zero_state", [True, False])
def test_prefill_27b_four_prompts_long_memory(zero_state):
    """The long-memory variant (A_log ~ U(-7, -4), alpha about 0.99) on the
    four prompts of the 27B-like pass: the state carried across all 74 chunks
    of the 4,722-row prompt, from zero and from a resumed state and tail."""
    shape, lengths, kw = gi.workload("prefill27b")
    kw = dict(kw, zero_state=zero_state)
    b = gi.make_batch(shape, lengths, long_memory=True, **kw)
    announce(f"prefill 27B-like long memory {lengths} zero_state={zero_state} seed={kw['seed']}")
    out, tail, state = run_prefill(b)
    e_o, e_s = check(b, out, tail, state)
    print(f"27B prefill, long memory: o err {e_o:.2e}, state err {e_s:.2e}")


def test_prefill_27b_resumed_state():
    """A non-zero initial state and tail (a resumed prompt) on the 27B-like layer."""
    shape = gi.QWEN_27B
    lengths = [700, 64, 1]
    b = gi.make_batch(shape, lengths, seed=35)
    announce(f"prefill 27B-like resumed {lengths}")
    out, tail, state = run_prefill(b)
    check(b, out, tail, state)


def test_prefill_then_steps_continue_the_stream():
    """A prompt pass followed by one-row steps gives what the recurrence gives
    for the whole sequence (the steps start from the prefill's state)."""
    shape = SMALL_27B_HEADS
    b = gi.make_batch(shape, [90, 4], seed=36)
    announce("prefill then steps")
    out, tail, state = run_prefill(b)
    # continue stream 0 with 3 more rows as steps
    more = gi.make_batch(shape, [3], seed=37)
    params = gdn.LayerParams.from_host(b.params, "cuda")
    o1 = torch.empty((1, shape.hv, shape.dv), device="cuda")
    tl, st = tail[0:1].clone(), state[0:1].clone()
    outs = []
    for t in range(3):
        gdn.conv_step(shape, params, more.qkv[t:t + 1].cuda(), more.a[t:t + 1].cuda(),
                      more.b[t:t + 1].cuda(), tl, st, o1)
        torch.cuda.synchronize()
        outs.append(o1[0].cpu().numpy().copy())
    # oracle: the whole 93-row sequence as one prompt
    whole = gi.Batch(shape=shape, params=b.params, row_start=torch.tensor([0, 93], dtype=torch.int32),
                     qkv=torch.cat([b.qkv[:90], more.qkv]), a=torch.cat([b.a[:90], more.a]),
                     b=torch.cat([b.b[:90], more.b]), tail=b.tail[0:1], state=b.state[0:1])
    o_ref, st_ref, tl_ref, o_mag, _ = oracle_prefill(whole)
    assert bound_err(np.stack(outs), o_ref[90:93], o_mag[90:93]) <= TOL_PREFILL
    assert max_rel_err(st.cpu().numpy(), st_ref, 2) <= TOL_PREFILL
    assert np.array_equal(bits16(tl), tl_ref)


@pytest.mark.parametrize("shape_name,length,cut", [("small27b", 700, 256), ("small27b", 130, 64),
                                                   ("27b", 4722, 4096)])
def test_prefill_resumed_at_chunk_grid_is_bitwise(shape_name, length, cut):
    """A prompt passed in two parts, cut at a chunk boundary, gives bit for bit
    what one pass gives: outputs, final state and conv tail (a pass resumed at
    a grid point computes what a fresh pass does: page "kept prompt states in
    host memory", commit notes on the family's snapshots and on resuming)."""
    shape = SMALL_27B_HEADS if shape_name == "small27b" else gi.QWEN_27B
    b = gi.make_batch(shape, [length], seed=38)
    announce(f"prefill resumed at a chunk boundary: {shape_name} {length} cut at {cut}")
    out, tail, state = run_prefill(b)
    first = gi.Batch(shape=shape, params=b.params, row_start=torch.tensor([0, cut], dtype=torch.int32),
                     qkv=b.qkv[:cut], a=b.a[:cut], b=b.b[:cut], tail=b.tail, state=b.state)
    o1, t1, s1 = run_prefill(first)
    second = gi.Batch(shape=shape, params=b.params,
                      row_start=torch.tensor([0, length - cut], dtype=torch.int32),
                      qkv=b.qkv[cut:], a=b.a[cut:], b=b.b[cut:], tail=t1.cpu(), state=s1.cpu())
    o2, t2, s2 = run_prefill(second)
    assert torch.equal(torch.cat([o1, o2]), out), "outputs differ from the single pass"
    assert torch.equal(s2, state), "final state differs from the single pass"
    assert torch.equal(t2, tail), "conv tail differs from the single pass"
