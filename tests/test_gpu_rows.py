"""GPU parity of the row kernels (step, window, tree, commit) against the oracle,
and the bitwise invariants the pages require: a window's rows equal one-row
steps, a tree's paths equal chains, a stream's results do not depend on what
else is packed with it.  Outputs start poisoned (NaN), so an element the
kernels fail to write shows up as a failure."""
import numpy as np
import pytest
import torch

from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import (TOL_ROWS, announce, bits16, bits32, bound_err, device_batch, max_rel_err,
                      oracle_rows, poisoned_outputs, row_rel_err)

pytestmark = pytest.mark.gpu


def run_window(b: gi.Batch, tree=False, max_rows=16, d=None):
    d = d or device_batch(b)
    out, tsnap, ssnap = poisoned_outputs(b.shape, b.rows)
    if tree:
        gdn.recur_tree(b.shape, d["params"], d["row_start"], d["parent"], d["qkv"], d["a"], d["b"],
                       d["tail"], d["state"], out, tsnap, ssnap, max_rows=max_rows)
    else:
        gdn.recur_window(b.shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"],
                         d["tail"], d["state"], out, tsnap, ssnap, max_rows=max_rows)
    torch.cuda.synchronize()
    return out, tsnap, ssnap


def check_against_oracle(b: gi.Batch, out, tsnap, ssnap, tree=False, tol=TOL_ROWS):
    """o and every state snapshot element within tol of its magnitude; each
    (row, head) state snapshot also within tol of its largest element; tail
    snapshots bit for bit."""
    ref = oracle_rows(b, tree=tree, snap_mag=True)
    o = out.cpu().numpy()
    s = ssnap.cpu().numpy()
    e_o = bound_err(o, ref["o"], ref["o_mag"])
    e_s = max_rel_err(s, ref["snap32"], 2)
    e_se = bound_err(s, ref["snap32"], ref["snap_mag"])
    print(f"o: bound err {e_o:.2e} (per-row rel {row_rel_err(o, ref['o']):.2e}); "
          f"snapshots: {e_s:.2e} (element bound {e_se:.2e})")
    assert e_o <= tol, f"o: element-wise bound err {e_o:.3e}"
    assert e_s <= tol, f"state snapshots: max rel err {e_s:.3e}"
    assert e_se <= tol, f"state snapshots: element-wise bound err {e_se:.3e}"
    assert np.array_equal(bits16(tsnap), ref["tail_snap"]), "tail snapshots must match bitwise"
    return e_o, e_s


CASES = {
    "step-small": ("step", {}),
    "window-2b": ("window2b", {}),
    "ragged-27b": ("ragged27b", {}),
    "verify-27b-16x16": ("verify27b", {}),
}


@pytest.mark.parametrize("case", list(CASES))
def test_window_matches_oracle(case):
    name, _ = CASES[case]
    shape, lengths, kw = gi.workload(name)
    b = gi.make_batch(shape, lengths, **kw)
    announce(f"recur_window {case} lengths={lengths} seed={kw['seed']}")
    out, tsnap, ssnap = run_window(b)
    e_o, e_s = check_against_oracle(b, out, tsnap, ssnap)
    print(f"{case}: o err {e_o:.2e}, snapshot err {e_s:.2e}")


@pytest.mark.parametrize("name", ["window2b", "verify27b", "ragged27b", "tree27b"])
def test_long_memory_full_size(name):
    """The long-memory variant (A_log ~ U(-7, -4): alpha about 0.99, so the
    initial state and every row's write persist through the whole window) at
    the workloads' full sizes."""
    shape, lengths, kw = gi.workload(name)
    tree = kw.get("tree", False)
    b = gi.make_batch(shape, lengths, long_memory=True, **kw)
    announce(f"long memory {name} lengths={lengths} seed={kw['seed']}")
    out, tsnap, ssnap = run_window(b, tree=tree)
    check_against_oracle(b, out, tsnap, ssnap, tree=tree)


MIXED = {"dk64-dv128": gi.Shape(hk=2, hv=6, dk=64, dv=128),
         "dk128-dv64": gi.Shape(hk=2, hv=4, dk=128, dv=64)}


def test_narrow_workgroups_stage_in_several_batches():
    """A launch of more than 256 workgroups gets no helper waves: with one
    value head of dv = 64 a key head a workgroup has 128 threads, and its 19
    staged rows of 320 channels (and 320 conv weights) take three batches of
    loads.  Windows and trees against the oracle."""
    shape = gi.Shape(hk=16, hv=16, dk=128, dv=64)
    lengths = [16] * 14 + [9, 1, 16, 5, 12, 16]
    for tree, seed in ((False, 95), (True, 96)):
        b = gi.make_batch(shape, lengths, seed=seed, tree=tree)
        announce(f"{'recur_tree' if tree else 'recur_window'} 20 streams hk=hv=16 dv=64 seed={seed}")
        out, tsnap, ssnap = run_window(b, tree=tree)
        check_against_oracle(b, out, tsnap, ssnap, tree=tree)


@pytest.mark.parametrize("hk,hv,d,n", [(1, 8, 64, 17), (1, 5, 128, 26), (2, 16, 128, 9)])
def test_many_value_heads_per_key_head(hk, hv, d, n):
    """Eight value heads a key head at d = 64 (a workgroup of 16 waves, the
    most one holds, on all eight heads), five at d = 128 (no divisor but one
    fits a workgroup) and eight at d = 128 (four heads a workgroup, two
    workgroups a key head), with enough streams that the launch keeps whole
    heads in a workgroup: windows and trees against the oracle."""
    shape = gi.Shape(hk=hk, hv=hv, dk=d, dv=d)
    lengths = ([16, 3, 11, 16, 1] * 6)[:n]
    for tree, seed in ((False, 120 + hv), (True, 130 + hv)):
        b = gi.make_batch(shape, lengths, seed=seed, tree=tree)
        announce(f"{'recur_tree' if tree else 'recur_window'} hk={hk} hv={hv} d={d} seed={seed}")
        out, tsnap, ssnap = run_window(b, tree=tree)
        check_against_oracle(b, out, tsnap, ssnap, tree=tree)


@pytest.mark.parametrize("geom", list(MIXED))
def test_mixed_head_sizes(geom):
    """dk != dv (both sizes the geometry allows): ragged windows and draft
    trees against the oracle, and a window's rows against one-row steps bit
    for bit."""
    shape = MIXED[geom]
    lengths = [16, 1, 7, 12, 3]
    b = gi.make_batch(shape, lengths, seed=93)
    announce(f"recur_window {geom} lengths={lengths} seed=93")
    d = device_batch(b)
    out, tsnap, ssnap = run_window(b, d=d)
    check_against_oracle(b, out, tsnap, ssnap)
    bt = gi.make_batch(shape, lengths, seed=94, tree=True)
    announce(f"recur_tree {geom} lengths={lengths} seed=94")
    o2, t2, s2 = run_window(bt, tree=True)
    check_against_oracle(bt, o2, t2, s2, tree=True)
    announce(f"window vs steps {geom}")
    tail, state = d["tail"][0:1].clone(), d["state"][0:1].clone()
    o1 = torch.empty((1, shape.hv, shape.dv), dtype=torch.float32, device="cuda")
    for r in range(lengths[0]):
        gdn.conv_step(shape, d["params"], d["qkv"][r:r + 1], d["a"][r:r + 1], d["b"][r:r + 1], tail, state, o1)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(o1[0]), bits32(out[r])), (geom, r, "o")
        assert np.array_equal(bits32(state[0]), bits32(ssnap[r])), (geom, r, "state")
        assert np.array_equal(bits16(tail[0]), bits16(tsnap[r])), (geom, r, "tail")


def test_tree_matches_oracle_and_commit():
    shape, lengths, kw = gi.workload("tree27b")
    b = gi.make_batch(shape, lengths, **kw)
    announce(f"recur_tree tree27b seed={kw['seed']}")
    d = device_batch(b)
    out, tsnap, ssnap = run_window(b, tree=True, d=d)
    check_against_oracle(b, out, tsnap, ssnap, tree=True)
    # commit each stream's accepted leaf (one stream keeps its state)
    acc = b.accept.clone()
    acc[3] = -1
    tail, state = d["tail"].clone(), d["state"].clone()
    announce("commit tree27b")
    gdn.commit(shape, d["row_start"], acc.cuda(), tsnap, ssnap, tail, state)
    torch.cuda.synchronize()
    for s in range(b.n):
        if acc[s] < 0:
            assert torch.equal(state[s], d["state"][s]) and torch.equal(tail[s], d["tail"][s])
        else:
            r = int(acc[s])
            assert torch.equal(state[s], ssnap[r]), s
            assert np.array_equal(bits16(tail[s]), bits16(tsnap[r])), s


def test_small_heads_windows_and_trees():
    """dk = dv = 64 (the small layer's heads, their own instantiation of the
    row kernel) beyond one row: ragged windows of up to 16 rows and draft
    trees against the oracle (outputs, state snapshots, tail snapshots)."""
    shape = gi.SMALL
    lengths = [16, 1, 7, 12, 3, 16]
    b = gi.make_batch(shape, lengths, seed=91)
    announce(f"recur_window small heads lengths={lengths} seed=91")
    out, tsnap, ssnap = run_window(b)
    check_against_oracle(b, out, tsnap, ssnap)
    bt = gi.make_batch(shape, lengths, seed=92, tree=True)
    announce(f"recur_tree small heads lengths={lengths} seed=92")
    out, tsnap, ssnap = run_window(bt, tree=True)
    check_against_oracle(bt, out, tsnap, ssnap, tree=True)


@pytest.mark.parametrize("name,n_streams", [("step", 1), ("window2b", 1), ("ragged27b", 3)])
def test_window_rows_equal_one_row_steps_bitwise(name, n_streams):
    shape, lengths, kw = gi.workload(name)
    lengths = lengths[:n_streams] if name != "step" else [5]
    b = gi.make_batch(shape, lengths, **kw)
    announce(f"window vs steps {name} lengths={lengths}")
    d = device_batch(b)
    out, tsnap, ssnap = run_window(b, d=d)
    rs = b.row_start.tolist()
    for s in range(b.n):
        tail = d["tail"][s:s + 1].clone()
        state = d["state"][s:s + 1].clone()
        o1 = torch.empty((1, shape.hv, shape.dv), dtype=torch.float32, device="cuda")
        for t in range(rs[s + 1] - rs[s]):
            r = rs[s] + t
            gdn.conv_step(shape, d["params"], d["qkv"][r:r + 1], d["a"][r:r + 1], d["b"][r:r + 1],
                          tail, state, o1)
            torch.cuda.synchronize()
            assert np.array_equal(bits32(o1[0]), bits32(out[r])), (s, t, "o")
            assert np.array_equal(bits32(state[0]), bits32(ssnap[r])), (s, t, "state")
            assert np.array_equal(bits16(tail[0]), bits16(tsnap[r])), (s, t, "tail")


def test_step_matches_oracle_many_streams():
    shape = gi.QWEN_27B
    b = gi.make_batch(shape, [1] * 16, seed=77)
    announce("conv_step 16 streams 27b")
    d = device_batch(b)
    out = torch.full((16, shape.hv, shape.dv), float("nan"), device="cuda")
    tail, state = d["tail"].clone(), d["state"].clone()
    gdn.conv_step(shape, d["params"], d["qkv"], d["a"], d["b"], tail, state, out)
    torch.cuda.synchronize()
    ref = oracle_rows(b)
    assert bound_err(out.cpu().numpy(), ref["o"], ref["o_mag"]) <= TOL_ROWS
    assert max_rel_err(state.cpu().numpy(), ref["snap32"], 2) <= TOL_ROWS
    assert np.array_equal(bits16(tail), ref["tail_snap"])


WIDE_STEPS = {"r8-d64": gi.Shape(hk=1, hv=8, dk=64, dv=64), "r4-d128": gi.Shape(hk=2, hv=8, dk=128, dv=128)}


@pytest.mark.parametrize("shape_name,n", [("SMALL", 300), ("dk64-dv128", 40), ("dk128-dv64", 40),
                                          ("r8-d64", 20), ("r4-d128", 12)])
def test_steps_many_streams_and_mixed_heads(shape_name, n):
    """One-row steps run one workgroup a (stream, key head): hundreds of
    streams on the small layer, both mixed head geometries, and the widest
    workgroups a step takes (16 waves: eight value heads of 64 columns, four
    of 128), against the oracle's one-step rows."""
    shape = gi.SMALL if shape_name == "SMALL" else MIXED.get(shape_name) or WIDE_STEPS[shape_name]
    b = gi.make_batch(shape, [1] * n, seed=91)
    announce(f"conv_step {n} streams {shape}")
    d = device_batch(b)
    out = torch.full((n, shape.hv, shape.dv), float("nan"), device="cuda")
    tail, state = d["tail"].clone(), d["state"].clone()
    gdn.conv_step(shape, d["params"], d["qkv"], d["a"], d["b"], tail, state, out)
    torch.cuda.synchronize()
    ref = oracle_rows(b)
    assert bound_err(out.cpu().numpy(), ref["o"], ref["o_mag"]) <= TOL_ROWS
    assert max_rel_err(state.cpu().numpy(), ref["snap32"], 2) <= TOL_ROWS
    assert np.array_equal(bits16(tail), ref["tail_snap"])


def test_tree_paths_equal_chains_bitwise():
    shape, lengths, kw = gi.workload("tree27b")
    b = gi.make_batch(shape, lengths[:4], **kw)
    announce("tree paths vs chains 27b, 4 streams")
    out, tsnap, ssnap = run_window(b, tree=True)
    par = b.parent.tolist()
    rs = b.row_start.tolist()
    for s in range(b.n):
        local = par[rs[s]:rs[s + 1]]
        for leaf in range(len(local)):
            rows = [rs[s] + i for i in gi.path_to_root(local, leaf)]
            chain = gi.Batch(shape=shape, params=b.params,
                             row_start=torch.tensor([0, len(rows)], dtype=torch.int32),
                             qkv=b.qkv[rows], a=b.a[rows], b=b.b[rows], tail=b.tail[s:s + 1],
                             state=b.state[s:s + 1])
            co, ct, cs = run_window(chain)
            assert np.array_equal(bits32(co), bits32(out[rows])), (s, leaf)
            assert np.array_equal(bits32(cs), bits32(ssnap[rows])), (s, leaf)
            assert np.array_equal(bits16(ct), bits16(tsnap[rows])), (s, leaf)


def test_packed_equals_solo_bitwise():
    """A stream's rows do not depend on the other streams of the pass nor on
    its packing offset."""
    shape, lengths, kw = gi.workload("ragged27b")
    b = gi.make_batch(shape, lengths[:5], **kw)
    announce(f"packed vs solo lengths={lengths[:5]}")
    out, tsnap, ssnap = run_window(b)
    rs = b.row_start.tolist()
    for s in (0, 2, 4):
        rows = list(range(rs[s], rs[s + 1]))
        solo = gi.Batch(shape=shape, params=b.params,
                        row_start=torch.tensor([0, len(rows)], dtype=torch.int32),
                        qkv=b.qkv[rows], a=b.a[rows], b=b.b[rows], tail=b.tail[s:s + 1],
                        state=b.state[s:s + 1])
        so, st, ss = run_window(solo)
        assert np.array_equal(bits32(so), bits32(out[rows]))
        assert np.array_equal(bits32(ss), bits32(ssnap[rows]))
        assert np.array_equal(bits16(st), bits16(tsnap[rows]))


@pytest.mark.parametrize("name", ["window2b", "verify27b"])
def test_workgroup_split_is_bitwise_invariant(name, monkeypatch):
    """A small launch gives each value head several workgroups (each a share
    of its column tiles); LIBGDN_HEADS_PER_BLOCK forces the plain one-workgroup-
    per-head layout.  Both must give the same bits, recorded and logged."""
    shape, lengths, kw = gi.workload(name)
    b = gi.make_batch(shape, lengths[:1], **kw)   # one stream: the launch that splits
    d = device_batch(b)
    announce(f"workgroup split {name} lengths={lengths[:1]}")
    runs = []
    for env in (None, "1"):
        if env is None:
            monkeypatch.delenv("LIBGDN_HEADS_PER_BLOCK", raising=False)
        else:
            monkeypatch.setenv("LIBGDN_HEADS_PER_BLOCK", env)
        out, tsnap, ssnap = run_window(b, d=d)
        o_l = torch.full_like(out, float("nan"))
        la = torch.full((b.rows, shape.hv), float("nan"), device="cuda")
        ld = torch.full((b.rows, shape.hv, shape.dv), float("nan"), device="cuda")
        lk = torch.full((b.rows, shape.hk, shape.dk), float("nan"), device="cuda")
        gdn.recur_log(shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"], d["tail"], d["state"],
                      o_l, la, ld, lk)
        torch.cuda.synchronize()
        runs.append((out, tsnap, ssnap, o_l, la, ld, lk))
    for x, y in zip(*runs):
        bx = bits16(x) if x.dtype == torch.bfloat16 else bits32(x)
        by = bits16(y) if y.dtype == torch.bfloat16 else bits32(y)
        assert np.array_equal(bx, by)


def test_empty_streams_and_zero_rows():
    shape = gi.QWEN_27B
    b = gi.make_batch(shape, [3, 0, 16, 0, 1], seed=5)
    announce("windows with empty streams")
    out, tsnap, ssnap = run_window(b)
    check_against_oracle(b, out, tsnap, ssnap)
    # a call with no rows at all does nothing
    e = gi.make_batch(shape, [0, 0], seed=6)
    d = device_batch(e)
    o, t, s = poisoned_outputs(shape, 0)
    gdn.recur_window(shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"], d["tail"],
                     d["state"], o, t, s)
    torch.cuda.synchronize()


def test_device_layout_breaking_rules_is_skipped():
    """A window longer than max_rows is skipped by the kernel's own check: its
    outputs stay poisoned and the other streams are unaffected."""
    shape = gi.SMALL
    b = gi.make_batch(shape, [4, 9, 2], seed=21)
    announce("window longer than max_rows is skipped")
    out, tsnap, ssnap = run_window(b, max_rows=8)
    assert torch.isnan(out[4:13]).all() and torch.isnan(ssnap[4:13]).all()
    ref = oracle_rows(b)
    keep = list(range(0, 4)) + list(range(13, 15))
    assert bound_err(out.cpu().numpy()[keep], ref["o"][keep], ref["o_mag"][keep]) <= TOL_ROWS
    # a tree row whose parent is not an earlier row: that stream is skipped
    t = gi.make_batch(shape, [3, 3], seed=22, tree=True)
    t.parent[4] = 1   # stream 1, row 1 names itself
    out, tsnap, ssnap = run_window(t, tree=True)
    assert torch.isnan(out[3:6]).all()
    assert not torch.isnan(out[0:3]).any()


def test_special_cases_through_the_kernels():
    """alpha = 1 and beta = 1 (A_log = -inf, b = +inf) with q's channels equal
    to k's: each row writes v at key khat and reads it back, o = v / sqrt(dk);
    beta = 0 (b = -inf) and A_log = 0 with a + dt_bias = 0 halve the state each
    row."""
    shape = gi.Shape(hk=4, hv=8, dk=128, dv=64)
    b = gi.make_batch(shape, [6, 3], seed=23)
    hkdk = shape.hk * shape.dk
    b.params.a_log[:] = -float("inf")
    b.b[:] = float("inf")
    b.qkv[:, :hkdk] = b.qkv[:, hkdk:2 * hkdk]
    b.tail[:, :, :hkdk] = b.tail[:, :, hkdk:2 * hkdk]
    b.params.conv_w[:hkdk] = b.params.conv_w[hkdk:2 * hkdk]
    announce("unit write read-back")
    out, tsnap, ssnap = run_window(b)
    check_against_oracle(b, out, tsnap, ssnap)
    ref = oracle_rows(b)
    assert bound_err(out.cpu().numpy(), ref["o"], ref["o_mag"]) <= 1e-4

    c = gi.make_batch(shape, [5], seed=24)
    c.params.a_log[:] = 0.0
    c.params.dt_bias[:] = 0.25
    c.a[:] = -0.25
    c.b[:] = -float("inf")
    announce("pure decay")
    out, tsnap, ssnap = run_window(c)
    for t in range(5):
        expect = c.state[0] * 0.5 ** (t + 1)
        assert torch.allclose(ssnap[t].cpu(), expect, rtol=1e-6, atol=0)
