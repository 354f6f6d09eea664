"""GPU log-and-replay verify: gdn_recur_log against the recording pass and the
oracle, and gdn_commit_replay against gdn_commit.

The logged pass must leave o bit for bit as the recording pass does, and the
commit by replay must reach bit for bit the state and tail the snapshot
commit copies (both are the same per-element operations in the same order).
The logged decay, write and key are compared with the oracle's log within the
row kernels' tolerance.  Outputs start poisoned (NaN), so an element the
kernels fail to write shows up as a failure."""
import numpy as np
import pytest
import torch

import oracle
from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import (TOL_ROWS, announce, bits16, bits32, bound_err, device_batch, host_batch,
                      max_rel_err, poisoned_outputs)

pytestmark = pytest.mark.gpu

SMALL_27B_HEADS = gi.Shape(hk=2, hv=6, dk=128, dv=128)   # 3 value heads a key head


def poisoned_log(shape: gi.Shape, rows: int, dev="cuda"):
    nan = float("nan")
    return (torch.full((rows, shape.hv), nan, dtype=torch.float32, device=dev),
            torch.full((rows, shape.hv, shape.dv), nan, dtype=torch.float32, device=dev),
            torch.full((rows, shape.hk, shape.dk), nan, dtype=torch.float32, device=dev))


def run_both(b: gi.Batch, tree: bool):
    d = device_batch(b)
    par = d["parent"] if tree else None
    out_r, tsnap, ssnap = poisoned_outputs(b.shape, b.rows)
    if tree:
        gdn.recur_tree(b.shape, d["params"], d["row_start"], par, d["qkv"], d["a"], d["b"],
                       d["tail"], d["state"], out_r, tsnap, ssnap)
    else:
        gdn.recur_window(b.shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"],
                         d["tail"], d["state"], out_r, tsnap, ssnap)
    out_l, _, _ = poisoned_outputs(b.shape, b.rows)
    la, ld, lk = poisoned_log(b.shape, b.rows)
    gdn.recur_log(b.shape, d["params"], d["row_start"], d["qkv"], d["a"], d["b"], d["tail"],
                  d["state"], out_l, la, ld, lk, parent=par)
    torch.cuda.synchronize()
    return d, out_r, tsnap, ssnap, out_l, (la, ld, lk)


def accept_cases(b: gi.Batch, tree: bool, gen: torch.Generator):
    rs = b.row_start.tolist()
    n = len(rs) - 1
    last = [rs[s + 1] - 1 if rs[s + 1] > rs[s] else -1 for s in range(n)]
    first = [rs[s] if rs[s + 1] > rs[s] else -1 for s in range(n)]
    rand = [int(torch.randint(rs[s], rs[s + 1], (1,), generator=gen)) if rs[s + 1] > rs[s] else -1
            for s in range(n)]
    mixed = list(rand)
    mixed[0] = -1
    cases = [last, first, rand, mixed]
    if tree and b.accept is not None:
        cases.append(b.accept.tolist())
    return cases


def check_commits(b: gi.Batch, d, tsnap, ssnap, log, tree: bool, seed: int):
    gen = torch.Generator().manual_seed(seed)
    la, ld, lk = log
    for acc in accept_cases(b, tree, gen):
        acc_d = torch.tensor(acc, dtype=torch.int32, device="cuda")
        tail_s, state_s = d["tail"].clone(), d["state"].clone()
        gdn.commit(b.shape, d["row_start"], acc_d, tsnap, ssnap, tail_s, state_s)
        tail_r, state_r = d["tail"].clone(), d["state"].clone()
        gdn.commit_replay(b.shape, d["row_start"], acc_d, d["qkv"], la, ld, lk, tail_r, state_r,
                          parent=d["parent"] if tree else None)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(state_r), bits32(state_s)), f"replayed state differs (accept {acc})"
        assert np.array_equal(bits16(tail_r), bits16(tail_s)), f"replayed tail differs (accept {acc})"


def check_log_against_oracle(b: gi.Batch, log, tree: bool):
    h = host_batch(b)
    fn = oracle.tree if tree else oracle.window
    args = [b.shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"]]
    if tree:
        args.append(b.parent.numpy())
    args += [h["qkv"], h["a"], h["b"], h["tail"], h["state"]]
    ref = fn(*args, snap64=False, snap32=False, tail_snap=False, log=True, mag=True)
    la, ld, lk = (t.cpu().numpy() for t in log)
    e_a = max_rel_err(la, ref["log_alpha"], 2)                      # each decay alone
    e_d = bound_err(ld, ref["log_delta"], ref["log_delta_mag"])     # each write element
    e_k = max_rel_err(lk, ref["log_key"], 2)                        # each unit key
    assert e_a <= TOL_ROWS and e_d <= TOL_ROWS and e_k <= TOL_ROWS, (e_a, e_d, e_k)
    return e_a, e_d, e_k


CASES = {
    "chains-small27b-ragged": (SMALL_27B_HEADS, [16, 1, 7, 0, 12, 3], False, 61),
    "trees-small27b": (SMALL_27B_HEADS, [16, 9, 1, 16, 5], True, 62),
    "chains-dk64": (gi.SMALL, [5, 16, 2], False, 63),
    "trees-dk64": (gi.SMALL, [16, 16, 4], True, 64),
    "window-2b": (gi.QWEN_2B, [16], False, 65),
    "chains-dk64-dv128": (gi.Shape(hk=2, hv=6, dk=64, dv=128), [16, 5, 9], False, 67),
    "trees-dk64-dv128": (gi.Shape(hk=2, hv=6, dk=64, dv=128), [16, 11, 2], True, 68),
    "chains-dk128-dv64": (gi.Shape(hk=2, hv=4, dk=128, dv=64), [3, 16, 8], False, 69),
    "trees-dk128-dv64": (gi.Shape(hk=2, hv=4, dk=128, dv=64), [16, 16, 6], True, 70),
    # enough streams that whole key heads stay in a workgroup: 16 waves
    "chains-r8-d64-wide": (gi.Shape(hk=1, hv=8, dk=64, dv=64), ([16, 3, 11, 16, 1] * 4)[:17], False, 71),
    "trees-r4-d128-wide": (gi.Shape(hk=2, hv=8, dk=128, dv=128), ([16, 9, 1, 16, 5] * 2)[:9], True, 72),
}


@pytest.mark.parametrize("case", list(CASES))
def test_logged_pass_equals_recording_pass_and_oracle(case):
    shape, lengths, tree, seed = CASES[case]
    b = gi.make_batch(shape, lengths, seed=seed, tree=tree)
    announce(f"recur_log {case} lengths={lengths} seed={seed}")
    d, out_r, tsnap, ssnap, out_l, log = run_both(b, tree)
    assert np.array_equal(bits32(out_l), bits32(out_r)), "logged o differs from the recording pass"
    e = check_log_against_oracle(b, log, tree)
    announce(f"commit_replay {case}")
    check_commits(b, d, tsnap, ssnap, log, tree, seed)
    print(f"{case}: log errs alpha {e[0]:.1e} delta {e[1]:.1e} key {e[2]:.1e}")


@pytest.mark.parametrize("name", ["verify27b", "tree27b", "ragged27b"])
def test_logged_pass_full_size(name):
    """The 27B-like layer at the verify workloads' full size: o and every commit
    bit for bit against the recording pass (whose parity with the oracle the
    row tests check at this size)."""
    shape, lengths, kw = gi.workload(name)
    tree = name == "tree27b"
    b = gi.make_batch(shape, lengths, **kw)
    announce(f"recur_log {name} full size seed={kw['seed']}")
    d, out_r, tsnap, ssnap, out_l, log = run_both(b, tree)
    assert np.array_equal(bits32(out_l), bits32(out_r)), "logged o differs from the recording pass"
    assert all(bool(torch.isfinite(t).all()) for t in log), "a log entry was not written"
    announce(f"commit_replay {name} full size")
    check_commits(b, d, tsnap, ssnap, log, tree, kw["seed"])


def test_commits_skip_rows_outside_the_window():
    shape = SMALL_27B_HEADS
    b = gi.make_batch(shape, [4, 3, 5], seed=66)
    announce("commit_replay outside rows")
    d, out_r, tsnap, ssnap, out_l, log = run_both(b, False)
    rs = b.row_start.tolist()
    acc = torch.tensor([rs[1], rs[3] + 7, rs[2] + 2], dtype=torch.int32, device="cuda")  # stream 0 and 1 invalid
    tail_r, state_r = d["tail"].clone(), d["state"].clone()
    gdn.commit_replay(shape, d["row_start"], acc, d["qkv"], *log, tail_r, state_r)
    tail_s, state_s = d["tail"].clone(), d["state"].clone()
    gdn.commit(shape, d["row_start"], torch.tensor([-1, -1, rs[2] + 2], dtype=torch.int32, device="cuda"),
               tsnap, ssnap, tail_s, state_s)
    # the snapshot commit skips the same streams: stream 0 names stream 1's
    # first row, stream 1 a row past the pass
    tail_x, state_x = d["tail"].clone(), d["state"].clone()
    gdn.commit(shape, d["row_start"], acc, tsnap, ssnap, tail_x, state_x)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(state_r), bits32(state_s))
    assert np.array_equal(bits16(tail_r), bits16(tail_s))
    assert np.array_equal(bits32(state_x), bits32(state_s)), "commit copied a row outside the stream's window"
    assert np.array_equal(bits16(tail_x), bits16(tail_s))
    assert torch.equal(state_x[0], d["state"][0]) and torch.equal(tail_x[1], d["tail"][1])
