"""GPU parity of the affine 4-bit in-projection against the fp64 oracle.

Bound, element by element: the kernel rounds each weight s*q + b to bf16
(relative error at most 2^-9), accumulates in fp32 and rounds the output to
bf16 (2^-9 relative), so with S = |x| |W|^T (exact, from the oracle)

    |y_gpu - y| <= 2^-9 S + 2^-9 |y| + K 2^-24 S

(the last term bounds fp32 accumulation over K inputs).  Outputs start
poisoned (NaN), so an element the kernel fails to write shows up."""
import numpy as np
import pytest
import torch

import oracle
from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

from gpu_util import announce

pytestmark = pytest.mark.gpu

inproj = oracle.inproj


def run(t: gi.Inproj):
    dev = "cuda"
    sh = t.shape
    nan = float("nan")
    qkv = torch.full((t.rows, sh.channels), nan, dtype=torch.bfloat16, device=dev)
    a = torch.full((t.rows, sh.hv), nan, dtype=torch.bfloat16, device=dev)
    b = torch.full((t.rows, sh.hv), nan, dtype=torch.bfloat16, device=dev)
    wt, st, bt = gdn.inproj_pack(sh, t.wq.to(dev), t.scales.to(dev), t.biases.to(dev), t.group)
    gdn.inproj_affine4(sh, t.x.to(dev), wt, st, bt, qkv, a, b, t.group)
    torch.cuda.synchronize()
    return torch.cat([qkv, a, b], dim=1).float().cpu().numpy().astype(np.float64)


def check(t: gi.Inproj, y_gpu: np.ndarray, rows=None):
    rows = np.arange(t.rows) if rows is None else np.asarray(rows)
    xb = gi.bf16_bits(t.x)[rows]
    sb, bb = gi.bf16_bits(t.scales), gi.bf16_bits(t.biases)
    y = inproj.project(xb, t.wq.numpy(), sb, bb, t.group)
    w = inproj.dequantize(t.wq.numpy(), sb, bb, t.hidden, t.group)
    S = np.abs(inproj.bf16_to_f64(xb)) @ np.abs(w).T
    bound = 2.0 ** -9 * S + 2.0 ** -9 * np.abs(y) + t.hidden * 2.0 ** -24 * S
    g = y_gpu[rows]
    assert np.all(np.isfinite(g)), "an output was not written"
    err = np.abs(g - y)
    worst = float((err / bound).max())
    assert worst <= 1.0, f"error {worst:.3f} of the bound"
    rel = float(err.max() / np.abs(y).max())
    return worst, rel


CASES = {
    # rows, hidden, group: the small kernel (1 and 2 row tiles), the large one
    # (a partial row tile, the feature tile that crosses into a and b; two
    # input shares while the tiles leave a compute unit each)
    "rows1-g32": (gi.SMALL, 1, 256, 32),
    "rows5-g64": (gi.SMALL, 5, 384, 64),
    "rows16-g128": (gi.SMALL, 16, 512, 128),
    "rows17-g64": (gi.SMALL, 17, 256, 64),
    "rows32-g32": (gi.SMALL, 32, 384, 32),
    "rows33-g64": (gi.SMALL, 33, 256, 64),
    "rows200-g128": (gi.SMALL, 200, 640, 128),
    "small27b-rows130": (gi.Shape(hk=2, hv=6, dk=128, dv=128), 130, 768, 64),
    # the 27B-like layer's 81 feature tiles: 4 tiles of 128 rows (more tiles
    # than compute units, one input share), then 256-row tiles (3, the last
    # one ragged)
    "27b-rows500-g64": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 500, 256, 64),
    "27b-rows700-g32": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 700, 384, 32),
    # the smallest hidden size (one 128-input chunk): seven of the small
    # kernel's eight waves without a chunk; one 64-input chunk a share; one
    # pair of chunks for 128- and 256-row tiles
    "rows3-h128-g128": (gi.SMALL, 3, 128, 128),
    "rows40-h128-g64": (gi.SMALL, 40, 128, 64),
    "27b-rows400-h128-g32": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 400, 128, 32),
    "27b-rows600-h128-g128": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 600, 128, 128),
    # up to 16 rows: three feature blocks a workgroup, every weight requested
    # up front (a partial row tile, 3 chunks a wave); the small kernel where
    # the scales and biases (groups of 32) or the chunks (48) exceed that
    # kernel's loads
    "27b-rows9-h3072-g64": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 9, 3072, 64),
    "27b-rows16-h5120-g32": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 16, 5120, 32),
    "27b-rows16-h6144-g64": (gi.Shape(hk=16, hv=48, dk=128, dv=128), 16, 6144, 64),
}


@pytest.mark.parametrize("case", list(CASES))
def test_inproj_matches_oracle(case):
    shape, rows, hidden, group = CASES[case]
    t = gi.make_inproj(shape, rows, hidden, group, seed=71 + list(CASES).index(case))
    announce(f"inproj {case}")
    worst, rel = check(t, run(t))
    print(f"{case}: {worst:.3f} of the bound, max rel err {rel:.2e}")


@pytest.mark.parametrize("name", ["inproj_decode27b", "inproj_verify27b", "inproj_window2b"])
def test_inproj_full_size(name):
    shape, rows, hidden, group, seed = gi.inproj_workload(name)
    t = gi.make_inproj(shape, rows, hidden, group, seed)
    announce(f"inproj {name} full size")
    worst, rel = check(t, run(t))
    print(f"{name}: {worst:.3f} of the bound, max rel err {rel:.2e}")


def test_inproj_prefill_size_sampled_rows():
    """The prompt pass's 8,306 rows in one call; the oracle checks 96 rows
    spread over all row tiles (and the last, partial one)."""
    shape, rows, hidden, group, seed = gi.inproj_workload("inproj_prefill27b")
    t = gi.make_inproj(shape, rows, hidden, group, seed)
    announce("inproj prefill27b full size")
    y = run(t)
    assert np.all(np.isfinite(y)), "an output was not written"
    sample = np.unique(np.concatenate([np.linspace(0, rows - 1, 90).astype(int), np.arange(rows - 6, rows)]))
    worst, rel = check(t, y, sample)
    print(f"prefill rows: {worst:.3f} of the bound, max rel err {rel:.2e}")


def test_inproj_feeds_the_mixer():
    """The projection's outputs, fed to a window, give what the oracle's window
    gives on the same (bf16) projection outputs: the two calls compose."""
    shape = gi.Shape(hk=2, hv=6, dk=128, dv=128)
    t = gi.make_inproj(shape, 12, 256, 64, seed=80)
    b = gi.make_batch(shape, [12], seed=81)
    dev = "cuda"
    qkv = torch.empty((12, shape.channels), dtype=torch.bfloat16, device=dev)
    a = torch.empty((12, shape.hv), dtype=torch.bfloat16, device=dev)
    bb = torch.empty((12, shape.hv), dtype=torch.bfloat16, device=dev)
    wt, st, bt = gdn.inproj_pack(shape, t.wq.to(dev), t.scales.to(dev), t.biases.to(dev), 64)
    gdn.inproj_affine4(shape, t.x.to(dev), wt, st, bt, qkv, a, bb, 64)
    params = gdn.LayerParams.from_host(b.params, dev)
    out = torch.empty((12, shape.hv, shape.dv), device=dev)
    ts = torch.empty((12, 3, shape.channels), dtype=torch.bfloat16, device=dev)
    ss = torch.empty((12, shape.hv, shape.dk, shape.dv), device=dev)
    gdn.recur_window(shape, params, b.row_start.to(dev), qkv, a, bb, b.tail.to(dev), b.state.to(dev), out, ts, ss)
    torch.cuda.synchronize()
    b.qkv, b.a, b.b = qkv.cpu(), a.cpu(), bb.cpu()
    from gpu_util import TOL_ROWS, bound_err, oracle_rows
    ref = oracle_rows(b)
    assert bound_err(out.cpu().numpy(), ref["o"], ref["o_mag"]) <= TOL_ROWS
