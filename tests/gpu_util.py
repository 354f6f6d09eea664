"""Helpers of the GPU tests: device copies of a batch, oracle runs, the error
metric, and poisoned output buffers."""
import sys

import numpy as np
import torch

import oracle
from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

# Tolerances of the row kernels (fp32 state, bf16 inputs) and of the chunked
# prompt pass (bf16 matrix-core operands), as max relative errors per vector.
TOL_ROWS = 2e-3
TOL_PREFILL = 2e-2

POISON_F32 = float("nan")
POISON_BF16_BITS = -1          # 0xFFFF, a NaN bit pattern


def announce(msg: str):
    """Names the case on stdout before a GPU step, so a run that dies says where."""
    print(f"\n[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def device_batch(b: gi.Batch, dev="cuda"):
    d = dict(
        row_start=b.row_start.to(dev), qkv=b.qkv.to(dev), a=b.a.to(dev), b=b.b.to(dev),
        tail=b.tail.to(dev), state=b.state.to(dev),
        params=gdn.LayerParams.from_host(b.params, dev),
    )
    if b.parent is not None:
        d["parent"] = b.parent.to(dev)
    if b.accept is not None:
        d["accept"] = b.accept.to(dev)
    return d


def host_batch(b: gi.Batch):
    return dict(conv_w=b.params.conv_w.numpy(), a_log=b.params.a_log.numpy(),
                dt_bias=b.params.dt_bias.numpy(), row_start=b.row_start.numpy(),
                qkv=gi.bf16_bits(b.qkv), a=gi.bf16_bits(b.a), b=gi.bf16_bits(b.b),
                tail=gi.bf16_bits(b.tail), state=b.state.numpy().astype(np.float64))


def poisoned_outputs(shape: gi.Shape, rows: int, dev="cuda"):
    out = torch.full((rows, shape.hv, shape.dv), POISON_F32, dtype=torch.float32, device=dev)
    tsnap = torch.full((rows, 3, shape.channels), POISON_BF16_BITS, dtype=torch.int16,
                       device=dev).view(torch.bfloat16)
    ssnap = torch.full((rows, shape.hv, shape.dk, shape.dv), POISON_F32, dtype=torch.float32,
                       device=dev)
    return out, tsnap, ssnap


def oracle_rows(b: gi.Batch, tree=False, snap64=False, snap32=True):
    h = host_batch(b)
    fn = oracle.tree if tree else oracle.window
    args = [b.shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"]]
    if tree:
        args.append(b.parent.numpy())
    args += [h["qkv"], h["a"], h["b"], h["tail"], h["state"]]
    return fn(*args, snap64=snap64, snap32=snap32)


def max_rel_err(gpu: np.ndarray, ref: np.ndarray, lead_dims: int) -> float:
    """max over blocks (the first ``lead_dims`` axes index them) of
    max|gpu - ref| / max(max|ref|, 1e-30).  Any non-finite GPU value is inf.

    Outputs o are compared per packed row (lead_dims=1, all heads of the row
    together): the readout o = S q of one head can cancel almost completely
    (a query nearly orthogonal to the state's rows gives |o| ~ 1e-6 of the
    terms it sums), and no fp32 result has a small relative error on such a
    vector.  States are compared per (row, head) matrix (lead_dims=2)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    lead = g.shape[:lead_dims]
    g = g.reshape(int(np.prod(lead)), -1)
    r = r.reshape(int(np.prod(lead)), -1)
    num = np.max(np.abs(g - r), axis=1)
    den = np.maximum(np.max(np.abs(r), axis=1), 1e-30)
    return float(np.max(num / den))


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int32).cpu().numpy()


def max_rel_err_segments(gpu: np.ndarray, ref: np.ndarray, starts) -> float:
    """Outputs of a prompt pass: for each prompt (rows starts[i]..starts[i+1]),
    max |gpu - ref| over its rows, heads and columns divided by max |ref| over
    the same, then the maximum over prompts.  The bf16 operands of the chunked
    form leave an absolute error of a few 1e-3 of the terms a readout sums, so
    a row whose outputs all cancel (|o| far below the prompt's typical
    magnitude) has no meaningful relative error of its own."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    worst = 0.0
    st = list(starts)
    for i in range(len(st) - 1):
        a, b = st[i], st[i + 1]
        if b > a:
            worst = max(worst, float(np.abs(g[a:b] - r[a:b]).max() / max(np.abs(r[a:b]).max(), 1e-30)))
    return worst
