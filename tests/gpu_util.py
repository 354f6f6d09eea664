"""Helpers of the GPU tests: device copies of a batch, oracle runs, the error
metric, and poisoned output buffers."""
import sys

import numpy as np
import torch

import oracle
from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi

# Tolerances of the row kernels (fp32 state, bf16 inputs) and of the chunked
# prompt pass (bf16 matrix-core operands).  Outputs o, logged writes and state
# elements are bounded element by element relative to their magnitude (the
# oracle's computation carried out on magnitudes, ``bound_err``); states also
# relative to the largest element of their (row, head) matrix (``max_rel_err``).
TOL_ROWS = 2e-3
TOL_PREFILL = 2e-2

# Only where the oracle's magnitude is exactly zero (every term zero) does
# this absolute floor decide; any fp32 rounding of a non-zero sum is far above.
MAG_FLOOR = 1e-30

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


def oracle_rows(b: gi.Batch, tree=False, snap64=False, snap32=True, log=False, snap_mag=False):
    h = host_batch(b)
    fn = oracle.tree if tree else oracle.window
    args = [b.shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"]]
    if tree:
        args.append(b.parent.numpy())
    args += [h["qkv"], h["a"], h["b"], h["tail"], h["state"]]
    return fn(*args, snap64=snap64, snap32=snap32, log=log, mag=True, snap_mag=snap_mag)


def bound_err(gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray) -> float:
    """max over elements of |gpu - ref| / max(mag, MAG_FLOOR), where ``mag``
    is the oracle's magnitude of the element: its row's step carried out on
    magnitudes from the state the row starts from (|M| and the inputs'
    absolute values, every sum by the sum of its terms' magnitudes, every
    product by the product of magnitudes, SiLU's output by its gate times
    the conv's term magnitude).  A test
    asserts it is at most the tolerance: every element then satisfies
    |gpu - ref| <= tol * mag (+ the floor where mag is exactly 0).

    Values can cancel far below their terms: a readout o = M^T qhat, a write
    beta (v - alpha M^T khat), a conv output that leaves v nearly 0 and every
    state column built from such a write.  fp32 rounding of the terms then
    gives a relative error of |o| far above 2e-3 (1.4e-2 on one (row, head)
    vector of a ragged 27B-like window; 2.5e-3 on single elements against
    sum_i |M_ij qhat_i| alone), so the error is scaled by the magnitude of
    every term that reached the element.  Any non-finite GPU value gives inf."""
    assert gpu.shape == ref.shape == mag.shape, (gpu.shape, ref.shape, mag.shape)
    if gpu.size == 0:
        return 0.0
    worst = 0.0
    step = max(1, (1 << 24) // max(1, gpu[0].size))      # about 16M elements at a time
    for i in range(0, gpu.shape[0], step):
        g = np.asarray(gpu[i:i + step], np.float64)
        if not np.all(np.isfinite(g)):
            return float("inf")
        r = np.asarray(ref[i:i + step], np.float64)
        m = np.asarray(mag[i:i + step], np.float64)
        worst = max(worst, float(np.max(np.abs(g - r) / np.maximum(m, MAG_FLOOR))))
    return worst


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Printed beside ``bound_err`` only: max over packed rows of
    max|gpu - ref| / max|ref| over the row's heads and columns."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    if g.size == 0:
        return 0.0
    g = g.reshape(g.shape[0], -1)
    r = r.reshape(r.shape[0], -1)
    return float(np.max(np.abs(g - r).max(1) / np.maximum(np.abs(r).max(1), 1e-30)))


def max_rel_err(gpu: np.ndarray, ref: np.ndarray, lead_dims: int) -> float:
    """max over blocks (the first ``lead_dims`` axes index them) of
    max|gpu - ref| / max(max|ref|, 1e-30).  Any non-finite GPU value is inf.

    Used for states (per (row, head) matrix, lead_dims=2), for unit keys
    (per (row, key head) vector) and, with lead_dims = ndim, element by
    element for values that cannot cancel (the decays alpha > 0)."""
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
