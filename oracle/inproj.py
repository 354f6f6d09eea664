"""fp64 CPU oracle of the affine 4-bit in-projection -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

The projection that produces the mixer's inputs runs on affine 4-bit weights
(page "perf(qwen3_5 cuda): deliver the first token before drafting", the note
on the MLX affine 4-bit checkpoint: its projections run through affine-4
kernels).  The pages do not spell the format out; the reading taken here is
MLX's published affine quantisation: weight ``w[n][k] = s[n][g] * q[n][k] +
b[n][g]`` with a 4-bit code ``q`` and, per output feature ``n`` and group
``g = k // group`` of consecutive inputs, a scale ``s`` and a bias ``b``
(bf16).  Codes are packed eight to a 32-bit word, code ``j`` of word ``w`` in
bits ``[4j, 4j + 4)`` holding input ``8w + j``.

The projection is the plain definition ``y = x W^T`` over exact (fp64) weights;
outputs ``[qkv | a | b]`` split at ``C`` and ``C + hv``.  Pinned in
``tests/test_oracle_inproj.py`` (code order, group indexing, the roles of scale
and bias, exact integer products, a brute-force loop).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Values of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def unpack_codes(wq, hidden: int) -> np.ndarray:
    """The 4-bit codes [N][hidden] (0..15) of packed int32/uint32 words [N][hidden/8]."""
    w = np.asarray(wq).view(np.uint32)
    assert w.shape[1] * 8 == hidden
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    codes = (w[:, :, None] >> shifts) & np.uint32(15)
    return codes.reshape(w.shape[0], hidden).astype(np.int64)


def dequantize(wq, scale_bits, bias_bits, hidden: int, group: int) -> np.ndarray:
    """Exact weights [N][hidden] in fp64: s * q + b, s and b of the input's group."""
    q = unpack_codes(wq, hidden).astype(np.float64)
    s = np.repeat(bf16_to_f64(scale_bits), group, axis=1)
    b = np.repeat(bf16_to_f64(bias_bits), group, axis=1)
    assert s.shape == q.shape
    return s * q + b


def project(x_bits, wq, scale_bits, bias_bits, group: int) -> np.ndarray:
    """y [R][N] = x W^T in fp64 (x: bf16 bit patterns [R][hidden])."""
    x = bf16_to_f64(x_bits)
    w = dequantize(wq, scale_bits, bias_bits, x.shape[1], group)
    return x @ w.T


def split(y: np.ndarray, channels: int, hv: int):
    """The mixer's inputs from the projection's features: qkv, a, b."""
    assert y.shape[1] == channels + 2 * hv
    return y[:, :channels], y[:, channels:channels + hv], y[:, channels + hv:]
