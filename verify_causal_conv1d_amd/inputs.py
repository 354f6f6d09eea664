"""Seeded synthetic inputs for the gated-delta-rule (GDN) mixer.

This module draws random tensors and row layouts and nothing else: it holds
none of the mixer's arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it.  Everything is drawn on the CPU from a
``torch.Generator`` seeded explicitly; bf16 tensors are rounded to nearest
even by ``Tensor.to(torch.bfloat16)``.

Distributions follow the layer workloads of the mixer (``N(0, s)`` means
standard deviation ``s``):

* packed rows ``qkv`` ~ N(0, 1), bf16, ``[R][C]`` with
  ``C = 2*hk*dk + hv*dv`` and channels ordered ``[q | k | v]``, head-major;
* depthwise conv weights ~ N(0, 0.3), fp32, ``[C][4]`` (tap 3 = current row);
* conv tail ~ N(0, 1), bf16, ``[n][3][C]`` (oldest row first);
* gate inputs ``a``, ``b`` ~ N(0, 1), bf16, ``[R][hv]``;
* ``A_log`` ~ U(0, 2.7) fp32 ``[hv]`` (the "long memory" variant draws
  U(-7, -4), which keeps the per-row decay near 1);
* ``dt_bias`` ~ N(0, 0.1) fp32 ``[hv]``;
* recurrent state ~ N(0, 0.05), fp32, ``[n][hv][dk][dv]``;
* the in-projection's hidden rows, codes, scales and biases (``make_inproj``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

CONV_WIDTH = 4
TAIL_ROWS = CONV_WIDTH - 1


@dataclass(frozen=True)
class Shape:
    hk: int
    hv: int
    dk: int
    dv: int

    @property
    def channels(self) -> int:
        return 2 * self.hk * self.dk + self.hv * self.dv

    @property
    def state_elems(self) -> int:
        return self.hv * self.dk * self.dv


# Layer geometries of the workloads: a small test layer, a 2B-like layer and a
# 27B-like layer of the Qwen3.5 hybrid family.
SMALL = Shape(hk=2, hv=4, dk=64, dv=64)
QWEN_2B = Shape(hk=16, hv=16, dk=128, dv=128)
QWEN_27B = Shape(hk=16, hv=48, dk=128, dv=128)


@dataclass
class LayerParams:
    conv_w: torch.Tensor   # fp32 [C][4]
    a_log: torch.Tensor    # fp32 [hv]
    dt_bias: torch.Tensor  # fp32 [hv]


@dataclass
class Batch:
    """Inputs of one call: packed rows plus per-stream state and tail."""
    shape: Shape
    params: LayerParams
    row_start: torch.Tensor          # int32 [n+1]
    qkv: torch.Tensor                # bf16 [R][C]
    a: torch.Tensor                  # bf16 [R][hv]
    b: torch.Tensor                  # bf16 [R][hv]
    tail: torch.Tensor               # bf16 [n][3][C]
    state: torch.Tensor              # fp32 [n][hv][dk][dv]
    parent: Optional[torch.Tensor] = None   # int32 [R], local index or -1
    accept: Optional[torch.Tensor] = None   # int32 [n], packed row index
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.row_start.numel()) - 1

    @property
    def rows(self) -> int:
        return int(self.qkv.shape[0])

    def lengths(self) -> list:
        rs = self.row_start.tolist()
        return [rs[i + 1] - rs[i] for i in range(len(rs) - 1)]


def _normal(gen, shape, std, dtype=torch.float32):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(dtype)


def make_params(shape: Shape, gen: torch.Generator, long_memory: bool = False) -> LayerParams:
    conv_w = _normal(gen, (shape.channels, CONV_WIDTH), 0.3)
    lo, hi = (-7.0, -4.0) if long_memory else (0.0, 2.7)
    a_log = torch.rand((shape.hv,), generator=gen, dtype=torch.float32) * (hi - lo) + lo
    dt_bias = _normal(gen, (shape.hv,), 0.1)
    return LayerParams(conv_w=conv_w, a_log=a_log, dt_bias=dt_bias)


def ragged_lengths(n: int, max_rows: int, gen: torch.Generator) -> list:
    """Window lengths drawn uniformly from 1..max_rows."""
    return (torch.randint(1, max_rows + 1, (n,), generator=gen)).tolist()


def starts_from_lengths(lengths) -> torch.Tensor:
    rs = [0]
    for ln in lengths:
        rs.append(rs[-1] + int(ln))
    return torch.tensor(rs, dtype=torch.int32)


def random_tree_parents(lengths, gen: torch.Generator) -> torch.Tensor:
    """Best-first draft trees with random shape: node 0 hangs off the stream's
    committed state (parent -1); node i > 0 takes a parent uniform in [0, i)."""
    par = []
    for ln in lengths:
        for i in range(int(ln)):
            if i == 0:
                par.append(-1)
            else:
                par.append(int(torch.randint(0, i, (1,), generator=gen)))
    return torch.tensor(par, dtype=torch.int32)


def chain_parents(lengths) -> torch.Tensor:
    par = []
    for ln in lengths:
        par.extend(range(-1, int(ln) - 1))
    return torch.tensor(par, dtype=torch.int32)


def random_leaves(lengths, parent: torch.Tensor, row_start: torch.Tensor,
                  gen: torch.Generator) -> torch.Tensor:
    """One accepted root-to-leaf path a stream: a leaf (a node no other node
    names as parent) chosen uniformly; returned as its packed row index."""
    out = []
    rs = row_start.tolist()
    par = parent.tolist()
    for s, ln in enumerate(lengths):
        base = rs[s]
        has_child = [False] * int(ln)
        for i in range(int(ln)):
            p = par[base + i]
            if p >= 0:
                has_child[p] = True
        leaves = [i for i in range(int(ln)) if not has_child[i]]
        pick = leaves[int(torch.randint(0, len(leaves), (1,), generator=gen))]
        out.append(base + pick)
    return torch.tensor(out, dtype=torch.int32)


def path_to_root(parent_local: list, leaf: int) -> list:
    """Local node indices from the root (node with parent -1) down to ``leaf``."""
    path = []
    i = leaf
    while i >= 0:
        path.append(i)
        i = parent_local[i]
    return path[::-1]


def make_batch(shape: Shape, lengths, seed: int, *, tree: bool = False,
               long_memory: bool = False, zero_state: bool = False) -> Batch:
    """Draw one call's inputs.  ``lengths`` gives each stream's row count."""
    gen = torch.Generator().manual_seed(int(seed))
    params = make_params(shape, gen, long_memory=long_memory)
    n = len(lengths)
    rows = int(sum(lengths))
    row_start = starts_from_lengths(lengths)
    qkv = _normal(gen, (rows, shape.channels), 1.0, torch.bfloat16)
    a = _normal(gen, (rows, shape.hv), 1.0, torch.bfloat16)
    b = _normal(gen, (rows, shape.hv), 1.0, torch.bfloat16)
    if zero_state:
        tail = torch.zeros((n, TAIL_ROWS, shape.channels), dtype=torch.bfloat16)
        state = torch.zeros((n, shape.hv, shape.dk, shape.dv), dtype=torch.float32)
    else:
        tail = _normal(gen, (n, TAIL_ROWS, shape.channels), 1.0, torch.bfloat16)
        state = _normal(gen, (n, shape.hv, shape.dk, shape.dv), 0.05)
    batch = Batch(shape=shape, params=params, row_start=row_start, qkv=qkv, a=a, b=b,
                  tail=tail, state=state)
    if tree:
        batch.parent = random_tree_parents(lengths, gen)
        batch.accept = random_leaves(lengths, batch.parent, row_start, gen)
    else:
        batch.parent = chain_parents(lengths)
    return batch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16 tensor, as uint16 (a copy)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


# ---- the affine 4-bit in-projection before the mixer: hidden rows x -> the
# mixer's packed rows qkv and its gate inputs a and b.  Weights come in MLX's
# affine 4-bit form: per output feature n and group g of ``group`` consecutive
# inputs, a bf16 scale and a bf16 bias, and a 4-bit code per weight, eight codes
# a 32-bit word (code j of a word in bits [4j, 4j + 4), word w of a row holding
# inputs 8w .. 8w + 7).  Output features are ordered [qkv (C) | a (hv) | b (hv)].
HIDDEN_2B = 2048     # synthetic hidden sizes of the 2B-like and 27B-like layers
HIDDEN_27B = 5120


@dataclass
class Inproj:
    shape: Shape
    hidden: int
    group: int
    x: torch.Tensor        # bf16 [R][hidden]
    wq: torch.Tensor       # int32 [N][hidden/8]: the packed codes' 32-bit patterns
    scales: torch.Tensor   # bf16 [N][hidden/group]
    biases: torch.Tensor   # bf16 [N][hidden/group]

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def features(self) -> int:
        return inproj_features(self.shape)


def inproj_features(shape: Shape) -> int:
    """Output features of the in-projection: C + 2 hv."""
    return shape.channels + 2 * shape.hv


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [N][K] (values 0..15) into int32 words [N][K/8]."""
    c = codes.astype(np.uint32).reshape(codes.shape[0], -1, 8)
    words = np.zeros(c.shape[:2], np.uint32)
    for j in range(8):
        words |= c[:, :, j] << np.uint32(4 * j)
    return words.view(np.int32)


def make_inproj(shape: Shape, rows: int, hidden: int, group: int, seed: int) -> Inproj:
    """Draw one in-projection call: x ~ N(0, 1); codes uniform in 0..15; per
    group a scale exp(N(0, 0.2)) / (4.6 sqrt(hidden)) and a bias of about
    -7.5 scales (so that the weights are centred, with a standard deviation
    near 1 / sqrt(hidden) and outputs near N(0, 1))."""
    gen = torch.Generator().manual_seed(int(seed))
    n = inproj_features(shape)
    ng = hidden // group
    x = _normal(gen, (rows, hidden), 1.0, torch.bfloat16)
    codes = torch.randint(0, 16, (n, hidden), generator=gen).numpy()
    scale = torch.exp(_normal(gen, (n, ng), 0.2)) / (4.6 * hidden ** 0.5)
    bias = -7.5 * scale * (1.0 + _normal(gen, (n, ng), 0.1))
    return Inproj(shape=shape, hidden=hidden, group=group, x=x,
                  wq=torch.from_numpy(pack_codes(codes)),
                  scales=scale.to(torch.bfloat16), biases=bias.to(torch.bfloat16))


def inproj_workload(name: str, seed: Optional[int] = None):
    """The in-projection's workloads, by name: (shape, rows, hidden, group, seed).

    * ``inproj_decode27b``  16 rows (one decode row of 16 streams), 27B-like layer
    * ``inproj_verify27b``  256 rows (16 streams x 16-row windows), 27B-like layer
    * ``inproj_prefill27b`` 8,306 rows (the four prompts of the prompt pass)
    * ``inproj_window2b``   16 rows, 2B-like layer
    """
    table = {
        "inproj_decode27b": (QWEN_27B, 16, HIDDEN_27B),
        "inproj_verify27b": (QWEN_27B, 256, HIDDEN_27B),
        "inproj_prefill27b": (QWEN_27B, 8306, HIDDEN_27B),
        "inproj_window2b": (QWEN_2B, 16, HIDDEN_2B),
    }
    shape, rows, hidden = table[name]
    if seed is None:
        seed = 1234 + 10 + list(table).index(name)
    return shape, rows, hidden, 64, seed


# Named workloads.  Each returns (shape, lengths, extra keyword arguments).
def workload(name: str, seed: Optional[int] = None):
    """The mixer's reference workloads, by name:

    * ``step``       1 stream, one-row decode step, small layer (hk=2, hv=4, d=64)
    * ``window2b``   1 stream, 16-row verify window, 2B-like layer
    * ``ragged27b``  16 streams with window lengths U{1..16}, 27B-like layer
    * ``verify27b``  16 streams x 16 rows = 256 rows, 27B-like layer
    * ``tree27b``    16 streams x 16-node random best-first trees, 27B-like layer
    * ``prefill27b`` 4 prompts of 512, 1024, 2048 and 4722 rows, 27B-like layer
    """
    ids = {"step": 0, "window2b": 1, "ragged27b": 2, "verify27b": 2, "tree27b": 3,
           "prefill27b": 4}
    if seed is None:
        seed = 1234 + ids[name]
    if name == "step":
        return SMALL, [1], dict(seed=seed)
    if name == "window2b":
        return QWEN_2B, [16], dict(seed=seed)
    if name == "ragged27b":
        gen = torch.Generator().manual_seed(seed + 100)
        return QWEN_27B, ragged_lengths(16, 16, gen), dict(seed=seed)
    if name == "verify27b":
        return QWEN_27B, [16] * 16, dict(seed=seed)
    if name == "tree27b":
        return QWEN_27B, [16] * 16, dict(seed=seed, tree=True)
    if name == "prefill27b":
        return QWEN_27B, [512, 1024, 2048, 4722], dict(seed=seed, zero_state=True)
    raise KeyError(name)
