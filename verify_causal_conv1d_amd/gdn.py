"""ctypes binding of libgdn.so: the same entry points as ``include/libgdn.h``.

Argument marshalling only: torch tensors go in as ``data_ptr()``, the launch
stream is torch's current stream on the tensors' device, and every step of the
computation runs in libgdn's HIP kernels.  A missing or unloadable library
raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading
from typing import Optional

import torch

from .inputs import Shape

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP = 0, -1, -2, -3, -4
MAX_WINDOW_ROWS = 16
PREFILL_SCRATCH_BYTES = 128 * 1024 * 1024   # the fixed workspace of prefill_chunked_noalloc

EXPORTED = (
    "gdn_status_name", "gdn_last_error", "gdn_channels", "gdn_conv_step", "gdn_recur_window",
    "gdn_recur_tree", "gdn_commit", "gdn_recur_log", "gdn_commit_replay",
    "gdn_prefill_workspace_bytes", "gdn_prefill_chunked", "gdn_prefill_chunked_noalloc",
    "gdn_check_layout",
    "gdn_inproj_affine4", "gdn_inproj_pack_affine4", "gdn_inproj_padded_features",
)


class GdnError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {msg} ({status_name(status)})")
        self.status = status


class _Shape(C.Structure):
    _fields_ = [("hk", C.c_int32), ("hv", C.c_int32), ("dk", C.c_int32), ("dv", C.c_int32),
                ("conv_width", C.c_int32)]


class _Params(C.Structure):
    _fields_ = [("conv_w", C.c_void_p), ("a_log", C.c_void_p), ("dt_bias", C.c_void_p)]


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded libgdn.so (built by ``verify_causal_conv1d_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run python -m verify_causal_conv1d_amd.build")
            L = C.CDLL(LIB_PATH)
            P, i32 = C.c_void_p, C.c_int32
            L.gdn_status_name.restype = C.c_char_p
            L.gdn_status_name.argtypes = [C.c_int]
            L.gdn_last_error.restype = C.c_char_p
            L.gdn_channels.restype = i32
            L.gdn_channels.argtypes = [P]
            L.gdn_conv_step.argtypes = [P, P, i32, P, P, P, P, P, P, P]
            L.gdn_recur_window.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
            L.gdn_recur_tree.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P]
            L.gdn_commit.argtypes = [P, i32, i32, P, P, P, P, P, P, P]
            L.gdn_recur_log.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P]
            L.gdn_commit_replay.argtypes = [P, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
            L.gdn_prefill_workspace_bytes.restype = C.c_size_t
            L.gdn_prefill_workspace_bytes.argtypes = [P, i32, i32]
            L.gdn_prefill_chunked.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P, P,
                                              C.c_size_t, P]
            L.gdn_prefill_chunked_noalloc.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P, P]
            L.gdn_check_layout.argtypes = [i32, i32, i32, P, P]
            L.gdn_inproj_affine4.argtypes = [P, i32, i32, i32, P, P, P, P, P, P, P, P]
            L.gdn_inproj_pack_affine4.argtypes = [P, i32, i32, P, P, P, P, P, P, P]
            L.gdn_inproj_padded_features.restype = i32
            L.gdn_inproj_padded_features.argtypes = [P]
            for name in ("gdn_conv_step", "gdn_recur_window", "gdn_recur_tree", "gdn_commit",
                         "gdn_recur_log", "gdn_commit_replay", "gdn_prefill_chunked",
                         "gdn_prefill_chunked_noalloc",
                         "gdn_check_layout", "gdn_inproj_affine4", "gdn_inproj_pack_affine4"):
                getattr(L, name).restype = C.c_int
            _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().gdn_status_name(int(status)).decode()


def _check(status: int, fn: str):
    if status != GDN_OK:
        raise GdnError(status, fn, lib().gdn_last_error().decode())


def _shape(shape: Shape) -> _Shape:
    return _Shape(shape.hk, shape.hv, shape.dk, shape.dv, 4)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


class LayerParams:
    """Device copies of one layer's parameters (conv weights, A_log, dt_bias)."""

    def __init__(self, conv_w: torch.Tensor, a_log: torch.Tensor, dt_bias: torch.Tensor):
        self.conv_w = _dev(conv_w, torch.float32, "conv_w")
        self.a_log = _dev(a_log, torch.float32, "a_log")
        self.dt_bias = _dev(dt_bias, torch.float32, "dt_bias")
        self._c = _Params(self.conv_w.data_ptr(), self.a_log.data_ptr(), self.dt_bias.data_ptr())

    @classmethod
    def from_host(cls, p, device="cuda"):
        return cls(p.conv_w.to(device), p.a_log.to(device), p.dt_bias.to(device))


def channels(shape: Shape) -> int:
    return int(lib().gdn_channels(C.byref(_shape(shape))))


def conv_step(shape: Shape, params: LayerParams, qkv, a, b, conv_tail, state, out):
    """One-row decode step of n streams; conv_tail and state are updated in place."""
    n = qkv.shape[0]
    for t, dt, nm in ((qkv, torch.bfloat16, "qkv"), (a, torch.bfloat16, "a"), (b, torch.bfloat16, "b"),
                      (conv_tail, torch.bfloat16, "conv_tail"), (state, torch.float32, "state"),
                      (out, torch.float32, "out")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    _check(lib().gdn_conv_step(C.byref(sh), C.byref(params._c), n, _ptr(qkv), _ptr(a), _ptr(b),
                               _ptr(conv_tail), _ptr(state), _ptr(out), _stream(qkv)),
           "gdn_conv_step")


def _rows_call(fn, shape, params, row_start, qkv, a, b, conv_tail, state, out, tail_snap,
               state_snap, max_rows, parent=None):
    n = row_start.shape[0] - 1
    total = qkv.shape[0]
    for t, dt, nm in ((row_start, torch.int32, "row_start"), (qkv, torch.bfloat16, "qkv"),
                      (a, torch.bfloat16, "a"), (b, torch.bfloat16, "b"),
                      (conv_tail, torch.bfloat16, "conv_tail"), (state, torch.float32, "state"),
                      (out, torch.float32, "out"), (tail_snap, torch.bfloat16, "tail_snap"),
                      (state_snap, torch.float32, "state_snap")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    args = [C.byref(sh), C.byref(params._c), n, total, int(max_rows), _ptr(row_start)]
    if parent is not None:
        _dev(parent, torch.int32, "parent")
        args.append(_ptr(parent))
    args += [_ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_tail), _ptr(state), _ptr(out),
             _ptr(tail_snap), _ptr(state_snap), _stream(qkv)]
    return getattr(lib(), fn)(*args)


def recur_window(shape, params, row_start, qkv, a, b, conv_tail, state, out, tail_snap,
                 state_snap, max_rows=MAX_WINDOW_ROWS):
    """Verify windows (chains), recording every row's state and tail."""
    _check(_rows_call("gdn_recur_window", shape, params, row_start, qkv, a, b, conv_tail, state,
                      out, tail_snap, state_snap, max_rows), "gdn_recur_window")


def recur_tree(shape, params, row_start, parent, qkv, a, b, conv_tail, state, out, tail_snap,
               state_snap, max_rows=MAX_WINDOW_ROWS):
    """Tree windows: ``parent`` holds local parent indices (-1 = stream state)."""
    _check(_rows_call("gdn_recur_tree", shape, params, row_start, qkv, a, b, conv_tail, state,
                      out, tail_snap, state_snap, max_rows, parent=parent), "gdn_recur_tree")


def commit(shape, row_start, accept_row, tail_snap, state_snap, conv_tail, state):
    """Each stream's accepted row (packed index within its window of
    ``row_start``, -1 = keep) becomes its state and tail."""
    for t, dt, nm in ((row_start, torch.int32, "row_start"), (accept_row, torch.int32, "accept_row"),
                      (tail_snap, torch.bfloat16, "tail_snap"),
                      (state_snap, torch.float32, "state_snap"), (conv_tail, torch.bfloat16, "conv_tail"),
                      (state, torch.float32, "state")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    _check(lib().gdn_commit(C.byref(sh), accept_row.shape[0], state_snap.shape[0], _ptr(row_start),
                            _ptr(accept_row), _ptr(tail_snap), _ptr(state_snap), _ptr(conv_tail), _ptr(state),
                            _stream(state)), "gdn_commit")


def recur_log(shape, params, row_start, qkv, a, b, conv_tail, state, out, log_alpha, log_delta,
              log_key, max_rows=MAX_WINDOW_ROWS, parent=None):
    """Verify windows (parent None) or trees that log every row's decay
    ``log_alpha`` [R][hv], write ``log_delta`` [R][hv][dv] and key ``log_key``
    [R][hk][dk] (fp32) instead of recording its state and tail."""
    n = row_start.shape[0] - 1
    total = qkv.shape[0]
    for t, dt, nm in ((row_start, torch.int32, "row_start"), (qkv, torch.bfloat16, "qkv"),
                      (a, torch.bfloat16, "a"), (b, torch.bfloat16, "b"),
                      (conv_tail, torch.bfloat16, "conv_tail"), (state, torch.float32, "state"),
                      (out, torch.float32, "out"), (log_alpha, torch.float32, "log_alpha"),
                      (log_delta, torch.float32, "log_delta"), (log_key, torch.float32, "log_key")):
        _dev(t, dt, nm)
    if parent is not None:
        _dev(parent, torch.int32, "parent")
    sh = _shape(shape)
    _check(lib().gdn_recur_log(C.byref(sh), C.byref(params._c), n, total, int(max_rows),
                               _ptr(row_start), _ptr(parent), _ptr(qkv), _ptr(a), _ptr(b),
                               _ptr(conv_tail), _ptr(state), _ptr(out), _ptr(log_alpha),
                               _ptr(log_delta), _ptr(log_key), _stream(qkv)), "gdn_recur_log")


def commit_replay(shape, row_start, accept_row, qkv, log_alpha, log_delta, log_key, conv_tail, state,
                  max_rows=MAX_WINDOW_ROWS, parent=None):
    """Each stream's kept path (accepted packed row, -1 = keep) replayed from
    the log onto its state; the path's last raw rows become its conv tail."""
    for t, dt, nm in ((row_start, torch.int32, "row_start"), (accept_row, torch.int32, "accept_row"),
                      (qkv, torch.bfloat16, "qkv"), (log_alpha, torch.float32, "log_alpha"),
                      (log_delta, torch.float32, "log_delta"), (log_key, torch.float32, "log_key"),
                      (conv_tail, torch.bfloat16, "conv_tail"), (state, torch.float32, "state")):
        _dev(t, dt, nm)
    if parent is not None:
        _dev(parent, torch.int32, "parent")
    sh = _shape(shape)
    _check(lib().gdn_commit_replay(C.byref(sh), accept_row.shape[0], qkv.shape[0], int(max_rows),
                                   _ptr(row_start), _ptr(parent), _ptr(accept_row), _ptr(qkv),
                                   _ptr(log_alpha), _ptr(log_delta), _ptr(log_key), _ptr(conv_tail),
                                   _ptr(state), _stream(state)), "gdn_commit_replay")


def prefill_workspace_bytes(shape: Shape, n_seqs: int, total_rows: int) -> int:
    sh = _shape(shape)
    return int(lib().gdn_prefill_workspace_bytes(C.byref(sh), int(n_seqs), int(total_rows)))


def prefill_chunked(shape, params, seq_start, qkv, a, b, conv_tail, state, out, workspace,
                    max_len: int):
    """Chunked prompt passes; conv_tail and state are updated in place."""
    for t, dt, nm in ((seq_start, torch.int32, "seq_start"), (qkv, torch.bfloat16, "qkv"),
                      (a, torch.bfloat16, "a"), (b, torch.bfloat16, "b"),
                      (conv_tail, torch.bfloat16, "conv_tail"), (state, torch.float32, "state"),
                      (out, torch.float32, "out"), (workspace, torch.uint8, "workspace")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    _check(lib().gdn_prefill_chunked(C.byref(sh), C.byref(params._c), seq_start.shape[0] - 1,
                                     qkv.shape[0], int(max_len), _ptr(seq_start), _ptr(qkv),
                                     _ptr(a), _ptr(b), _ptr(conv_tail), _ptr(state), _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(qkv)),
           "gdn_prefill_chunked")


def prefill_chunked_noalloc(shape, params, seq_start, qkv, a, b, conv_tail, state, out, max_len: int):
    """``prefill_chunked`` with the library's fixed workspace (allocates
    nothing; passes needing more than PREFILL_SCRATCH_BYTES are refused)."""
    for t, dt, nm in ((seq_start, torch.int32, "seq_start"), (qkv, torch.bfloat16, "qkv"),
                      (a, torch.bfloat16, "a"), (b, torch.bfloat16, "b"),
                      (conv_tail, torch.bfloat16, "conv_tail"), (state, torch.float32, "state"),
                      (out, torch.float32, "out")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    _check(lib().gdn_prefill_chunked_noalloc(C.byref(sh), C.byref(params._c), seq_start.shape[0] - 1,
                                             qkv.shape[0], int(max_len), _ptr(seq_start), _ptr(qkv),
                                             _ptr(a), _ptr(b), _ptr(conv_tail), _ptr(state), _ptr(out),
                                             _stream(qkv)),
           "gdn_prefill_chunked_noalloc")


def inproj_pack(shape, wq, scales, biases, group: int):
    """Repack affine 4-bit weights (MLX layout: codes int32 [C + 2 hv][hidden/8],
    bf16 scales and biases [C + 2 hv][hidden/group]) into the tiled layout of
    the in-projection kernels; returns (wq_tiled, scales_tiled, biases_tiled)."""
    for t, dt, nm in ((wq, torch.int32, "wq"), (scales, torch.bfloat16, "scales"),
                      (biases, torch.bfloat16, "biases")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    np_ = int(lib().gdn_inproj_padded_features(C.byref(sh)))
    if np_ < 0:
        raise ValueError("bad shape")
    hidden = wq.shape[1] * 8
    wt = torch.empty(np_ * hidden // 8, dtype=torch.int32, device=wq.device)
    st = torch.empty(np_ * hidden // group, dtype=torch.bfloat16, device=wq.device)
    bt = torch.empty_like(st)
    _check(lib().gdn_inproj_pack_affine4(C.byref(sh), hidden, int(group), _ptr(wq), _ptr(scales), _ptr(biases),
                                         _ptr(wt), _ptr(st), _ptr(bt), _stream(wq)), "gdn_inproj_pack_affine4")
    return wt, st, bt


def inproj_affine4(shape, x, wq, scales, biases, qkv, a, b, group: int):
    """The affine 4-bit in-projection: qkv, a, b (bf16, written) from hidden
    rows x (bf16 [R][hidden]) and the tiled weights of ``inproj_pack``."""
    for t, dt, nm in ((x, torch.bfloat16, "x"), (wq, torch.int32, "wq"), (scales, torch.bfloat16, "scales"),
                      (biases, torch.bfloat16, "biases"), (qkv, torch.bfloat16, "qkv"),
                      (a, torch.bfloat16, "a"), (b, torch.bfloat16, "b")):
        _dev(t, dt, nm)
    sh = _shape(shape)
    _check(lib().gdn_inproj_affine4(C.byref(sh), x.shape[0], x.shape[1], int(group), _ptr(x), _ptr(wq),
                                    _ptr(scales), _ptr(biases), _ptr(qkv), _ptr(a), _ptr(b), _stream(x)),
           "gdn_inproj_affine4")


def check_layout(row_start, max_rows: int, total_rows: int, parent=None):
    """Host-side check of a window / tree layout (CPU int32 tensors or arrays)."""
    import numpy as np
    rs = np.ascontiguousarray(np.asarray(row_start), dtype=np.int32)
    par = None if parent is None else np.ascontiguousarray(np.asarray(parent), dtype=np.int32)
    _check(lib().gdn_check_layout(rs.shape[0] - 1, int(total_rows), int(max_rows),
                                  rs.ctypes.data_as(C.c_void_p),
                                  None if par is None else par.ctypes.data_as(C.c_void_p)),
           "gdn_check_layout")
