"""ctypes binding of ``libgdn_oracle.so`` (fp64 reference; test infrastructure).

All arrays are numpy; bf16 tensors travel as their uint16 bit patterns, fp32
parameters as float32, states and results as float64.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np

from . import build_oracle

_lock = threading.Lock()
_lib = None


class OracleShape(C.Structure):
    _fields_ = [("hk", C.c_int32), ("hv", C.c_int32), ("dk", C.c_int32), ("dv", C.c_int32)]


def lib():
    """Loads the oracle library, compiling it first if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(build_oracle.LIB):
                build_oracle.build()
            L = C.CDLL(build_oracle.LIB)
            P = C.c_void_p
            i32 = C.c_int32
            L.gdn_oracle_gates.argtypes = [C.c_double] * 4 + [P, P]
            L.gdn_oracle_conv_silu.argtypes = [i32, P, P, P, P]
            L.gdn_oracle_raw_recurrence.argtypes = [i32, i32, i32] + [P] * 10
            L.gdn_oracle_window.argtypes = [P, P, P, P, i32] + [P] * 17
            L.gdn_oracle_window.restype = i32
            L.gdn_oracle_prefill.argtypes = [P, P, P, P, i32] + [P] * 9
            L.gdn_oracle_prefill.restype = i32
            L.gdn_oracle_commit.argtypes = [P, i32, i32, P, P, P, P, P]
            L.gdn_oracle_commit.restype = i32
            L.gdn_oracle_replay.argtypes = [i32, i32, i32, P, P, P, P]
            L.gdn_oracle_commit_replay.argtypes = [P, i32, P, P, P, P, P, P, P, P, P]
            L.gdn_oracle_commit_replay.restype = i32
            L.gdn_oracle_max_threads.restype = i32
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _shape(shape):
    return OracleShape(shape.hk, shape.hv, shape.dk, shape.dv)


def max_threads() -> int:
    return int(lib().gdn_oracle_max_threads())


def gates(a, b, a_log, dt_bias):
    """(alpha, beta) of one (row, value head), in fp64."""
    al, be = C.c_double(), C.c_double()
    lib().gdn_oracle_gates(float(a), float(b), float(a_log), float(dt_bias),
                           C.byref(al), C.byref(be))
    return al.value, be.value


def conv_silu(conv_w, taps):
    """One row's conv (pre-SiLU) and SiLU output for all channels.
    ``taps`` is four uint16 rows x_{t-3} .. x_t."""
    conv_w = _c(conv_w, np.float32)
    Cn = conv_w.shape[0]
    rows = [_c(t, np.uint16) for t in taps]
    arr = (C.c_void_p * 4)(*[r.ctypes.data for r in rows])
    pre = np.empty(Cn, np.float64)
    post = np.empty(Cn, np.float64)
    lib().gdn_oracle_conv_silu(Cn, _p(conv_w), arr, _p(pre), _p(post))
    return pre, post


def raw_recurrence(alpha, beta, khat, qhat, v, M0, keep_all=False, mag=False):
    """The recurrence on given alpha, beta, khat [T][dk], qhat [T][dk],
    v [T][dv] from M0 [dk][dv].  Returns (M_final, o [T][dv], M_all|None),
    and with ``mag`` a fourth item o_mag [T][dv]: each readout's magnitude
    (each row's step carried out on magnitudes, from |M| of the state it
    starts from, with |khat|, |qhat|, |v|)."""
    khat = _c(khat, np.float64)
    T, dk = khat.shape
    v = _c(v, np.float64)
    dv = v.shape[1]
    M_out = np.empty((dk, dv), np.float64)
    o = np.empty((T, dv), np.float64)
    M_all = np.empty((T, dk, dv), np.float64) if keep_all else None
    o_mag = np.empty((T, dv), np.float64) if mag else None
    lib().gdn_oracle_raw_recurrence(dk, dv, T, _p(_c(alpha, np.float64)),
                                    _p(_c(beta, np.float64)), _p(khat),
                                    _p(_c(qhat, np.float64)), _p(v),
                                    _p(_c(M0, np.float64)), _p(M_out), _p(o), _p(M_all),
                                    _p(o_mag))
    return (M_out, o, M_all, o_mag) if mag else (M_out, o, M_all)


def _window(shape, conv_w, a_log, dt_bias, row_start, parent, qkv, a, b, tail, state,
            snap64, snap32, tail_snap, log, mag, snap_mag):
    row_start = _c(row_start, np.int32)
    n = row_start.shape[0] - 1
    R = int(row_start[-1]) if n > 0 else 0
    Cn = 2 * shape.hk * shape.dk + shape.hv * shape.dv
    o = np.zeros((R, shape.hv, shape.dv), np.float64)
    ts = np.zeros((R, 3, Cn), np.uint16) if tail_snap else None
    s64 = np.zeros((R, shape.hv, shape.dk, shape.dv), np.float64) if snap64 else None
    s32 = np.zeros((R, shape.hv, shape.dk, shape.dv), np.float32) if snap32 else None
    la = np.zeros((R, shape.hv), np.float64) if log else None
    ld = np.zeros((R, shape.hv, shape.dv), np.float64) if log else None
    lk = np.zeros((R, shape.hk, shape.dk), np.float64) if log else None
    om = np.zeros((R, shape.hv, shape.dv), np.float64) if mag else None
    ldm = np.zeros((R, shape.hv, shape.dv), np.float64) if (log and mag) else None
    sm = np.zeros((R, shape.hv, shape.dk, shape.dv), np.float32) if snap_mag else None
    sh = _shape(shape)
    rc = lib().gdn_oracle_window(
        C.byref(sh), _p(_c(conv_w, np.float32)), _p(_c(a_log, np.float32)),
        _p(_c(dt_bias, np.float32)), n, _p(row_start),
        _p(None if parent is None else _c(parent, np.int32)),
        _p(_c(qkv, np.uint16)), _p(_c(a, np.uint16)), _p(_c(b, np.uint16)),
        _p(_c(tail, np.uint16)), _p(_c(state, np.float64)), _p(o), _p(ts), _p(s64), _p(s32),
        _p(la), _p(ld), _p(lk), _p(om), _p(ldm), _p(sm))
    if rc != 0:
        raise ValueError("oracle refused the layout")
    return dict(o=o, o_mag=om, tail_snap=ts, snap64=s64, snap32=s32, snap_mag=sm, log_alpha=la,
                log_delta=ld, log_key=lk, log_delta_mag=ldm)


def window(shape, conv_w, a_log, dt_bias, row_start, qkv, a, b, tail, state, *,
           snap64=True, snap32=False, tail_snap=True, log=False, mag=False, snap_mag=False):
    """Verify windows: each stream's rows form a chain.  Returns a dict with
    ``o`` [R][hv][dv], ``tail_snap`` [R][3][C] (uint16), the per-row states
    ``snap64`` (fp64) and/or ``snap32`` (rounded to fp32), and with ``log``
    each row's decay ``log_alpha`` [R][hv], write ``log_delta`` [R][hv][dv]
    and key ``log_key`` [R][hk][dk].  With ``mag`` also the magnitudes
    ``o_mag`` of o (and ``log_delta_mag`` of the writes), with ``snap_mag``
    those of the per-row states (fp32).

    A magnitude is the row's step carried out on magnitudes, from the state
    the row starts from: |M| and the inputs' absolute values, every sum by
    the sum of its terms' magnitudes, every product by the product of
    magnitudes, SiLU's output by its gate sigmoid(y) times the conv's term
    magnitude.  It scales what rounding can do to a value whose terms
    cancel."""
    return _window(shape, conv_w, a_log, dt_bias, row_start, None, qkv, a, b, tail, state,
                   snap64, snap32, tail_snap, log, mag, snap_mag)


def tree(shape, conv_w, a_log, dt_bias, row_start, parent, qkv, a, b, tail, state, *,
         snap64=True, snap32=False, tail_snap=True, log=False, mag=False, snap_mag=False):
    """Tree windows: ``parent`` [R] holds each row's parent as a local index
    in its stream's window (-1 = the stream's own state and tail)."""
    return _window(shape, conv_w, a_log, dt_bias, row_start, parent, qkv, a, b, tail, state,
                   snap64, snap32, tail_snap, log, mag, snap_mag)


def replay(alpha, delta, key, M):
    """Logged rows replayed onto one head's state M [dk][dv] (fp64, a new
    array): M <- alpha_t M + key_t delta_t^T for t in order."""
    key = _c(np.atleast_2d(key), np.float64)
    delta = _c(np.atleast_2d(delta), np.float64)
    out = np.array(M, dtype=np.float64, copy=True, order="C")
    dk, dv = out.shape
    lib().gdn_oracle_replay(dk, dv, key.shape[0], _p(_c(np.atleast_1d(alpha), np.float64)),
                            _p(delta), _p(key), _p(out))
    return out


def commit_replay(shape, row_start, parent, accept, qkv, log_alpha, log_delta, log_key, tail, state):
    """Returns (tail, state) after replaying each stream's kept path (accept:
    packed row index within the stream's window, or -1)."""
    row_start = _c(row_start, np.int32)
    accept = _c(accept, np.int32)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    tl = np.array(tail, dtype=np.uint16, copy=True, order="C")
    sh = _shape(shape)
    rc = lib().gdn_oracle_commit_replay(
        C.byref(sh), accept.shape[0], _p(row_start),
        _p(None if parent is None else _c(parent, np.int32)), _p(accept), _p(_c(qkv, np.uint16)),
        _p(_c(log_alpha, np.float64)), _p(_c(log_delta, np.float64)), _p(_c(log_key, np.float64)),
        _p(tl), _p(st))
    if rc != 0:
        raise ValueError("oracle refused the layout or the accepted rows")
    return tl, st


def prefill(shape, conv_w, a_log, dt_bias, seq_start, qkv, a, b, tail, state, mag=False):
    """Prompt passes (recurrent form).  Returns (o, final_state fp64, final_tail),
    and with ``mag`` two more items: the magnitudes of o and of the final
    states (see ``window``)."""
    seq_start = _c(seq_start, np.int32)
    n = seq_start.shape[0] - 1
    T = int(seq_start[-1]) if n > 0 else 0
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    tl = np.array(tail, dtype=np.uint16, copy=True, order="C")
    o = np.zeros((T, shape.hv, shape.dv), np.float64)
    om = np.zeros((T, shape.hv, shape.dv), np.float64) if mag else None
    fm = np.zeros((n, shape.hv, shape.dk, shape.dv), np.float64) if mag else None
    sh = _shape(shape)
    rc = lib().gdn_oracle_prefill(
        C.byref(sh), _p(_c(conv_w, np.float32)), _p(_c(a_log, np.float32)),
        _p(_c(dt_bias, np.float32)), n, _p(seq_start), _p(_c(qkv, np.uint16)),
        _p(_c(a, np.uint16)), _p(_c(b, np.uint16)), _p(tl), _p(st), _p(o), _p(om), _p(fm))
    if rc != 0:
        raise ValueError("oracle refused the layout")
    return (o, st, tl, om, fm) if mag else (o, st, tl)


def commit(shape, accept, tail_snap, snap64, tail, state):
    """Returns (tail, state) after committing each stream's accepted row."""
    accept = _c(accept, np.int32)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    tl = np.array(tail, dtype=np.uint16, copy=True, order="C")
    sh = _shape(shape)
    rc = lib().gdn_oracle_commit(C.byref(sh), accept.shape[0], snap64.shape[0], _p(accept),
                                 _p(_c(tail_snap, np.uint16)), _p(_c(snap64, np.float64)),
                                 _p(tl), _p(st))
    if rc != 0:
        raise ValueError("oracle refused the accepted rows")
    return tl, st
