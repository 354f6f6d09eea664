"""The C ABI without a GPU: symbols, status names and every host-side refusal.

Every call here is refused by the host-side checks before any HIP call is
made, so nothing runs on a device.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from verify_causal_conv1d_amd import gdn
from verify_causal_conv1d_amd import inputs as gi
from verify_causal_conv1d_amd.inputs import QWEN_27B, SMALL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgdn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        from verify_causal_conv1d_amd import build
        build.build()
    return gdn.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), f"{name} declared in libgdn.h but not exported"
    assert sorted(gdn.EXPORTED) == names


def test_status_names(L):
    assert gdn.status_name(0) == "GDN_OK"
    assert gdn.status_name(-1) == "GDN_EINVAL"
    assert gdn.status_name(-2) == "GDN_EUNSUPPORTED"
    assert gdn.status_name(-3) == "GDN_EWORKSPACE"
    assert gdn.status_name(-4) == "GDN_EHIP"
    assert gdn.status_name(-99) == "GDN_UNKNOWN"


def _shape(hk=16, hv=48, dk=128, dv=128, cw=4):
    return gdn._Shape(hk, hv, dk, dv, cw)


def test_channels(L):
    assert gdn.channels(QWEN_27B) == 10240
    assert gdn.channels(SMALL) == 512
    for bad in (_shape(hk=0), _shape(hv=47), _shape(dk=96), _shape(dv=32), _shape(cw=3)):
        assert L.gdn_channels(C.byref(bad)) == -1


# Fake device pointers: never dereferenced, because every call below is refused first.
P16 = C.c_void_p(0x10000)
P_ODD = C.c_void_p(0x10004)


def _params(ok=True):
    return gdn._Params(0x20000 if ok else 0, 0x30000, 0x40000)


def window(L, shape=None, params=None, n=16, total=256, max_rows=16, row_start=P16, qkv=P16,
           a=P16, b=P16, tail=P16, state=P16, out=P16, tsnap=P16, ssnap=P16):
    shape = shape or _shape()
    params = params or _params()
    return L.gdn_recur_window(C.byref(shape), C.byref(params), n, total, max_rows, row_start, qkv,
                              a, b, tail, state, out, tsnap, ssnap, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(shape=_shape(hk=0)), gdn.GDN_EINVAL, "positive"),
    (dict(shape=_shape(hv=40, hk=16)), gdn.GDN_EINVAL, "multiple"),
    (dict(shape=_shape(cw=3)), gdn.GDN_EUNSUPPORTED, "conv_width"),
    (dict(shape=_shape(dk=96)), gdn.GDN_EUNSUPPORTED, "dk"),
    (dict(shape=_shape(dv=256)), gdn.GDN_EUNSUPPORTED, "dv"),
    (dict(params=gdn._Params(0, 1, 2)), gdn.GDN_EINVAL, "NULL"),
    (dict(n=-1), gdn.GDN_EINVAL, "negative"),
    (dict(total=-5), gdn.GDN_EINVAL, "negative"),
    (dict(max_rows=0), gdn.GDN_EINVAL, "max_rows"),
    (dict(max_rows=17), gdn.GDN_EINVAL, "max_rows"),
    (dict(total=257), gdn.GDN_EINVAL, "exceeds"),
    (dict(row_start=None), gdn.GDN_EINVAL, "row_start"),
    (dict(qkv=None), gdn.GDN_EINVAL, "qkv"),
    (dict(qkv=P_ODD), gdn.GDN_EINVAL, "aligned"),
    (dict(a=None), gdn.GDN_EINVAL, "a or b"),
    (dict(tail=None), gdn.GDN_EINVAL, "conv_tail"),
    (dict(state=None), gdn.GDN_EINVAL, "state"),
    (dict(out=None), gdn.GDN_EINVAL, "out"),
    (dict(tsnap=None), gdn.GDN_EINVAL, "tail_snap"),
    (dict(ssnap=P_ODD), gdn.GDN_EINVAL, "state_snap"),
])
def test_window_refusals(L, kw, code, needle):
    assert window(L, **kw) == code
    assert needle in L.gdn_last_error().decode()


def test_empty_calls_do_nothing(L):
    # no streams / no rows: accepted without touching any pointer
    assert window(L, n=0, total=0, row_start=None, qkv=None) == gdn.GDN_OK
    assert window(L, n=4, total=0, row_start=None, qkv=None) == gdn.GDN_OK
    sh = _shape()
    assert L.gdn_conv_step(C.byref(sh), C.byref(_params()), 0, None, None, None, None, None, None,
                           None) == gdn.GDN_OK
    assert L.gdn_commit(C.byref(sh), 0, 0, None, None, None, None, None, None, None) == gdn.GDN_OK


def test_tree_needs_parents(L):
    sh, pa = _shape(), _params()
    rc = L.gdn_recur_tree(C.byref(sh), C.byref(pa), 16, 256, 16, P16, None, P16, P16, P16, P16, P16,
                          P16, P16, P16, None)
    assert rc == gdn.GDN_EINVAL and "parent" in L.gdn_last_error().decode()


def test_step_refusals(L):
    sh, pa = _shape(), _params()
    assert L.gdn_conv_step(C.byref(sh), C.byref(pa), 2, None, P16, P16, P16, P16, P16, None) == gdn.GDN_EINVAL
    assert L.gdn_conv_step(C.byref(sh), C.byref(pa), -1, P16, P16, P16, P16, P16, P16, None) == gdn.GDN_EINVAL
    # nine value heads of 128 per key head need more than one workgroup
    wide = _shape(hk=1, hv=9)
    assert L.gdn_conv_step(C.byref(wide), C.byref(pa), 1, P16, P16, P16, P16, P16, P16,
                           None) == gdn.GDN_EUNSUPPORTED


def test_commit_refusals(L):
    sh = _shape()
    assert L.gdn_commit(C.byref(sh), 2, 10, P16, None, P16, P16, P16, P16, None) == gdn.GDN_EINVAL
    assert "accept_row" in L.gdn_last_error().decode()
    assert L.gdn_commit(C.byref(sh), 2, 10, None, P16, P16, P16, P16, P16, None) == gdn.GDN_EINVAL
    assert "row_start" in L.gdn_last_error().decode()
    assert L.gdn_commit(C.byref(sh), -1, 10, P16, P16, P16, P16, P16, P16, None) == gdn.GDN_EINVAL
    assert L.gdn_commit(C.byref(sh), 2, 10, P16, P16, P16, P16, P16, P_ODD, None) == gdn.GDN_EINVAL


def test_log_refusals(L):
    sh, pa = _shape(), _params()

    def log(n=16, total=256, max_rows=16, parent=None, la=P16, ld=P16, lk=P16):
        return L.gdn_recur_log(C.byref(sh), C.byref(pa), n, total, max_rows, P16, parent, P16, P16,
                               P16, P16, P16, P16, la, ld, lk, None)
    assert log(la=None) == gdn.GDN_EINVAL and "log_alpha" in L.gdn_last_error().decode()
    assert log(ld=P_ODD) == gdn.GDN_EINVAL and "log_delta" in L.gdn_last_error().decode()
    assert log(lk=None) == gdn.GDN_EINVAL and "log_key" in L.gdn_last_error().decode()
    assert log(max_rows=17) == gdn.GDN_EINVAL
    assert log(total=257) == gdn.GDN_EINVAL
    assert log(n=0, total=0) == gdn.GDN_OK

    def replay(n=16, total=256, max_rows=16, rs=P16, acc=P16, la=P16, state=P16):
        return L.gdn_commit_replay(C.byref(sh), n, total, max_rows, rs, None, acc, P16, la, P16, P16,
                                   P16, state, None)
    assert replay(rs=None) == gdn.GDN_EINVAL and "row_start" in L.gdn_last_error().decode()
    assert replay(acc=None) == gdn.GDN_EINVAL and "accept_row" in L.gdn_last_error().decode()
    assert replay(la=None) == gdn.GDN_EINVAL and "log_alpha" in L.gdn_last_error().decode()
    assert replay(state=P_ODD) == gdn.GDN_EINVAL and "state" in L.gdn_last_error().decode()
    assert replay(max_rows=0) == gdn.GDN_EINVAL
    assert replay(n=-1) == gdn.GDN_EINVAL
    assert replay(n=0, total=0, rs=None, acc=None) == gdn.GDN_OK


def test_prefill_refusals(L):
    sh, pa = _shape(), _params()

    def call(n=4, total=100, max_len=50, seq=P16, ws=P16, wsb=1 << 40, shape=sh):
        return L.gdn_prefill_chunked(C.byref(shape), C.byref(pa), n, total, max_len, seq, P16, P16,
                                     P16, P16, P16, P16, ws, wsb, None)
    assert call(n=-1) == gdn.GDN_EINVAL
    assert call(max_len=0) == gdn.GDN_EINVAL
    assert call(max_len=101) == gdn.GDN_EINVAL
    assert call(n=0, total=0, seq=None) == gdn.GDN_OK
    small = _shape(hk=2, hv=4, dk=64, dv=64)
    assert call(shape=small) == gdn.GDN_EUNSUPPORTED
    assert call(wsb=1) == gdn.GDN_EWORKSPACE
    assert call(ws=None) == gdn.GDN_EWORKSPACE
    assert call(ws=P_ODD) == gdn.GDN_EINVAL


def test_prefill_noalloc_refusals(L):
    """The allocation-free prompt pass refuses, before any device call, what
    gdn_prefill_chunked refuses, and any pass whose workspace is over its
    fixed array."""
    sh, pa = _shape(), _params()

    rows = 64     # the fewest rows of one prompt over the fixed array
    while gdn.prefill_workspace_bytes(gi.QWEN_27B, 1, rows) <= gdn.PREFILL_SCRATCH_BYTES:
        rows += 64

    def call(n=1, total=rows, max_len=rows, seq=P16, qkv=P16, shape=sh):
        return L.gdn_prefill_chunked_noalloc(C.byref(shape), C.byref(pa), n, total, max_len, seq, qkv, P16,
                                             P16, P16, P16, P16, None)
    assert call() == gdn.GDN_EWORKSPACE and "pieces" in L.gdn_last_error().decode()
    assert call(n=-1) == gdn.GDN_EINVAL
    assert call(max_len=0) == gdn.GDN_EINVAL
    assert call(seq=None) == gdn.GDN_EINVAL
    assert call(qkv=P_ODD) == gdn.GDN_EINVAL
    assert call(shape=_shape(hk=2, hv=4, dk=64, dv=64)) == gdn.GDN_EUNSUPPORTED
    assert call(n=0, total=0, seq=None) == gdn.GDN_OK


def test_inproj_refusals(L):
    sh = _shape()

    def call(rows=16, hidden=5120, group=64, x=P16, wq=P16, sc=P16, qkv=P16, a=P16, shape=sh):
        return L.gdn_inproj_affine4(C.byref(shape), rows, hidden, group, x, wq, sc, P16, qkv, a, P16, None)
    assert call(rows=-1) == gdn.GDN_EINVAL
    assert call(hidden=5000) == gdn.GDN_EUNSUPPORTED and "hidden" in L.gdn_last_error().decode()
    assert call(hidden=0) == gdn.GDN_EUNSUPPORTED
    assert call(group=16) == gdn.GDN_EUNSUPPORTED and "group" in L.gdn_last_error().decode()
    assert call(x=None) == gdn.GDN_EINVAL and "x" in L.gdn_last_error().decode()
    assert call(wq=P_ODD) == gdn.GDN_EINVAL and "wq" in L.gdn_last_error().decode()
    assert call(sc=None) == gdn.GDN_EINVAL
    assert call(qkv=None) == gdn.GDN_EINVAL
    assert call(a=None) == gdn.GDN_EINVAL
    assert call(rows=0, x=None, wq=None, sc=None, qkv=None, a=None) == gdn.GDN_OK
    assert call(shape=_shape(hv=47)) == gdn.GDN_EINVAL

    def pack(hidden=5120, group=64, wq=P16, wt=P16, st=P16):
        return L.gdn_inproj_pack_affine4(C.byref(sh), hidden, group, wq, P16, P16, wt, st, P16, None)
    assert pack(hidden=100) == gdn.GDN_EUNSUPPORTED
    assert pack(group=256) == gdn.GDN_EUNSUPPORTED
    assert pack(wq=None) == gdn.GDN_EINVAL
    assert pack(wt=P_ODD) == gdn.GDN_EINVAL and "wq_tiled" in L.gdn_last_error().decode()
    assert pack(st=None) == gdn.GDN_EINVAL
    # features padded to a multiple of 16: 10240 + 96 at the 27B-like layer, 512 + 8 -> 528
    assert L.gdn_inproj_padded_features(C.byref(sh)) == 10336
    assert L.gdn_inproj_padded_features(C.byref(_shape(hk=2, hv=4, dk=64, dv=64))) == 528
    assert L.gdn_inproj_padded_features(C.byref(_shape(hv=47))) == -1


def test_prefill_workspace_bytes(L):
    sh = _shape()
    n, T, hk, hv, d = 4, 8306, 16, 48, 128
    need = L.gdn_prefill_workspace_bytes(C.byref(sh), n, T)
    # per chunk and value head (at most T/64 + n chunks): the sweep's bf16
    # operand block (W: 64 x dk; U~: 64 x dv; P: 64 x 64) and its gates
    # (fp32: e^{gamma_L}, e^gamma and e^{gamma_L - gamma} of each row, 132
    # floats); per chunk and key head the shared fragments (K K^T and Q K^T in
    # fp32, k^ and q^ fragments in bf16: 4 x 64 x 64 x 4 bytes); nothing per row
    nc = T // 64 + n
    blk = (64 * d + 64 * d + 64 * 64) * 2
    frag = 4 * 64 * 64 * 4
    lower = nc * hv * (blk + 132 * 4) + nc * hk * frag
    assert lower <= need <= lower + 3 * 256
    assert L.gdn_prefill_workspace_bytes(C.byref(_shape(dk=64)), 4, 100) == 0


def test_check_layout(L):
    gdn.check_layout([0, 3, 3, 19], max_rows=16, total_rows=19)
    with pytest.raises(gdn.GdnError, match="max_rows"):
        gdn.check_layout([0, 17], max_rows=16, total_rows=17)
    with pytest.raises(gdn.GdnError, match="decreases"):
        gdn.check_layout([0, 5, 4], max_rows=16, total_rows=5)
    with pytest.raises(gdn.GdnError, match="past"):
        gdn.check_layout([0, 5, 9], max_rows=16, total_rows=8)
    gdn.check_layout([0, 3], 16, 3, parent=[-1, 0, 0])
    with pytest.raises(gdn.GdnError, match="parent"):
        gdn.check_layout([0, 3], 16, 3, parent=[-1, 0, 2])
    with pytest.raises(gdn.GdnError, match="parent"):
        gdn.check_layout([0, 2], 16, 2, parent=[0, 0])
