"""Pins of the oracle's log of a verify pass and of its commit by replay.

A verify pass may log each row's decay, write and key instead of its state,
and keeping a row replays the kept path (page "perf(qwen3_5 cuda): deliver the
first token before drafting", commit note on tree-shaped verify windows).
The log is pinned against the oracle's recorded states (themselves pinned in
``test_oracle.py``): replaying a row's path from the stream's state reaches
that row's state, the logged key is the row's khat, the logged decay is the
gate, and with alpha = beta = 1 the logged write is exactly what makes the
key read back v.  The commit by replay is pinned against the snapshot commit.
"""
import numpy as np
import pytest

import oracle
from verify_causal_conv1d_amd import inputs as gi

TINY = gi.Shape(hk=2, hv=4, dk=8, dv=6)


def _np_batch(b: gi.Batch):
    return dict(conv_w=b.params.conv_w.numpy(), a_log=b.params.a_log.numpy(),
                dt_bias=b.params.dt_bias.numpy(), row_start=b.row_start.numpy(),
                qkv=gi.bf16_bits(b.qkv), a=gi.bf16_bits(b.a), b=gi.bf16_bits(b.b),
                tail=gi.bf16_bits(b.tail), state=b.state.numpy().astype(np.float64))


def _pass(shape, d, parent, **kw):
    if parent is None:
        return oracle.window(shape, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"],
                             d["qkv"], d["a"], d["b"], d["tail"], d["state"], log=True, **kw)
    return oracle.tree(shape, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"], parent,
                       d["qkv"], d["a"], d["b"], d["tail"], d["state"], log=True, **kw)


def _bf(bits):
    """The value of one bf16 bit pattern."""
    return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])


def _path(parent_local, t):
    return gi.path_to_root(parent_local, t) if parent_local is not None else list(range(t + 1))


@pytest.mark.parametrize("tree", [False, True])
def test_replaying_a_rows_path_reaches_its_state(tree):
    batch = gi.make_batch(TINY, [7, 1, 5], seed=41, tree=tree)
    d = _np_batch(batch)
    par = batch.parent.numpy() if tree else None
    res = _pass(TINY, d, par)
    r = TINY.hv // TINY.hk
    for s, ln in enumerate(batch.lengths()):
        r0 = int(d["row_start"][s])
        local = par[r0:r0 + ln].tolist() if tree else None
        for t in range(ln):
            rows = [r0 + i for i in _path(local, t)]
            for h in range(TINY.hv):
                M = oracle.replay(res["log_alpha"][rows, h], res["log_delta"][rows, h],
                                  res["log_key"][rows, h // r], d["state"][s, h])
                ref = res["snap64"][r0 + t, h]
                assert np.max(np.abs(M - ref)) <= 1e-13 * max(1.0, np.abs(ref).max()), (s, t, h)


def test_logged_decay_and_key_are_the_rows_gate_and_khat():
    batch = gi.make_batch(TINY, [4, 3], seed=42)
    d = _np_batch(batch)
    res = _pass(TINY, d, None)
    Cn = TINY.channels
    hkdk = TINY.hk * TINY.dk
    for s, ln in enumerate(batch.lengths()):
        r0 = int(d["row_start"][s])
        hist = list(d["tail"][s])
        for t in range(ln):
            row = r0 + t
            hist.append(d["qkv"][row])
            for h in range(TINY.hv):
                al, _ = oracle.gates(_bf(d["a"][row, h]), _bf(d["b"][row, h]),
                                     d["a_log"][h], d["dt_bias"][h])
                assert res["log_alpha"][row, h] == al
            _, post = oracle.conv_silu(d["conv_w"], hist[-4:])
            kk = post[hkdk:2 * hkdk].reshape(TINY.hk, TINY.dk)
            khat = kk / np.sqrt((kk * kk).sum(axis=1, keepdims=True) + 1e-6)
            assert np.allclose(res["log_key"][row], khat, rtol=1e-14, atol=1e-15)
    assert Cn == d["qkv"].shape[1]


def test_unit_gates_write_makes_the_key_read_back_v():
    """alpha = beta = 1: the logged write is delta = v - M_p^T khat, so the kept
    state reads v back along khat up to the normalisation's eps:
    M_t^T khat = M_p^T khat + delta |khat|^2."""
    shape = gi.Shape(hk=2, hv=4, dk=16, dv=8)
    batch = gi.make_batch(shape, [4], seed=43)
    d = _np_batch(batch)
    d["a_log"][:] = -np.inf
    d["b"][:] = np.uint16(0x7F80)   # +inf: beta = 1
    res = _pass(shape, d, None)
    r = shape.hv // shape.hk
    hkdk = shape.hk * shape.dk
    hist = list(d["tail"][0])
    M_prev = d["state"][0]
    for t in range(4):
        hist.append(d["qkv"][t])
        _, post = oracle.conv_silu(d["conv_w"], hist[-4:])
        vrow = post[2 * hkdk:].reshape(shape.hv, shape.dv)
        for h in range(shape.hv):
            k = res["log_key"][t, h // r]
            assert res["log_alpha"][t, h] == 1.0
            assert np.allclose(res["log_delta"][t, h], vrow[h] - M_prev[h].T @ k, rtol=0, atol=1e-12)
            read = res["snap64"][t, h].T @ k
            assert np.allclose(read, vrow[h], rtol=0, atol=1e-5 * (1 + np.abs(vrow[h]).max()))
        M_prev = res["snap64"][t]


def test_replay_special_cases():
    rng = np.random.default_rng(5)
    M0 = rng.standard_normal((4, 3))
    k = rng.standard_normal((2, 4))
    # no write: pure decay, exactly
    assert np.array_equal(oracle.replay([0.5, 0.25], np.zeros((2, 3)), k, M0), M0 * 0.125)
    # from zero: the sum of the rank-one writes, the earlier one decayed
    dl = rng.standard_normal((2, 3))
    M = oracle.replay([1.0, 0.5], dl, k, np.zeros((4, 3)))
    assert np.allclose(M, 0.5 * np.outer(k[0], dl[0]) + np.outer(k[1], dl[1]), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("tree", [False, True])
def test_commit_by_replay_equals_commit_of_snapshots(tree):
    batch = gi.make_batch(TINY, [6, 2, 5, 1], seed=44, tree=tree)
    d = _np_batch(batch)
    par = batch.parent.numpy() if tree else None
    res = _pass(TINY, d, par)
    rs = d["row_start"]
    cases = [
        [int(rs[1]) - 1, int(rs[2]) - 1, int(rs[3]) - 1, int(rs[4]) - 1],   # last rows
        [int(rs[0]), -1, int(rs[2]) + 1, int(rs[3])],                        # short paths, a kept stream
    ]
    if tree:
        cases.append(batch.accept.numpy().tolist())
    for acc in cases:
        acc = np.array(acc, np.int32)
        tl, st = oracle.commit_replay(TINY, rs, par, acc, d["qkv"], res["log_alpha"],
                                      res["log_delta"], res["log_key"], d["tail"], d["state"])
        tl_ref, st_ref = oracle.commit(TINY, acc, res["tail_snap"], res["snap64"], d["tail"], d["state"])
        assert np.array_equal(tl, tl_ref), acc
        assert np.max(np.abs(st - st_ref)) <= 1e-13 * max(1.0, np.abs(st_ref).max()), acc


def test_commit_by_replay_refuses_rows_outside_the_window():
    batch = gi.make_batch(TINY, [3, 2], seed=45)
    d = _np_batch(batch)
    res = _pass(TINY, d, None)
    for acc in ([3, -1], [0, 0], [-2, -1]):   # row 3 is stream 1's, row 0 stream 0's
        with pytest.raises(ValueError):
            oracle.commit_replay(TINY, d["row_start"], None, np.array(acc, np.int32), d["qkv"],
                                 res["log_alpha"], res["log_delta"], res["log_key"], d["tail"],
                                 d["state"])
