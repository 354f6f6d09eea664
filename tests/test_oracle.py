"""Pins of the fp64 oracle against what the mathematics and the pages fix.

Each test checks the oracle against something other than itself: special
values of the gates, exact dyadic cases of the update, brute-force matrix
products on tiny heads, a hand-worked example, identities of the conv and of
SiLU, and structural facts of windows and trees (a window equals its one-row
steps; a tree's path equals the chain over that path).  The chunked (WY) form
is pinned against the recurrence in ``test_chunked_algebra.py``.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from verify_causal_conv1d_amd import inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF16_NEG_INF = np.uint16(0xFF80)
BF16_POS_INF = np.uint16(0x7F80)


def bf16(x):
    return gi.bf16_bits(torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16))


# --------------------------------------------------------------------------- gates

def test_gates_special_values_are_exact():
    # b = -inf gives beta = 0, b = +inf gives beta = 1, A_log = -inf gives alpha = 1
    assert oracle.gates(0.3, -math.inf, 1.0, 0.0)[1] == 0.0
    assert oracle.gates(0.3, math.inf, 1.0, 0.0)[1] == 1.0
    assert oracle.gates(0.3, 0.0, -math.inf, 0.1)[0] == 1.0


def test_gates_closed_forms():
    # softplus(0) = ln 2, so A_log = ln n and a + dt_bias = 0 give alpha = 2^-n
    for n in (1, 2, 3, 5):
        al, be = oracle.gates(0.25, 0.0, math.log(n), -0.25)
        assert abs(al - 2.0 ** (-n)) <= 4e-16 * n
        assert be == 0.5
    # sigmoid(ln 3) = 3/4
    assert abs(oracle.gates(0.0, math.log(3.0), 0.0, 0.0)[1] - 0.75) < 1e-15
    # softplus(x) -> x for large x: alpha = e^{-x}
    al, _ = oracle.gates(30.0, 0.0, 0.0, 0.0)
    assert abs(al / math.exp(-30.0) - 1) < 1e-12
    # softplus(x) -> e^x for very negative x: A_log = 30, x = -30 give
    # g = -e^30 * softplus(-30) = -(1 - e^-30 / 2 + ...), so alpha = 1/e
    al, _ = oracle.gates(-30.0, 0.0, 30.0, 0.0)
    assert abs(al * math.e - 1) < 1e-12
    # monotone: a larger decay rate gives a smaller alpha
    vals = [oracle.gates(0.0, 0.0, la, 0.0)[0] for la in np.linspace(-2, 3, 11)]
    assert all(x > y for x, y in zip(vals, vals[1:]))


# --------------------------------------------------------------------------- conv / SiLU

def test_conv_single_tap_selects_that_row():
    rng = np.random.default_rng(0)
    Cn = 37
    taps = [bf16(rng.standard_normal(Cn)) for _ in range(4)]
    vals = [t.astype(np.uint32) << 16 for t in taps]
    vals = [v.view(np.float32).astype(np.float64) for v in vals]
    for j in range(4):
        w = np.zeros((Cn, 4), np.float32)
        w[:, j] = 1.0
        pre, _ = oracle.conv_silu(w, taps)
        assert np.array_equal(pre, vals[j]), f"tap {j} must read x_(t-3+{j})"


def test_conv_is_linear_in_weights_and_rows():
    rng = np.random.default_rng(1)
    Cn = 64
    taps = [bf16(rng.standard_normal(Cn)) for _ in range(4)]
    w1 = rng.standard_normal((Cn, 4)).astype(np.float32)
    w2 = rng.standard_normal((Cn, 4)).astype(np.float32)
    p1, _ = oracle.conv_silu(w1, taps)
    p2, _ = oracle.conv_silu(w2, taps)
    p12, _ = oracle.conv_silu((w1.astype(np.float64) + w2).astype(np.float32), taps)
    # w1 + w2 rounds to fp32; allow that rounding
    assert np.max(np.abs(p12 - (p1 + p2))) < 1e-5
    # a zero row contributes nothing: shifting the taps by one with a zero
    # oldest row equals dropping the oldest tap's weight
    z = np.zeros(Cn, np.uint16)
    pa, _ = oracle.conv_silu(w1, [z, taps[1], taps[2], taps[3]])
    w1b = w1.copy()
    w1b[:, 0] = 0
    pb, _ = oracle.conv_silu(w1b, taps)
    assert np.array_equal(pa, pb)


def test_silu_identities():
    rng = np.random.default_rng(2)
    Cn = 50
    x = bf16(rng.standard_normal(Cn) * 3)
    z = np.zeros(Cn, np.uint16)
    w = np.zeros((Cn, 4), np.float32)
    w[:, 3] = 1.0
    pre, post = oracle.conv_silu(w, [z, z, z, x])
    wn = -w
    pre_n, post_n = oracle.conv_silu(wn, [z, z, z, x])
    assert np.array_equal(pre_n, -pre)
    # silu(y) - silu(-y) = y exactly in real arithmetic
    assert np.max(np.abs((post - post_n) - pre)) < 1e-15 * (1 + np.abs(pre)).max()
    # silu(0) = 0, silu(y) ~ y for large y, ~0 for very negative y
    _, p0 = oracle.conv_silu(w, [z, z, z, np.zeros(Cn, np.uint16)])
    assert np.all(p0 == 0)
    big = bf16(np.full(Cn, 60.0))
    _, pb = oracle.conv_silu(w, [z, z, z, big])
    assert np.allclose(pb, 60.0, rtol=1e-20, atol=1e-20)
    _, pn = oracle.conv_silu(w, [z, z, z, bf16(np.full(Cn, -60.0))])
    assert np.all(np.abs(pn) < 1e-24) and np.all(pn <= 0)
    # silu is 1/2 * y at y -> 0 to first order: silu(y)/y -> 1/2
    small = bf16(np.full(Cn, 2.0 ** -20))
    _, ps = oracle.conv_silu(w, [z, z, z, small])
    assert np.allclose(ps / 2.0 ** -20, 0.5, rtol=1e-6)


# --------------------------------------------------------------------------- raw recurrence

def _read_golden():
    recs = {"in": [], "o": [], "M": [], "mag": []}
    M0 = None
    with open(os.path.join(GOLDEN, "raw_recurrence_worked.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            vals = [float(v) for v in vals]
            if tag == "M0":
                M0 = np.array(vals).reshape(2, 2)
            else:
                recs[tag].append(vals)
    return M0, recs


def test_hand_worked_example():
    M0, recs = _read_golden()
    rows = np.array(recs["in"])
    alpha, beta = rows[:, 1], rows[:, 2]
    k, v, q = rows[:, 3:5], rows[:, 5:7], rows[:, 7:9]
    M, o, M_all, mag = oracle.raw_recurrence(alpha, beta, k, q, v, M0, keep_all=True, mag=True)
    for t, rec in enumerate(recs["o"]):
        assert np.allclose(o[t], rec[1:], rtol=0, atol=1e-14), (t, o[t], rec)
    for t, rec in enumerate(recs["M"]):
        assert np.allclose(M_all[t].ravel(), rec[1:], rtol=0, atol=1e-14), (t, M_all[t], rec)
    for t, rec in enumerate(recs["mag"]):
        assert np.allclose(mag[t], rec[1:], rtol=0, atol=1e-14), (t, mag[t], rec)
    assert np.array_equal(M, M_all[-1])
    assert len(recs["mag"]) == len(recs["o"]) == 4


def test_readout_magnitude_bounds_and_equalities():
    """The readout magnitude (the row's step carried out on magnitudes) is at least
    |o_j|, equals it where no term has the other sign, scales with |q|, is
    read from the state after the row's update, and counts the delta rule's
    subtraction as a term (a write of what the state already holds changes
    nothing, yet triples that row's magnitude)."""
    rng = np.random.default_rng(5)
    dk, dv, T = 6, 5, 7
    M0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    alpha, beta = rng.uniform(0.2, 1.0, T), rng.uniform(0.0, 1.0, T)
    _, o, _, mag = oracle.raw_recurrence(alpha, beta, k, q, v, M0, mag=True)
    assert np.all(mag >= np.abs(o) * (1 - 1e-15))
    assert np.any(mag > 1.5 * np.abs(o))            # random signs do cancel
    _, o2, _, mag2 = oracle.raw_recurrence(alpha, beta, k, -3.0 * q, v, M0, mag=True)
    assert np.allclose(o2, -3.0 * o, rtol=1e-14, atol=0) and np.allclose(mag2, 3.0 * mag, rtol=1e-14)
    # one sign: no write (beta = 0), non-negative state and query
    Mp, qp = np.abs(M0), np.abs(q)
    _, o3, _, mag3 = oracle.raw_recurrence(alpha, np.zeros(T), k, qp, v, Mp, mag=True)
    assert np.allclose(mag3, o3, rtol=1e-15, atol=0)
    for i in range(dk):
        e = np.zeros((1, dk)); e[0, i] = 1.0
        # a unit write from the zero state with q = k = e_i: o = v, magnitude |v|
        # (the state before the update would give 0)
        _, o4, _, mag4 = oracle.raw_recurrence([1.0], [1.0], e, e, v[:1], np.zeros((dk, dv)), mag=True)
        assert np.array_equal(o4[0], v[0]) and np.array_equal(mag4[0], np.abs(v[0]))
        # writing back row i of the state (v = M0^T e_i, alpha = beta = 1):
        # M is unchanged, and row i's magnitude is |M0_i| + |M0_i| (the
        # subtracted readout) + |v| = 3 |M0_i|
        _, o5, _, mag5 = oracle.raw_recurrence([1.0], [1.0], e, e, M0[i][None], M0, mag=True)
        assert np.array_equal(o5[0], M0[i]) and np.allclose(mag5[0], 3 * np.abs(M0[i]), rtol=1e-15)
        # and with alpha = 1/2: the old state and the subtracted term halve
        _, _, _, mag6 = oracle.raw_recurrence([0.5], [1.0], e, e, M0[i][None], M0, mag=True)
        assert np.allclose(mag6[0], 2 * np.abs(M0[i]), rtol=1e-15)


def test_delta_write_exact_with_unit_axis_key():
    # alpha = beta = 1, k = e_i, dyadic M and v: row i of M becomes v^T exactly,
    # so M'^T k = v, and every other row is untouched
    rng = np.random.default_rng(3)
    dk, dv = 8, 6
    M0 = rng.integers(-1024, 1024, (dk, dv)) / 256.0
    for i in range(dk):
        k = np.zeros((1, dk)); k[0, i] = 1.0
        v = rng.integers(-1024, 1024, (1, dv)) / 256.0
        q = k.copy()
        M, o, _ = oracle.raw_recurrence([1.0], [1.0], k, q, v, M0)
        assert np.array_equal(M.T @ k[0], v[0])
        assert np.array_equal(o[0], v[0])
        keep = [r for r in range(dk) if r != i]
        assert np.array_equal(M[keep], M0[keep])


def test_pure_decay_when_beta_zero():
    rng = np.random.default_rng(4)
    dk, dv, T = 5, 4, 6
    M0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    alpha = np.full(T, 0.5)
    M, o, M_all = oracle.raw_recurrence(alpha, np.zeros(T), k, q, v, M0, keep_all=True)
    for t in range(T):
        assert np.array_equal(M_all[t], M0 * 0.5 ** (t + 1))
        assert np.allclose(o[t], (M0 * 0.5 ** (t + 1)).T @ q[t], rtol=1e-14, atol=1e-15)


def _brute_force(alpha, beta, k, q, v, M0):
    """Transfer matrices: M_t = Phi_{t,0} M0 + sum_j Phi_{t,j} beta_j k_j v_j^T with
    Phi_{t,j} = A_t ... A_{j+1} and A_i = alpha_i (I - beta_i k_i k_i^T)."""
    T, dk = k.shape
    A = [alpha[i] * (np.eye(dk) - beta[i] * np.outer(k[i], k[i])) for i in range(T)]
    out_M, out_o = [], []
    for t in range(T):
        Phi = np.eye(dk)
        for i in range(t, -1, -1):
            Phi = Phi @ A[i]
        M = Phi @ M0
        for j in range(t + 1):
            P = np.eye(dk)
            for i in range(t, j, -1):
                P = P @ A[i]
            M = M + beta[j] * P @ np.outer(k[j], v[j])
        out_M.append(M)
        out_o.append(M.T @ q[t])
    return np.array(out_M), np.array(out_o)


@pytest.mark.parametrize("dk,dv,T,seed", [(2, 2, 4, 0), (3, 4, 6, 1), (4, 3, 5, 2), (4, 4, 6, 3)])
def test_brute_force_tiny_heads(dk, dv, T, seed):
    rng = np.random.default_rng(10 + seed)
    M0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.05, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    M, o, M_all = oracle.raw_recurrence(alpha, beta, k, q, v, M0, keep_all=True)
    BM, Bo = _brute_force(alpha, beta, k, q, v, M0)
    assert np.max(np.abs(M_all - BM)) < 1e-12
    assert np.max(np.abs(o - Bo)) < 1e-12


# --------------------------------------------------------------------------- full path

def _np_batch(b: gi.Batch):
    return dict(conv_w=b.params.conv_w.numpy(), a_log=b.params.a_log.numpy(),
                dt_bias=b.params.dt_bias.numpy(), row_start=b.row_start.numpy(),
                qkv=gi.bf16_bits(b.qkv), a=gi.bf16_bits(b.a), b=gi.bf16_bits(b.b),
                tail=gi.bf16_bits(b.tail), state=b.state.numpy().astype(np.float64))


def _run_window(shape, d, **kw):
    return oracle.window(shape, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"],
                         d["qkv"], d["a"], d["b"], d["tail"], d["state"], **kw)


TINY = gi.Shape(hk=2, hv=4, dk=8, dv=6)


def test_window_equals_one_row_steps():
    batch = gi.make_batch(TINY, [5, 1, 3], seed=7)
    d = _np_batch(batch)
    full = _run_window(TINY, d)
    Cn = TINY.channels
    for s, ln in enumerate(batch.lengths()):
        r0 = int(d["row_start"][s])
        tail = d["tail"][s:s + 1].copy()
        state = d["state"][s:s + 1].copy()
        for t in range(ln):
            r = r0 + t
            step = oracle.window(TINY, d["conv_w"], d["a_log"], d["dt_bias"],
                                 np.array([0, 1], np.int32), d["qkv"][r:r + 1],
                                 d["a"][r:r + 1], d["b"][r:r + 1], tail, state)
            assert np.array_equal(step["o"][0], full["o"][r])
            assert np.array_equal(step["snap64"][0], full["snap64"][r])
            assert np.array_equal(step["tail_snap"][0], full["tail_snap"][r])
            tail = step["tail_snap"][0:1].reshape(1, 3, Cn)
            state = step["snap64"][0:1]


def test_tail_snapshots_are_the_last_three_raw_rows():
    batch = gi.make_batch(TINY, [6, 2], seed=8)
    d = _np_batch(batch)
    res = _run_window(TINY, d)
    for s, ln in enumerate(batch.lengths()):
        r0 = int(d["row_start"][s])
        hist = [d["tail"][s][0], d["tail"][s][1], d["tail"][s][2]]
        for t in range(ln):
            hist.append(d["qkv"][r0 + t])
            assert np.array_equal(res["tail_snap"][r0 + t], np.stack(hist[-3:]))


def _tree_batch(lengths, seed):
    return gi.make_batch(TINY, lengths, seed=seed, tree=True)


def test_tree_path_equals_chain():
    batch = _tree_batch([9, 7, 1], seed=9)
    d = _np_batch(batch)
    par = batch.parent.numpy()
    res = oracle.tree(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"], par,
                      d["qkv"], d["a"], d["b"], d["tail"], d["state"])
    rs = d["row_start"]
    for s, ln in enumerate(batch.lengths()):
        r0 = int(rs[s])
        local = par[r0:r0 + ln].tolist()
        for leaf in range(ln):
            path = gi.path_to_root(local, leaf)
            rows = [r0 + i for i in path]
            chain = oracle.window(TINY, d["conv_w"], d["a_log"], d["dt_bias"],
                                  np.array([0, len(rows)], np.int32), d["qkv"][rows],
                                  d["a"][rows], d["b"][rows], d["tail"][s:s + 1],
                                  d["state"][s:s + 1])
            assert np.array_equal(chain["o"], res["o"][rows])
            assert np.array_equal(chain["snap64"], res["snap64"][rows])
            assert np.array_equal(chain["tail_snap"], res["tail_snap"][rows])


def test_tree_of_chain_parents_equals_window():
    batch = gi.make_batch(TINY, [4, 3], seed=10)
    d = _np_batch(batch)
    w = _run_window(TINY, d)
    t = oracle.tree(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"],
                    batch.parent.numpy(), d["qkv"], d["a"], d["b"], d["tail"], d["state"])
    for key in ("o", "snap64", "tail_snap"):
        assert np.array_equal(w[key], t[key])


def _frozen_state_batch(shape, lengths, seed, tap):
    """alpha = 1 and beta = 0 freeze the state, so o_t = M0^T qhat_t depends only
    on row t's conv output; weights with a single tap make that the raw row
    x_(t-3+tap)."""
    batch = gi.make_batch(shape, lengths, seed=seed)
    d = _np_batch(batch)
    d["a_log"][:] = -np.inf
    d["b"][:] = BF16_NEG_INF
    w = np.zeros_like(d["conv_w"])
    w[:, tap] = 1.0
    d["conv_w"] = w
    return batch, d


@pytest.mark.parametrize("tap", [0, 1, 2])
def test_conv_taps_follow_the_branch(tap):
    batch = _tree_batch([10, 6], seed=11)
    _, d = _frozen_state_batch(TINY, [10, 6], 11, tap)
    par = batch.parent.numpy()
    res = oracle.tree(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"], par,
                      d["qkv"], d["a"], d["b"], d["tail"], d["state"])
    w3 = np.zeros_like(d["conv_w"]); w3[:, 3] = 1.0
    rs = d["row_start"]
    for s, ln in enumerate(batch.lengths()):
        r0 = int(rs[s])
        local = par[r0:r0 + ln].tolist()
        for i in range(ln):
            # walk 3 - tap ancestors up; past the root, read the tail backwards
            node = i
            for _ in range(3 - tap):
                node = local[node] if node >= 0 else node - 1
            # -1, -2, -3 stand for the tail's rows 2, 1, 0 above the root
            src = d["qkv"][r0 + node] if node >= 0 else d["tail"][s][node + 3]
            one = oracle.window(TINY, w3, d["a_log"], d["dt_bias"], np.array([0, 1], np.int32),
                                src[None], d["a"][r0 + i:r0 + i + 1], d["b"][r0 + i:r0 + i + 1],
                                d["tail"][s:s + 1], d["state"][s:s + 1])
            assert np.array_equal(one["o"][0], res["o"][r0 + i]), (s, i, tap)


def test_unit_write_reads_back_v_scaled():
    """alpha = beta = 1 and q's channels equal to k's: the row writes v at key
    khat, and q reads it back, so o = M'^T qhat = v / sqrt(dk) up to the eps of
    the normalisation."""
    shape = gi.Shape(hk=2, hv=4, dk=16, dv=8)
    batch = gi.make_batch(shape, [5], seed=12)
    d = _np_batch(batch)
    d["a_log"][:] = -np.inf
    d["b"][:] = BF16_POS_INF
    hkdk = shape.hk * shape.dk
    d["qkv"][:, :hkdk] = d["qkv"][:, hkdk:2 * hkdk]
    d["tail"][:, :, :hkdk] = d["tail"][:, :, hkdk:2 * hkdk]
    d["conv_w"][:hkdk] = d["conv_w"][hkdk:2 * hkdk]
    res = _run_window(shape, d)
    Cn = shape.channels
    hist = list(d["tail"][0])
    for t in range(5):
        hist.append(d["qkv"][t])
        _, post = oracle.conv_silu(d["conv_w"], hist[-4:])
        vrow = post[2 * hkdk:].reshape(shape.hv, shape.dv)
        kk = post[hkdk:2 * hkdk].reshape(shape.hk, shape.dk)
        for h in range(shape.hv):
            knorm2 = float(kk[h // 2] @ kk[h // 2])
            tol = 1e-12 + 4e-6 / knorm2 * np.abs(res["snap64"][t, h]).max() * 10
            assert np.allclose(res["o"][t, h] * math.sqrt(shape.dk), vrow[h],
                               rtol=0, atol=tol), (t, h)
    assert Cn == d["qkv"].shape[1]


def test_query_scale_with_identity_state():
    """alpha = 1, beta = 0 and M0 = I: o = qhat, whose squared norm is
    |q|^2 / (|q|^2 + eps) / dk: pins the 1/sqrt(dk) scale of q."""
    shape = gi.Shape(hk=1, hv=2, dk=8, dv=8)
    batch = gi.make_batch(shape, [3], seed=13)
    d = _np_batch(batch)
    d["a_log"][:] = -np.inf
    d["b"][:] = BF16_NEG_INF
    d["state"][:] = np.eye(8)[None, None]
    res = _run_window(shape, d)
    n2 = np.sum(res["o"] ** 2, axis=-1)
    assert np.allclose(n2, 1.0 / shape.dk, rtol=1e-4)
    assert np.array_equal(res["snap64"][:, 0], np.broadcast_to(np.eye(8), (3, 8, 8)))


def test_heads_sharing_a_key_head_agree():
    shape = gi.Shape(hk=2, hv=6, dk=8, dv=4)   # three value heads per key head
    batch = gi.make_batch(shape, [4, 2], seed=14)
    d = _np_batch(batch)
    vo = 2 * shape.hk * shape.dk
    for g in range(shape.hk):
        h0 = 3 * g
        for h in (h0 + 1, h0 + 2):
            d["qkv"][:, vo + h * 4: vo + h * 4 + 4] = d["qkv"][:, vo + h0 * 4: vo + h0 * 4 + 4]
            d["tail"][:, :, vo + h * 4: vo + h * 4 + 4] = d["tail"][:, :, vo + h0 * 4: vo + h0 * 4 + 4]
            d["conv_w"][vo + h * 4: vo + h * 4 + 4] = d["conv_w"][vo + h0 * 4: vo + h0 * 4 + 4]
            d["a"][:, h] = d["a"][:, h0]
            d["b"][:, h] = d["b"][:, h0]
            d["a_log"][h] = d["a_log"][h0]
            d["dt_bias"][h] = d["dt_bias"][h0]
            d["state"][:, h] = d["state"][:, h0]
    res = _run_window(shape, d)
    for g in range(shape.hk):
        h0 = 3 * g
        assert np.array_equal(res["o"][:, h0], res["o"][:, h0 + 1])
        assert np.array_equal(res["o"][:, h0], res["o"][:, h0 + 2])
    # and the two key heads differ
    assert not np.array_equal(res["o"][:, 0], res["o"][:, 3])


def test_output_affine_in_initial_state():
    batch = gi.make_batch(TINY, [6, 3], seed=15)
    d = _np_batch(batch)
    rng = np.random.default_rng(15)
    N0 = rng.standard_normal(d["state"].shape) * 0.05

    def run(st):
        dd = dict(d); dd["state"] = st
        return _run_window(TINY, dd)
    z = run(np.zeros_like(d["state"]))
    a = run(d["state"])
    b = run(N0)
    ab = run(d["state"] + N0)
    lhs = ab["o"] - z["o"]
    rhs = (a["o"] - z["o"]) + (b["o"] - z["o"])
    assert np.max(np.abs(lhs - rhs)) < 1e-12 * max(1.0, np.abs(lhs).max())
    lhs = ab["snap64"] - z["snap64"]
    rhs = (a["snap64"] - z["snap64"]) + (b["snap64"] - z["snap64"])
    assert np.max(np.abs(lhs - rhs)) < 1e-12


def test_pure_decay_through_the_whole_path():
    """beta = 0 and alpha = 1/2 (A_log = 0, a + dt_bias = 0): M_t = 2^-t M0, and
    with every row and tail row equal, o_t = 2^-(t-1) o_1."""
    batch = gi.make_batch(TINY, [6], seed=16)
    d = _np_batch(batch)
    d["a_log"][:] = 0.0
    d["dt_bias"][:] = 0.25
    d["a"][:] = bf16(-0.25)
    d["b"][:] = BF16_NEG_INF
    d["qkv"][:] = d["qkv"][0]
    d["tail"][:] = d["qkv"][0]
    res = _run_window(TINY, d)
    for t in range(6):
        assert np.allclose(res["snap64"][t, :, :, :], d["state"][0] * 0.5 ** (t + 1),
                           rtol=1e-15, atol=0)
        assert np.allclose(res["o"][t], res["o"][0] * 0.5 ** t, rtol=1e-14, atol=1e-18)


def _signed_inputs(shape, lengths, seed, q_sign, k_sign, v_sign):
    """Conv weights that pass the current row through (tap 3 = 1, so no conv
    output cancels) and raw rows whose q, k and v channels have the given
    signs, which SiLU keeps in qhat, khat and v; the initial state is made
    non-negative."""
    batch = gi.make_batch(shape, lengths, seed=seed)
    d = _np_batch(batch)
    w = np.zeros_like(d["conv_w"]); w[:, 3] = 1.0
    d["conv_w"] = w
    hkdk = shape.hk * shape.dk
    vals = np.abs(batch.qkv.float().numpy()) + 0.25
    vals[:, :hkdk] *= q_sign
    vals[:, hkdk:2 * hkdk] *= k_sign
    vals[:, 2 * hkdk:] *= v_sign
    d["qkv"] = bf16(vals)
    d["state"] = np.abs(d["state"])
    return d


def test_magnitudes_through_the_whole_path():
    """The magnitudes of full windows: never below the value's own size;
    equal to it where no term has the other sign (no write, a non-negative
    state read by a positive query; a first row whose negative v meets a
    positive key on a non-negative state; a first write from the zero state);
    a tree row's magnitudes are those of the chain over its path."""
    shape = gi.Shape(hk=2, hv=4, dk=8, dv=6)
    batch = gi.make_batch(shape, [5, 3], seed=20)
    d = _np_batch(batch)
    res = _run_window(shape, d, log=True, mag=True, snap_mag=True)
    assert np.all(res["o_mag"] >= np.abs(res["o"]) * (1 - 1e-14))
    assert np.all(res["log_delta_mag"] >= np.abs(res["log_delta"]) * (1 - 1e-14))
    assert np.all(res["snap_mag"] >= np.abs(res["snap64"]).astype(np.float32) * (1 - 1e-6))
    # no write, non-negative state, positive query: every magnitude is the value
    dq = _signed_inputs(shape, [4, 2], 21, 1.0, 1.0, 1.0)
    dq["b"][:] = BF16_NEG_INF
    r = _run_window(shape, dq, mag=True, snap_mag=True)
    assert np.all(r["o"] > 0) and np.allclose(r["o_mag"], r["o"], rtol=1e-14, atol=0)
    assert np.allclose(r["snap_mag"], r["snap64"], rtol=1e-6, atol=0)
    # first rows: negative v, positive key, non-negative state: |delta| = its magnitude
    dk_ = _signed_inputs(shape, [1, 1, 1], 22, 1.0, 1.0, -1.0)
    r = _run_window(shape, dk_, log=True, mag=True)
    assert np.all(r["log_delta"] < 0)
    assert np.allclose(r["log_delta_mag"], np.abs(r["log_delta"]), rtol=1e-14, atol=0)
    # from the zero state the write is beta v: magnitude beta |v| = |delta|
    dz = _signed_inputs(shape, [3, 2], 23, 1.0, -1.0, 1.0)
    dz["qkv"] = bf16(batch.qkv.float().numpy()[:5])       # mixed signs again
    dz["state"] = np.zeros_like(dz["state"])
    r = _run_window(shape, dz, log=True, mag=True)
    first = [0, 3]
    assert np.allclose(r["log_delta_mag"][first], np.abs(r["log_delta"][first]), rtol=1e-15, atol=0)
    # a tree: each row's magnitudes are those of the chain over its path
    tb = _tree_batch([6, 4], seed=24)
    td = _np_batch(tb)
    tr = oracle.tree(TINY, td["conv_w"], td["a_log"], td["dt_bias"], td["row_start"], tb.parent.numpy(),
                     td["qkv"], td["a"], td["b"], td["tail"], td["state"], mag=True, snap_mag=True)
    par = tb.parent.numpy()
    rs = td["row_start"]
    for st in range(2):
        local = par[rs[st]:rs[st + 1]].tolist()
        for leaf in range(len(local)):
            rows = [int(rs[st]) + i for i in gi.path_to_root(local, leaf)]
            ch = oracle.window(TINY, td["conv_w"], td["a_log"], td["dt_bias"], np.array([0, len(rows)], np.int32),
                               td["qkv"][rows], td["a"][rows], td["b"][rows], td["tail"][st:st + 1],
                               td["state"][st:st + 1], mag=True, snap_mag=True)
            assert np.array_equal(ch["o_mag"], tr["o_mag"][rows])
            assert np.array_equal(ch["snap_mag"], tr["snap_mag"][rows])


def test_conv_cancellation_counts_its_terms():
    """v channels with weights (1, 0, 0, -1) on equal oldest and current
    rows: the conv output cancels to exactly 0, so v = 0 and, from the zero
    state, the write is 0; its magnitude is beta times sigmoid(0) (SiLU's gate)
    times the conv's terms |x| + |x|, i.e. |x| / 2 with b = 0 (beta = 1/2)."""
    shape = gi.Shape(hk=1, hv=2, dk=4, dv=3)
    batch = gi.make_batch(shape, [1], seed=25, zero_state=True)
    d = _np_batch(batch)
    hkdk = shape.hk * shape.dk
    w = np.zeros_like(d["conv_w"]); w[:, 3] = 1.0
    w[2 * hkdk:, 0] = 1.0
    w[2 * hkdk:, 3] = -1.0
    d["conv_w"] = w
    x = d["qkv"][0]
    d["tail"][0, 0, 2 * hkdk:] = x[2 * hkdk:]
    d["b"][:] = bf16(0.0)
    r = _run_window(shape, d, log=True, mag=True)
    xv = (x[2 * hkdk:].astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(shape.hv, shape.dv)
    assert np.all(r["log_delta"] == 0) and np.all(r["o"] == 0)
    assert np.allclose(r["log_delta_mag"][0], 0.5 * np.abs(xv), rtol=1e-15, atol=0)
    assert np.all(r["o_mag"] > 0)


def test_prefill_matches_window_and_updates_in_place():
    batch = gi.make_batch(TINY, [7, 3, 1], seed=17)
    d = _np_batch(batch)
    w = _run_window(TINY, d, mag=True)
    o, st, tl, om, fm = oracle.prefill(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"],
                                       d["qkv"], d["a"], d["b"], d["tail"], d["state"], mag=True)
    assert np.array_equal(o, w["o"])
    assert np.array_equal(om, w["o_mag"])
    wm = _run_window(TINY, d, snap_mag=True)
    for s_ in range(3):
        assert np.array_equal(fm[s_].astype(np.float32), wm["snap_mag"][int(d["row_start"][s_ + 1]) - 1])
    rs = d["row_start"]
    for s in range(3):
        last = int(rs[s + 1]) - 1
        assert np.array_equal(st[s], w["snap64"][last])
        assert np.array_equal(tl[s], w["tail_snap"][last])


def test_prefill_short_prompts_mix_old_tail():
    batch = gi.make_batch(TINY, [1, 2, 0], seed=18)
    d = _np_batch(batch)
    o, st, tl = oracle.prefill(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"],
                               d["qkv"], d["a"], d["b"], d["tail"], d["state"])
    assert np.array_equal(tl[0], np.stack([d["tail"][0][1], d["tail"][0][2], d["qkv"][0]]))
    assert np.array_equal(tl[1], np.stack([d["tail"][1][2], d["qkv"][1], d["qkv"][2]]))
    assert np.array_equal(tl[2], d["tail"][2])       # an empty prompt changes nothing
    assert np.array_equal(st[2], d["state"][2])


def test_commit_takes_the_accepted_rows():
    batch = _tree_batch([5, 4, 3], seed=19)
    d = _np_batch(batch)
    res = oracle.tree(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"],
                      batch.parent.numpy(), d["qkv"], d["a"], d["b"], d["tail"], d["state"])
    acc = batch.accept.numpy().copy()
    acc[2] = -1
    tl, st = oracle.commit(TINY, acc, res["tail_snap"], res["snap64"], d["tail"], d["state"])
    for s in range(2):
        assert np.array_equal(st[s], res["snap64"][acc[s]])
        assert np.array_equal(tl[s], res["tail_snap"][acc[s]])
    assert np.array_equal(st[2], d["state"][2]) and np.array_equal(tl[2], d["tail"][2])


def test_malformed_layouts_are_refused():
    batch = gi.make_batch(TINY, [3, 2], seed=20)
    d = _np_batch(batch)
    bad = np.array([0, 3, 1], np.int32)
    with pytest.raises(ValueError):
        oracle.window(TINY, d["conv_w"], d["a_log"], d["dt_bias"], bad, d["qkv"], d["a"],
                      d["b"], d["tail"], d["state"])
    par = batch.parent.numpy().copy()
    par[1] = 1       # a node may not be its own parent
    with pytest.raises(ValueError):
        oracle.tree(TINY, d["conv_w"], d["a_log"], d["dt_bias"], d["row_start"], par,
                    d["qkv"], d["a"], d["b"], d["tail"], d["state"])
