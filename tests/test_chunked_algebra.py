"""The chunkwise (WY) form of the gated delta rule against the recurrence.

An independent fp64 NumPy formulation of the chunked algebra, written from the
derivation below, must reach the oracle's row-by-row recurrence to rounding.
This pins the oracle's recurrence from a second, differently structured
computation, and checks the algebra the MFMA prompt kernels use.

Derivation (stored form M = S^T, rows of K, Q, V are k_t^T, q_t^T, v_t^T):
the step M_t = alpha_t M_{t-1} + k_t d_t^T with
d_t = beta_t (v_t - alpha_t M_{t-1}^T k_t).  Inside a chunk that starts from
M0, with g_t = log alpha_t and gamma_t = g_1 + ... + g_t,
    M_t = e^{gamma_t} M0 + sum_{j<=t} e^{gamma_t - gamma_j} k_j d_j^T,
so the d_t satisfy the unit lower-triangular system
    (I + A) D = diag(beta) V - diag(beta e^gamma) K M0,
    A_tj = beta_t e^{gamma_t - gamma_j} k_t^T k_j   (j < t),
whence D = U~ - W M0 with T = (I + A)^{-1}, U~ = T diag(beta) V and
W = T diag(beta e^gamma) K.  Outputs and the state leaving the chunk are
    O = diag(e^gamma) Q M0 + P D,  P_tj = e^{gamma_t - gamma_j} q_t^T k_j (j <= t),
    M_L = e^{gamma_L} M0 + (diag(e^{gamma_L - gamma}) K)^T D.
Since D = U~ - W M0, the output also reads O = Q' M0 + P U~ with
Q' = diag(e^gamma) Q - P W: every product without M0 can be formed per chunk
in parallel, and the sequential part needs only [W; Q'] M0 and the update.
"""
import numpy as np
import pytest

import oracle


def chunked(alpha, beta, K, Q, V, M0, chunk, fold_pw=False):
    T = K.shape[0]
    M = M0.copy()
    O = np.zeros((T, V.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        L = c1 - c0
        k, q, v, b = K[c0:c1], Q[c0:c1], V[c0:c1], beta[c0:c1]
        gam = np.cumsum(np.log(alpha[c0:c1]))
        diff = gam[:, None] - gam[None, :]
        lower = np.tril(np.ones((L, L), bool), -1)
        decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        A = b[:, None] * decay * (k @ k.T)
        Tm = np.linalg.solve(np.eye(L) + A, np.eye(L))
        Ut = Tm @ (b[:, None] * v)
        W = Tm @ ((b * np.exp(gam))[:, None] * k)
        D = Ut - W @ M
        incl = np.tril(np.ones((L, L), bool))
        P = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0) * (q @ k.T)
        if fold_pw:
            Qp = np.exp(gam)[:, None] * q - P @ W
            O[c0:c1] = Qp @ M + P @ Ut
        else:
            O[c0:c1] = (np.exp(gam)[:, None] * q) @ M + P @ D
        M = np.exp(gam[-1]) * M + (np.exp(gam[-1] - gam)[:, None] * k).T @ D
    return M, O


@pytest.mark.parametrize("fold_pw", [False, True])
@pytest.mark.parametrize("T,chunk,dk,dv,lo,hi,seed", [
    (150, 64, 8, 6, 0.05, 1.0, 0),      # partial last chunk (22 rows)
    (64, 64, 8, 8, 0.05, 1.0, 1),       # exactly one chunk
    (37, 16, 4, 5, 0.9, 1.0, 2),        # long memory
    (200, 64, 16, 8, 0.02, 0.2, 3),     # strong decay: cumulative gates reach e^-250
    (5, 64, 4, 4, 0.3, 0.9, 4),         # shorter than a chunk
])
def test_chunked_form_equals_recurrence(T, chunk, dk, dv, lo, hi, seed, fold_pw):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, dk)); K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((T, dk)) / np.sqrt(dk)
    V = rng.standard_normal((T, dv))
    alpha = rng.uniform(lo, hi, T)
    beta = rng.uniform(0.0, 1.0, T)
    M0 = rng.standard_normal((dk, dv)) * 0.05
    M_ref, O_ref, _ = oracle.raw_recurrence(alpha, beta, K, Q, V, M0)
    M, O = chunked(alpha, beta, K, Q, V, M0, chunk, fold_pw)
    scale = max(1.0, np.abs(O_ref).max())
    assert np.max(np.abs(O - O_ref)) < 1e-10 * scale
    assert np.max(np.abs(M - M_ref)) < 1e-10 * max(1.0, np.abs(M_ref).max())


def test_chunk_size_does_not_change_the_result():
    rng = np.random.default_rng(9)
    T, dk, dv = 90, 8, 8
    K = rng.standard_normal((T, dk)); K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    M0 = rng.standard_normal((dk, dv))
    M1, O1 = chunked(alpha, beta, K, Q, V, M0, 1)
    M64, O64 = chunked(alpha, beta, K, Q, V, M0, 64)
    assert np.max(np.abs(O1 - O64)) < 1e-10 * np.abs(O1).max()
    assert np.max(np.abs(M1 - M64)) < 1e-10 * np.abs(M1).max()


def blocked_unit_lower_inverse(A, nb=16):
    """(I + A)^-1 for strictly lower-triangular A by nb x nb blocks: the
    diagonal blocks by forward substitution, then
    T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, one diagonal distance at a time."""
    n = A.shape[0]
    m = n // nb
    blk = lambda X, i, j: X[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb]
    T = np.zeros_like(A)
    for i in range(m):
        Aii = blk(A, i, i)
        Tii = np.zeros((nb, nb))
        for t in range(nb):
            Tii[t] = -Aii[t, :t] @ Tii[:t]
            Tii[t, t] = 1.0
        T[i * nb:(i + 1) * nb, i * nb:(i + 1) * nb] = Tii
    for d in range(1, m):
        for i in range(d, m):
            j = i - d
            S = sum(blk(A, i, k) @ blk(T, k, j) for k in range(j, i))
            T[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb] = -blk(T, i, i) @ S
    return T


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_blocked_triangular_inverse(seed):
    rng = np.random.default_rng(seed)
    n = 64
    A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
    T = blocked_unit_lower_inverse(A)
    ref = np.linalg.inv(np.eye(n) + A)
    assert np.max(np.abs(T - ref)) < 1e-10 * max(1.0, np.abs(ref).max())
    assert np.array_equal(np.triu(T, 1), np.zeros((n, n)))
