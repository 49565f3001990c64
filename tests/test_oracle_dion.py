"""Pins of the oracle's Dion step ([MS] "What Breaks at Scale", subsection
"The Matrix Does Not Fit"), each independent of the formula path:
  * exact rank-r input with Q = its right singular vectors: closed form
    P = U, R = V S, M' = mu B, Q' = V, X' = X - lr U V^T;
  * rank(B) <= r with a generic Q: P spans range(B), so the whole of B
    leaves M (M' = mu B) and the update has rank <= r;
  * warm-started power iteration: repeated steps with G = 0 and mu = 1
    (M stays B) make P span the top-r left singular subspace of B, and Q'
    the top-r right one (a transposed operand or a dropped orthogonalisation
    fails this);
  * orthonormal P (P^T P = I) and unit columns of Q' on random inputs;
    ColNorm leaves a zero column zero;
  * the basis is QR's with a positive diagonal: P^T (B Q) is upper triangular
    with a positive diagonal.
"""
import numpy as np

from oracle import muon_oracle as O


def rng(seed):
    return np.random.default_rng(seed)


def orth(g, n, k):
    return np.linalg.qr(g.standard_normal((n, k)))[0]


def test_exact_rank_r_closed_form():
    g = rng(1)
    m, n, r = 40, 30, 5
    U, V = orth(g, m, r), orth(g, n, r)
    s = np.array([5.0, 3.0, 2.0, 1.0, 0.5])
    B = U @ np.diag(s) @ V.T
    G = 0.3 * B
    M = B - G
    X = g.standard_normal((m, n))
    mu, lr = 0.95, 0.02
    Xn, Mn, Qn, P, R = O.dion_step(X, G, M, V, mu=mu, lr=lr)
    assert np.allclose(P, U, atol=1e-12)
    assert np.allclose(R, V * s[None, :], atol=1e-12)
    assert np.allclose(Mn, mu * B, atol=1e-12)
    assert np.allclose(Qn, V, atol=1e-12)
    assert np.allclose(Xn, X - lr * U @ V.T, atol=1e-12)


def test_low_rank_input_leaves_m_entirely():
    g = rng(2)
    m, n, k, r = 50, 36, 4, 8
    B = g.standard_normal((m, k)) @ g.standard_normal((k, n))
    G = g.standard_normal((m, n)) * 0.0 + 0.5 * B
    M = B - G
    Q = g.standard_normal((n, r))
    Xn, Mn, Qn, P, R = O.dion_step(np.zeros((m, n)), G, M, Q, mu=0.9, lr=0.1)
    assert np.allclose(Mn, 0.9 * B, atol=1e-10)
    assert np.linalg.matrix_rank(Xn, tol=1e-9) <= r


def test_power_iteration_finds_top_subspace():
    g = rng(3)
    m, n, r = 60, 45, 3
    Uf, Vf = orth(g, m, n), orth(g, n, n)
    s = np.concatenate([[10.0, 8.0, 6.0], np.linspace(2.0, 0.1, n - 3)])
    B = Uf @ np.diag(s) @ Vf.T
    Q = g.standard_normal((n, r))
    M = B.copy()
    for _ in range(40):
        _, M, Q, P, _ = O.dion_step(np.zeros((m, n)), np.zeros((m, n)), M, Q, mu=1.0, lr=0.0)
    assert np.allclose(M, B, atol=1e-12)
    top_u, top_v = Uf[:, :r], Vf[:, :r]
    assert np.allclose(P @ P.T, top_u @ top_u.T, atol=1e-8)
    Qo = O.orthonormal_basis(Q)
    assert np.allclose(Qo @ Qo.T, top_v @ top_v.T, atol=1e-8)


def test_orthonormal_and_unit_columns():
    g = rng(4)
    m, n, r = 33, 70, 6
    X, G, M, Q = (g.standard_normal(s) for s in ((m, n), (m, n), (m, n), (n, r)))
    _, _, Qn, P, R = O.dion_step(X, G, M, Q, mu=0.95, lr=0.02)
    assert np.allclose(P.T @ P, np.eye(r), atol=1e-12)
    assert np.allclose(np.linalg.norm(Qn, axis=0), 1.0, atol=1e-12)
    T = P.T @ ((M + G) @ Q)
    assert np.allclose(np.tril(T, -1), 0.0, atol=1e-10)
    assert np.all(np.diag(T) > 0)


def test_column_normalize_zero_column():
    R = np.array([[3.0, 0.0], [4.0, 0.0]])
    assert np.array_equal(O.column_normalize(R), np.array([[0.6, 0.0], [0.8, 0.0]]))
