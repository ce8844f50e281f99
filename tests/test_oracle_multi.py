"""Pins of the multi-adapter oracle (one base, an adapter per token).

The per-row formula is checked against things it must agree with that are
computed another way: the single-adapter layer when every row shares one
adapter, the plain base product for rows with no adapter, each row's merged
weight Ŵ + s_a·A_a·B_a, and row permutations.
"""

import numpy as np

from oracle import linear, multi


def _case(M=7, d=48, o=40, r=6, n=3, seed=5):
    g = np.random.default_rng(seed)
    X = g.standard_normal((M, d))
    Wq = g.standard_normal((o, d)) * 0.1
    A = g.standard_normal((n, d, r)) * 0.1
    B = g.standard_normal((n, r, o)) * 0.1
    s = np.array([2.0, 0.5, -1.25])[:n]
    idx = g.integers(-1, n, size=M)
    idx[0], idx[1] = -1, n - 1
    return X, Wq, A, B, s, idx


def test_shared_adapter_equals_single_adapter_layer():
    X, Wq, A, B, s, _ = _case()
    for a in range(A.shape[0]):
        Y, T = multi.forward(X, Wq, A, B, s, np.full(X.shape[0], a))
        Yr, Tr = linear.forward(X, Wq, A[a], B[a], s[a])
        np.testing.assert_allclose(Y, Yr, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(T, Tr, rtol=1e-13, atol=1e-13)


def test_rows_without_adapter_are_the_base_product():
    X, Wq, A, B, s, idx = _case()
    Y, T = multi.forward(X, Wq, A, B, s, idx)
    for m in np.flatnonzero(idx < 0):
        ref = [sum(X[m, k] * Wq[n, k] for k in range(X.shape[1])) for n in range(Wq.shape[0])]
        np.testing.assert_allclose(Y[m], ref, rtol=1e-12, atol=1e-12)
        assert not T[m].any()


def test_each_row_uses_its_merged_weight():
    """Associativity: X[m]·(Ŵ + s_a·A_a·B_a) row by row."""
    X, Wq, A, B, s, idx = _case(M=9, n=3, seed=8)
    Y, _ = multi.forward(X, Wq, A, B, s, idx)
    for m, a in enumerate(idx):
        Wm = Wq.T + (s[a] * (A[a] @ B[a]) if a >= 0 else 0.0)
        np.testing.assert_allclose(Y[m], X[m] @ Wm, rtol=1e-12, atol=1e-12)


def test_row_permutation_equivariance():
    X, Wq, A, B, s, idx = _case(M=11, seed=9)
    p = np.random.default_rng(1).permutation(X.shape[0])
    Y, T = multi.forward(X, Wq, A, B, s, idx)
    Yp, Tp = multi.forward(X[p], Wq, A, B, s, idx[p])
    np.testing.assert_allclose(Yp, Y[p], rtol=0, atol=0)
    np.testing.assert_allclose(Tp, T[p], rtol=0, atol=0)


def test_a_wrong_index_is_caught():
    """A plausible slip (taking B from the neighbouring adapter) changes Y."""
    X, Wq, A, B, s, idx = _case(M=5, n=3, seed=3)
    idx[:] = 1
    Y, _ = multi.forward(X, Wq, A, B, s, idx)
    Bshift = B[[1, 2, 0]]
    Yw, _ = multi.forward(X, Wq, A, Bshift, s, idx)
    assert np.max(np.abs(Y - Yw)) > 1e-3
