"""Pins of the oracle's linear forward/backward.

Checked against: naive index-by-index loops in pure Python (the definition
written out with explicit indices, so a transposed operand or a dropped term
fails), the special cases s = 0, A = 0 and B = 0, the merged-weight form
X·(Ŵ + s·A·B) (associativity), central finite differences of L = Σ dY ⊙ Y
(linear in each of X, A, B, so differences are exact up to rounding) and the
adjoint identity ⟨dY, X·Ŵ⟩ = ⟨dY·Ŵᵀ, X⟩.
"""

import numpy as np
import pytest

from oracle import linear


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.fixture
def small():
    M, d, o, r = 3, 5, 4, 2
    return (_rand((M, d), 1), _rand((o, d), 2), _rand((d, r), 3), _rand((r, o), 4),
            _rand((M, o), 5), 1.75)


def naive_forward(X, Wq, A, B, s):
    M, d = len(X), len(X[0])
    o, r = len(Wq), len(A[0])
    Y = [[0.0] * o for _ in range(M)]
    for m in range(M):
        for n in range(o):
            base = sum(X[m][k] * Wq[n][k] for k in range(d))
            lora = sum(sum(X[m][k] * A[k][j] for k in range(d)) * B[j][n] for j in range(r))
            Y[m][n] = base + s * lora
    return np.array(Y)


def test_forward_matches_naive_loops(small):
    X, W, A, B, _, s = small
    Y, T = linear.forward(X, W, A, B, s)
    assert np.allclose(Y, naive_forward(X.tolist(), W.tolist(), A.tolist(), B.tolist(), s),
                       rtol=1e-13, atol=1e-13)
    Tref = [[sum(X[m, k] * A[k, j] for k in range(X.shape[1])) for j in range(A.shape[1])]
            for m in range(X.shape[0])]
    assert np.allclose(T, np.array(Tref), rtol=1e-13, atol=1e-13)


def test_forward_tiny_128_shapes_naive():
    """The smallest workload's shapes (M=8, d=o=128, r=8) against loops on a slice."""
    X, W, A, B = _rand((8, 128), 6), _rand((128, 128), 7), _rand((128, 8), 8), _rand((8, 128), 9)
    Y, _ = linear.forward(X, W, A, B, 2.0)
    cols = [0, 17, 127]
    ref = naive_forward(X.tolist(), W[cols].tolist(), A.tolist(), B[:, cols].tolist(), 2.0)
    assert np.allclose(Y[:, cols], ref, rtol=1e-12, atol=1e-12)


def test_s_zero_is_plain_matmul(small):
    X, W, A, B, _, _ = small
    Y, _ = linear.forward(X, W, A, B, 0.0)
    ref = np.array([[sum(X[m, k] * W[n, k] for k in range(X.shape[1])) for n in range(W.shape[0])]
                    for m in range(X.shape[0])])
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)


def test_merged_weight_form(small):
    X, W, A, B, _, s = small
    Y, _ = linear.forward(X, W, A, B, s)
    merged = X @ (W.T + s * (A @ B))
    assert np.allclose(Y, merged, rtol=1e-12, atol=1e-12)


def _loss(X, W, A, B, dY, s):
    return float(np.sum(dY * linear.forward(X, W, A, B, s)[0]))


@pytest.mark.parametrize("which", ["X", "A", "B"])
def test_finite_differences(small, which):
    X, W, A, B, dY, s = small
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    target = {"X": (X, dX), "A": (A, dA), "B": (B, dB)}[which]
    P, G = target
    h = 1e-3
    num = np.zeros_like(P)
    for idx in np.ndindex(P.shape):
        old = P[idx]
        P[idx] = old + h
        lp = _loss(X, W, A, B, dY, s)
        P[idx] = old - h
        lm = _loss(X, W, A, B, dY, s)
        P[idx] = old
        num[idx] = (lp - lm) / (2 * h)
    assert np.allclose(G, num, rtol=1e-9, atol=1e-9)


def test_no_weight_gradient_and_adjoint(small):
    X, W, A, B, dY, s = small
    out = linear.backward(dY, X, W, A, B, s)
    assert len(out) == 3                       # dX, dA, dB; the 4-bit base gets none
    dX0, _, _ = linear.backward(dY, X, W, A, B, 0.0)
    assert np.isclose(np.sum(dY * (X @ W.T)), np.sum(dX0 * X), rtol=1e-12)


def test_zero_adapters(small):
    X, W, A, B, dY, s = small
    _, dA, _ = linear.backward(dY, X, W, A, np.zeros_like(B), s)
    assert np.all(dA == 0)
    _, _, dB = linear.backward(dY, X, W, np.zeros_like(A), B, s)
    assert np.all(dB == 0)
    Y, _ = linear.forward(X, W, A, np.zeros_like(B), s)
    assert np.allclose(Y, X @ W.T, rtol=1e-14, atol=1e-14)


def test_sampled_helpers_agree(small):
    X, W, A, B, dY, s = small
    Y, _ = linear.forward(X, W, A, B, s)
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    rows = [0, 2]
    assert np.allclose(linear.forward_rows(X, W, A, B, s, rows), Y[rows])
    assert np.allclose(linear.dx_rows(dY, W, A, B, s, rows), dX[rows])
    ga, gb = linear.grad_cols(dY, X, A, B, s, [1, 4], [0, 3])
    assert np.allclose(ga, dA[[1, 4]]) and np.allclose(gb, dB[:, [0, 3]])
