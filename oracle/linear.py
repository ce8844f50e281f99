"""Oracle: forward and backward of the QLoRA linear layer in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Given the dequantized weight, the layer is plain linear algebra, so the
oracle is that definition written out with fp64 matrix products.  The bf16
inputs (X, A, B, dY) and the bf16 weight operand are taken at their exact
values (every bf16 number is exact in fp64).

Shapes (reading of [QLoRA-074 §一], with the weight stored as nn.Linear does):
  X [M][d], Wq [o][d] (so Ŵ = Wqᵀ is d×o), A [d][r], B [r][o], Y [M][o].
"""

from __future__ import annotations

import numpy as np


def forward(X: np.ndarray, Wq: np.ndarray, A: np.ndarray, B: np.ndarray, s: float):
    """Y = X·Ŵ + s·X·A·B  [QLoRA-074 §一], with T = X·A returned too.

    Ŵ = Wqᵀ.  Everything fp64.
    """
    X = np.asarray(X, np.float64)
    T = X @ np.asarray(A, np.float64)
    Y = X @ np.asarray(Wq, np.float64).T + s * (T @ np.asarray(B, np.float64))
    return Y, T


def backward(dY: np.ndarray, X: np.ndarray, Wq: np.ndarray, A: np.ndarray,
             B: np.ndarray, s: float):
    """Input and adapter gradients of L = Σ dY ⊙ Y; the 4-bit base gets none.

    [QLoRA-074, note on what the backward pass still needs]: passing the
    error to earlier layers multiplies by the transpose of the dequantized
    matrix, while the frozen base stores no gradient of its own.  With
    Y = X·Ŵ + s·(X·A)·B:
      U  = dY·Bᵀ
      dX = dY·Ŵᵀ + s·U·Aᵀ
      dB = s·(X·A)ᵀ·dY
      dA = s·Xᵀ·U
    Returns (dX, dA, dB).
    """
    dY = np.asarray(dY, np.float64)
    X = np.asarray(X, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    W = np.asarray(Wq, np.float64)          # Ŵᵀ = Wq, so dY·Ŵᵀ = dY·Wq
    U = dY @ B.T
    dX = dY @ W + s * (U @ A.T)
    T = X @ A
    dB = s * (T.T @ dY)
    dA = s * (X.T @ U)
    return dX, dA, dB


def forward_rows(X, Wq, A, B, s, rows):
    """Y restricted to the given rows of X (for sampled checks at full size)."""
    return forward(np.asarray(X)[rows], Wq, A, B, s)[0]


def dx_rows(dY, Wq, A, B, s, rows):
    """dX restricted to the given rows of dY."""
    dY = np.asarray(dY, np.float64)[rows]
    U = dY @ np.asarray(B, np.float64).T
    return dY @ np.asarray(Wq, np.float64) + s * (U @ np.asarray(A, np.float64).T)


def grad_cols(dY, X, A, B, s, a_rows, b_cols):
    """dA[a_rows, :] and dB[:, b_cols] (reductions over all M tokens)."""
    dY = np.asarray(dY, np.float64)
    X = np.asarray(X, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    U = dY @ B.T
    T = X @ A
    dA = s * (X[:, a_rows].T @ U)
    dB = s * (T.T @ dY[:, b_cols])
    return dA, dB
