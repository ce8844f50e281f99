"""Oracle: one frozen 4-bit base shared by several LoRA adapters, chosen per token.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[LoRA-PyTorch §四.5] keeps several independent adapter pairs (A_i, B_i)
beside one base model and switches between them per request; the weimeta
glossary's FAQ describes serving many customers from one 4-bit base with a
different adapter each, never merged.  For a batch of tokens that means
every row m of X carries an adapter index a(m):

    Y[m] = X[m]·Ŵ + s_a(m) · (X[m]·A_a(m)) · B_a(m)

Reading: a(m) < 0 selects no adapter (the base alone).  Shapes: X [M][d],
Wq [o][d] (Ŵ = Wqᵀ), A [n][d][r], B [n][r][o], s [n], idx [M].  fp64.
"""

from __future__ import annotations

import numpy as np


def forward(X, Wq, A, B, s, idx):
    """(Y, T): Y [M][o] and T[m] = X[m]·A_a(m) (zero for rows with no adapter)."""
    X = np.asarray(X, np.float64)
    Wq = np.asarray(Wq, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    M = X.shape[0]
    r = A.shape[2]
    Y = X @ Wq.T
    T = np.zeros((M, r))
    for m in range(M):
        a = int(idx[m])
        if a < 0:
            continue
        T[m] = X[m] @ A[a]
        Y[m] += float(s[a]) * (T[m] @ B[a])
    return Y, T
