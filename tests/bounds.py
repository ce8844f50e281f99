"""Rounding bounds shared by the CPU pins of the merge and AdamW oracles and by
the GPU tests that check the kernels against the plain fp64 definitions.

Both oracles follow a fixed fp32 order that the pages leave open; these
bounds tie any such order to the exact (fp64) definition, so a kernel can be
held to the definition directly, independent of the order it uses."""

from __future__ import annotations

import numpy as np

U = 2.0 ** -24          # unit roundoff of fp32


def merge_bound(w_hat, A, B, s, r):
    """(bound, exact) for W' = fl32(ŵ + fl32(s·Σ_j A[k][j]·B[j][n])) computed
    with one fp32 rounding per rank term and two more: |fl(W') − exact| <=
    |s|·(r+1)·u·Σ_j|A||B| + u·|exact| (plus u² terms, the 1.0001 factor).
    w_hat [o][d] fp32 values; A [d][r], B [r][o] as fp64 values."""
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    absum = np.abs(A) @ np.abs(B)                     # [d][o]
    exact = np.asarray(w_hat, np.float64) + s * (A @ B).T
    return abs(s) * (r + 1) * U * absum.T * 1.0001 + U * np.abs(exact) * 1.0001, exact


def adamw_magnitudes(Mabs, Vabs, g, b1=0.9, b2=0.999):
    """One step of the moment recurrences on magnitudes: Mabs' = b1·Mabs +
    (1−b1)·|g|, Vabs' = b2·Vabs + (1−b2)·g², the sums the moments would be
    without cancellation (start from |m0| and v0)."""
    g = np.asarray(g, np.float64)
    b1, b2 = float(np.float32(b1)), float(np.float32(b2))
    return b1 * Mabs + (1 - b1) * np.abs(g), b2 * Vabs + (1 - b2) * g ** 2


def adamw_state_bounds(t, Mabs, Vabs):
    """Bounds on |m − m64| and |v − v64| after t steps of an fp32 AdamW whose
    operations each round once.  Per step three roundings (the two products
    and the sum) add at most 2u·Mabs_t (u·Mabs_t for the products, u·|m_t|
    for the sum) and the carried error shrinks by b1, so after t steps the
    error is at most 2t·u·Mabs_t (the same for v; 1 − b1 and 1 − b2 of the
    fp32 b1, b2 and the bf16 g² are exact in fp32).  3t·u leaves room for
    the fp64 reference's own rounding."""
    return 3 * t * U * Mabs + 1e-30, 3 * t * U * Vabs + 1e-30


def adamw_param_bound(t):
    """|p − p64| after t steps for |p| < 0.1: one or two fp32 roundings of p per step."""
    return 3 * t * float(np.spacing(np.float32(0.1)))
