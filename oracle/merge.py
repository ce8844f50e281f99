"""Oracle: merging the adapter into the base and quantizing the result again.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[QLoRA-074 §五, §六] warns that merging an adapter into the weights and
quantizing again may change the outputs; the weimeta glossary's FAQ says the
merge has to happen in 16-bit precision, not on the 4-bit weights, before the
merged model is quantized.  The merged weight, stored as Wq [o][d] (Ŵ = Wqᵀ):

    W'[n][k] = fl32( ŵ[n][k] + s · Δ[k][n] ),   Δ = A·B,

Reading: Δ[k][n] = Σ_j A[k][j]·B[j][n] is summed in fp64 in increasing j
(every bf16 × bf16 product is exact in fp64, so the sum has one rounding per
term and a fixed order); s·Δ and the addition of the fp32 dequantized weight
ŵ are one fp64 rounding each; the result is rounded once to fp32.  The
merged fp32 tensor is then quantized with the same blockwise NF4 + double
quantization as any fp32 weight.
"""

from __future__ import annotations

import numpy as np

from . import nf4


def merge(w_hat: np.ndarray, A: np.ndarray, B: np.ndarray, s: float) -> np.ndarray:
    """fp32 merged weight [o][d] from the fp32 dequantized weight [o][d]."""
    w_hat = np.asarray(w_hat, np.float32)
    A = np.asarray(A, np.float64)            # [d][r]
    B = np.asarray(B, np.float64)            # [r][o]
    o, d = w_hat.shape
    delta = np.zeros((d, o))
    for j in range(A.shape[1]):              # fixed order, one rounding per term
        delta += np.outer(A[:, j], B[j, :])
    merged = w_hat.astype(np.float64) + np.float64(s) * delta.T
    return merged.astype(np.float32)


def merge_and_requantize(codes, scale8, scale2, shape, A, B, s):
    """(merged fp32 weight, its codes, scale8, scale2)."""
    o, d = shape
    w_hat = nf4.dequant_f32(codes, scale8, scale2, o * d).reshape(o, d)
    merged = merge(w_hat, A, B, s)
    return (merged,) + tuple(nf4.quantize_chunked(merged.ravel()))
