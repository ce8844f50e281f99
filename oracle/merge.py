"""Oracle: merging the adapter into the base and quantizing the result again.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[QLoRA-074 §五, §六] warns that merging an adapter into the weights and
quantizing again may change the outputs; the weimeta glossary's FAQ says the
merge has to happen in 16-bit precision, not on the 4-bit weights, before the
merged model is quantized.  The merged weight, stored as Wq [o][d] (Ŵ = Wqᵀ):

    W'[n][k] = fl32( ŵ[n][k] + fl32(s · Δ[k][n]) ),   Δ = A·B,

Reading (the pages fix only "16-bit or better, not on the 4-bit codes"):
Δ[k][n] = Σ_j A[k][j]·B[j][n] is accumulated in fp32 in increasing j, one
rounding per term (every bf16 × bf16 product is exact in fp32, so a fused
multiply-add and a product-then-add give the same bits); s·Δ is rounded to
fp32, then added to the fp32 dequantized weight ŵ with one more rounding.
The merged fp32 tensor is then quantized with the same blockwise NF4 +
double quantization as any fp32 weight.
"""

from __future__ import annotations

import numpy as np

from . import nf4


def merge(w_hat: np.ndarray, A: np.ndarray, B: np.ndarray, s: float) -> np.ndarray:
    """fp32 merged weight [o][d] from the fp32 dequantized weight [o][d]."""
    w_hat = np.asarray(w_hat, np.float32)
    A = np.asarray(A, np.float32)            # [d][r], bf16 values (exact in fp32)
    B = np.asarray(B, np.float32)            # [r][o]
    o, d = w_hat.shape
    delta = np.zeros((o, d), np.float32)
    for j in range(A.shape[1]):              # increasing j, one fp32 rounding per term
        delta = delta + np.outer(B[j, :], A[:, j])    # products exact in fp32
    return w_hat + np.float32(s) * delta


def merge_and_requantize(codes, scale8, scale2, shape, A, B, s):
    """(merged fp32 weight, its codes, scale8, scale2)."""
    o, d = shape
    w_hat = nf4.dequant_f32(codes, scale8, scale2, o * d).reshape(o, d)
    merged = merge(w_hat, A, B, s)
    return (merged,) + tuple(nf4.quantize_chunked(merged.ravel()))
