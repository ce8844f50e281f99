"""Pins of the merge-and-requantize oracle.

The merged weight is pinned against exact rational arithmetic on small
inputs, against a plain fp64 matrix product (to within one fp32 ulp, with
almost every element identical), and against the cases where the merge must
leave the base untouched (s = 0, zero adapter).
"""

from fractions import Fraction

import numpy as np

import synth
from oracle import merge, nf4


def _bf16(x):
    """Round fp64 values to bf16 (RNE), returned as fp64."""
    return nf4.bf16_bits_to_f64(nf4.bf16_rne_bits(np.asarray(x, np.float32)))


def _case(o=24, d=64, r=8, seed=3):
    g = np.random.default_rng(seed)
    W = (g.standard_normal((o, d)) * 0.02).astype(np.float32)
    c, s8, s2 = nf4.quantize(W.ravel())
    w_hat = nf4.dequant_f32(c, s8, s2, W.size).reshape(o, d)
    A = _bf16(g.standard_normal((d, r)) * 0.02)
    B = _bf16(g.standard_normal((r, o)) * 0.02)
    return w_hat, A, B


def test_exact_rational_on_small_inputs():
    w_hat, A, B = _case(o=8, d=64, r=8)
    s = 2.0
    got = merge.merge(w_hat, A, B, s)
    for n in range(8):
        for k in range(0, 64, 7):
            exact = Fraction(float(w_hat[n, k])) + Fraction(s) * sum(
                Fraction(float(A[k, j])) * Fraction(float(B[j, n])) for j in range(8))
            want = np.float32(float(exact))          # nearest fp32 of the exact value
            assert got[n, k] == want, (n, k)


def test_close_to_a_plain_matrix_product():
    w_hat, A, B = _case(o=40, d=128, r=16, seed=4)
    s = 0.5
    got = merge.merge(w_hat, A, B, s)
    ref = (w_hat.astype(np.float64) + s * (A @ B).T).astype(np.float32)
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
    assert np.mean(got == ref) > 0.999


def test_nothing_to_merge_leaves_the_base():
    w_hat, A, B = _case()
    assert np.array_equal(merge.merge(w_hat, A, B, 0.0), w_hat)
    assert np.array_equal(merge.merge(w_hat, np.zeros_like(A), B, 2.0), w_hat)


def test_requantized_tensor_uses_the_blockwise_scheme():
    wl = synth.WORKLOADS["tiny_128"]
    W, X, A, B, dY = synth.layer_inputs(wl, wl.projs[0])
    c, s8, s2 = nf4.quantize(W.ravel())
    merged, c2, s82, s22 = merge.merge_and_requantize(c, s8, s2, W.shape, synth_bf16(A), synth_bf16(B), wl.s)
    rc, rs8, rs2 = nf4.quantize(merged.ravel())
    assert np.array_equal(c2, rc) and np.array_equal(s82, rs8) and np.array_equal(s22, rs2)
    # a small adapter moves only some codes: most survive the round trip
    assert 0.5 < np.mean(nf4.unpack_nibbles(c2, W.size) == nf4.unpack_nibbles(c, W.size)) < 1.0


def synth_bf16(bits):
    return nf4.bf16_bits_to_f64(bits)
