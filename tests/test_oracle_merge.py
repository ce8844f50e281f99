"""Pins of the merge-and-requantize oracle.

The merged weight is pinned against the exact value (rational arithmetic on
small inputs, an fp64 matrix product at larger ones) within the error bound
of r sequential fp32 roundings plus two more, against the fp32 rounding of
the exact result for most elements, and against the cases where the
merge must leave the base untouched (s = 0, zero adapter).
"""

from fractions import Fraction

import numpy as np

import synth
from bounds import merge_bound
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


def _bound(w_hat, A, B, s, r):
    return merge_bound(w_hat, A, B, s, r)


def test_exact_rational_on_small_inputs():
    w_hat, A, B = _case(o=8, d=64, r=8)
    s = 2.0
    got = merge.merge(w_hat, A, B, s)
    bound, _ = _bound(w_hat, A, B, s, 8)
    for n in range(8):
        for k in range(0, 64, 7):
            exact = Fraction(float(w_hat[n, k])) + Fraction(s) * sum(
                Fraction(float(A[k, j])) * Fraction(float(B[j, n])) for j in range(8))
            assert abs(Fraction(float(got[n, k])) - exact) <= Fraction(float(bound[n, k])), (n, k)


def test_within_the_rounding_bound_of_the_exact_merge():
    w_hat, A, B = _case(o=40, d=128, r=64, seed=4)
    s = 0.5
    got = merge.merge(w_hat, A, B, s)
    bound, exact = _bound(w_hat, A, B, s, 64)
    assert np.all(np.abs(got.astype(np.float64) - exact) <= bound)
    # and mostly the fp32 rounding of the exact value itself (64 fp32
    # roundings of the rank sum move the last bit of about one in ten)
    assert np.mean(got == exact.astype(np.float32)) > 0.8


def test_a_transposed_or_missing_term_breaks_the_bound():
    w_hat, A, B = _case(o=32, d=64, r=16, seed=6)
    bound, exact = _bound(w_hat, A, B, 2.0, 16)
    wrong = merge.merge(w_hat, A[:, :15], B[:15], 2.0)        # a dropped rank term
    assert np.any(np.abs(wrong.astype(np.float64) - exact) > bound)
    wrong = merge.merge(w_hat, A, B, -2.0)                     # a wrong sign
    assert np.any(np.abs(wrong.astype(np.float64) - exact) > bound)


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
