"""Pins of the double-quantization variants with a tensor offset (oracle.dq).

The E4M3 table is checked against values fixed by the format; the tensor
mean against an exactly rounded sum; both second-level encoders against
exact-rational brute force over every code (with their tie rules); the
reconstruction against its error bound; and the first-level codes against
the default scheme (the variants change only the constants)."""

import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import dq, nf4


def test_e4m3_table():
    V = dq.e4m3_values()
    assert V.size == 127 and np.all(np.diff(V) > 0)
    assert V[0] == 0.0 and V[1] == 2.0 ** -9 and V[8] == 2.0 ** -6        # smallest subnormal, normal
    assert V[0x38] == 1.0 and V[-1] == 448.0 and V[0x7E] == 448.0
    assert V[0x3C] == 1.5 and V[0x47] == 3.75                               # 1.1b, 1.111b·2


def test_mean_is_the_rounded_exact_mean():
    c1 = np.abs(synth.normal_f32((256 * 37 + 11,), 0.05, [5, 0, 0]))
    mu = dq.tensor_mean(c1)
    exact = math.fsum(float(x) for x in c1) / c1.size
    assert abs(float(mu) - exact) <= float(np.spacing(np.float32(exact)))


def _c1(seed, nb=256 * 3 + 17):
    c = np.abs(synth.normal_f32((nb,), 0.03, [seed, 0, 0])) + np.float32(0.01)
    c[5] = 0.0                                  # a zero block
    return c


@pytest.mark.parametrize("variant", ["int8_mean", "fp8_mean"])
def test_encoder_is_the_exact_nearest_code(variant):
    c1 = _c1(1)
    s8, s2 = dq.second_level(c1, variant)
    nb = c1.size
    ng = -(-nb // 256)
    mu = Fraction(float(s2[ng]))
    if variant == "int8_mean":
        cand = [(q, Fraction(q)) for q in range(-127, 128)]
    else:
        V = dq.e4m3_values()
        cand = [(k, Fraction(float(V[k]))) for k in range(127)]
        cand += [(0x80 | k, -Fraction(float(V[k]))) for k in range(1, 127)]
    for b in range(0, nb, 7):
        step = Fraction(float(s2[b // 256]))
        cp = Fraction(float(np.float32(c1[b] - np.float32(s2[ng]))))
        if step == 0:
            assert s8[b] == 0
            continue
        x = cp / step
        best = min(abs(x - val) for _, val in cand)
        ties = [(code, val) for code, val in cand if abs(x - val) == best]
        if variant == "int8_mean":
            want = min(ties, key=lambda cv: abs(cv[1]))[0] & 0xFF       # ties: smaller magnitude
        else:
            want = [code for code, val in ties if (code & 1) == 0][0] if len(ties) > 1 else ties[0][0]
        assert s8[b] == want, (variant, b)
    assert np.isclose(float(s2[ng]), float(np.mean(c1.astype(np.float64))), rtol=1e-6)


@pytest.mark.parametrize("variant,rel", [("int8_mean", None), ("fp8_mean", 2.0 ** -4)])
def test_reconstruction_error_bound(variant, rel):
    c1 = _c1(2)
    s8, s2 = dq.second_level(c1, variant)
    nb, ng = c1.size, -(-c1.size // 256)
    ch = dq.chat(s8, s2, nb, variant).astype(np.float64)
    step = np.repeat(s2[:ng].astype(np.float64), 256)[:nb]
    cp = np.abs((c1 - s2[ng]).astype(np.float64))
    ulp = np.spacing(np.abs(ch).astype(np.float32)).astype(np.float64) * 2
    if rel is None:
        assert np.all(np.abs(ch - c1) <= step / 2 + ulp)
    else:   # E4M3 has 3 mantissa bits: half-ulp relative 2^-4, and subnormal steps 2^-10·448·step
        assert np.all(np.abs(ch - c1) <= rel * cp + step * 2.0 ** -10 + ulp)


@pytest.mark.parametrize("variant", ["int8_mean", "fp8_mean"])
def test_codes_unchanged_and_dequant_close(variant):
    w = synth.normal_f32((16384 * 2 + 640,), 0.02, [9, 0, 0])
    c, s8, s2 = dq.quantize(w, variant)
    rc, _, _ = nf4.quantize(w)
    assert np.array_equal(c, rc)
    d = dq.dequant_f32(c, s8, s2, w.size, variant)
    base = nf4.dequant_f32(*nf4.quantize(w), w.size)
    # the second level moves ĉ by at most a small fraction: dequant stays close to the default
    assert np.max(np.abs(d - base)) < 0.05 * np.max(np.abs(w))
    assert abs(dq.quantization_mse(w, variant) / w.var() - 0.0085) < 0.001
