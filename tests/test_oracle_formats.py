"""Pins of the other 4-bit tables (int4, FP4 E2M1, FP4 E3M0) in the oracle.

The pages compare NF4 with these formats ([QLoRA-074 §四, Table 2]) without
printing their tables; each table is pinned here by an independent
construction (integer grid, IEEE minifloat decoding written separately,
powers of two), the encode by exact-rational brute force, and the claim that
NF4 suits normally distributed weights best by quantization error on
Gaussian data.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats, nf4


def brute_code(w: float, c1: float, V) -> int:
    """argmin_k |w/c1 − V[k]| in exact rationals, ties to the lower index,
    except that where a table holds both −0 and +0 a weight that rounds to
    zero keeps its sign: +0 for w/c1 > 0, −0 otherwise."""
    if c1 == 0:
        return 7
    x = Fraction(w) / Fraction(c1)
    dists = [abs(x - Fraction(float(v))) for v in V]
    k = dists.index(min(dists))
    if float(V[k]) == 0.0 and k + 1 < len(V) and float(V[k + 1]) == 0.0 and x > 0:
        k += 1
    return k


def test_int4_is_the_integer_grid():
    V = formats.codebook("int4")
    assert V.dtype == np.float32 and V.size == 16
    for i, v in enumerate(V):
        assert v == np.float32((i - 8) / 7.0)
    assert V[8] == 0.0 and V[1] == -1.0 and V[15] == 1.0


def test_int4_encode_is_round_half_down_of_w_times_7():
    """For int4 the nearest value is an integer rounding of 7·w/c1 (ties to the
    lower integer), computed here with Fractions, not through midpoints."""
    w = (np.random.default_rng(3).standard_normal(64 * 8) * 0.02).astype(np.float32)
    w[:8] = [0.0, -0.0, 0.01, -0.01, 0.005, 0.0, 0.0, 0.0]
    c1 = nf4.block_absmax(w)
    k = nf4.nf4_encode(w, c1, formats.codebook("int4"))
    for i, wi in enumerate(w):
        c = Fraction(float(c1[i // 64]))
        y = Fraction(float(wi)) * 7 / c              # in [-7, 7]
        j = -((-(2 * y - 1)) // 2)                   # ceil(y - 1/2): halves go down
        assert k[i] == j + 8, (i, float(wi))


def test_e2m1_table_is_the_minifloat_value_set():
    # textbook FP4 E2M1 magnitudes, scaled by their maximum
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    want = sorted([-m / 6.0 for m in mags[1:]] + [-0.0, 0.0] + [m / 6.0 for m in mags[1:]])
    V = formats.codebook("fp4_e2m1")
    assert [float(v) for v in V] == [float(np.float32(x)) for x in want]
    assert np.signbit(V[7]) and not np.signbit(V[8])      # −0 then +0


def test_e3m0_table_is_signed_powers_of_two():
    V = formats.codebook("fp4_e3m0")
    pos = [float(v) for v in V[8:]]
    assert pos == [0.0] + [2.0 ** -k for k in range(6, -1, -1)]
    assert [float(v) for v in V[:8]] == [-x for x in reversed(pos)]


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_every_table_ascends_within_unit_range(fmt):
    V = formats.codebook(fmt).astype(np.float64)
    assert np.all(np.diff(V) >= 0) and V[-1] == 1.0 and np.any(V == 0.0)
    if fmt == "int4":
        assert V[1] == -1.0 and V[0] < -1.0          # -8/7 is never the nearest value
    else:
        assert V[0] == -1.0


@pytest.mark.parametrize("fmt", ["int4", "fp4_e2m1", "fp4_e3m0"])
def test_encode_matches_exact_brute_force(fmt):
    V = formats.codebook(fmt)
    w = (np.random.default_rng(7).standard_normal(64 * 5) * 0.02).astype(np.float32)
    w[3], w[70] = 0.0, -0.0
    c1 = nf4.block_absmax(w)
    # weights exactly on the midpoints of the last block (ties go down)
    vd = V.astype(np.float64)
    mids = (vd[:-1] + vd[1:]) / 2
    c = float(c1[-1])
    for t, m in enumerate(mids):
        x = np.float32(m * c)
        if float(x) == m * c:
            w[64 * 4 + 1 + t] = x
    c1 = nf4.block_absmax(w)
    k = nf4.nf4_encode(w, c1, V)
    for i, wi in enumerate(w):
        assert k[i] == brute_code(float(wi), float(c1[i // 64]), V), (fmt, i)


def test_second_level_does_not_depend_on_the_table():
    w = synth.normal_f32((16384 * 3,), 0.02, [11, 0, 0])
    ref = formats.quantize(w, "nf4")
    for fmt in ("int4", "fp4_e2m1", "fp4_e3m0"):
        c, s8, s2 = formats.quantize(w, fmt)
        assert np.array_equal(s8, ref[1]) and np.array_equal(s2, ref[2])


def test_nf4_has_the_lowest_error_on_gaussian_weights():
    """NF4 places its values at normal quantiles, so on N(0, σ) weights its
    blockwise quantization error is the smallest of the four formats; E3M0,
    with its coarse powers of two, is the largest."""
    w = synth.normal_f32((1 << 18,), 0.02, [12, 0, 0])
    mse = {fmt: formats.quantization_mse(w, fmt) for fmt in formats.FORMATS}
    assert mse["nf4"] < min(mse["int4"], mse["fp4_e2m1"], mse["fp4_e3m0"])
    assert mse["fp4_e3m0"] > max(mse["nf4"], mse["int4"], mse["fp4_e2m1"])
