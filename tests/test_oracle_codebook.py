"""Pins of the oracle's NF4 codebook against what the pages and mathematics fix.

The pages fix: 16 values, built from normal quantiles, finer spacing near 0
and coarser in the tails, an exact zero, absmax normalisation to [−1, 1]
(074 QLoRA page §二; weimeta glossary "NF4 4-bit 量化是什么").  The exact tail
level is a reading (see oracle.nf4.P_MAX); the values are therefore pinned by
that construction, checked through a third, independent Φ⁻¹ (SciPy's ndtri).
"""

import math

import numpy as np
import pytest
from scipy import special

from oracle import nf4


@pytest.fixture(scope="module")
def V():
    return nf4.codebook()


def test_sixteen_ascending_values_one_exact_zero(V):
    assert V.dtype == np.float32 and V.size == 16
    assert np.all(np.diff(V.astype(np.float64)) > 0)
    assert np.count_nonzero(V == 0) == 1 and V[7] == 0.0
    assert V[0] == -1.0 and V[15] == 1.0
    assert np.count_nonzero(V > 0) == 8 and np.count_nonzero(V < 0) == 7


def test_spacing_finer_near_zero(V):
    v = V.astype(np.float64)
    pos_gaps = np.diff(v[7:])            # 0 → 1
    neg_gaps = -np.diff(v[:8][::-1])     # 0 → −1
    assert np.all(np.diff(pos_gaps) > 0)
    assert np.all(np.diff(neg_gaps) > 0)


def test_two_oracle_routes_agree_bitwise():
    a = nf4.codebook("wichura")
    b = nf4.codebook("bisect")
    assert a.tobytes() == b.tobytes()


def test_against_scipy_ndtri_third_route(V):
    """Rebuild the table from SciPy's Φ⁻¹ (Cephes ndtri, not used by the oracle)."""
    pm = 1.0 - 0.5 * (1.0 / 32 + 1.0 / 30)
    z = special.ndtri(pm)
    pos = [special.ndtri(0.5 + (pm - 0.5) * j / 8) / z for j in range(1, 9)]
    neg = [-special.ndtri(0.5 + (pm - 0.5) * j / 7) / z for j in range(1, 8)]
    ref = np.array(sorted(neg + [0.0] + pos), dtype=np.float64).astype(np.float32)
    assert ref.tobytes() == V.tobytes()


def test_equal_probability_mass_per_interval(V):
    """Each side splits the normal mass between the median and p_max evenly."""
    pm = 1.0 - 0.5 * (1.0 / 32 + 1.0 / 30)
    z = special.ndtri(pm)
    cdf = special.ndtr(V.astype(np.float64) * z)
    pos_steps = np.diff(cdf[7:])
    neg_steps = np.diff(cdf[:8])
    assert np.allclose(pos_steps, (pm - 0.5) / 8, rtol=0, atol=2e-7)
    assert np.allclose(neg_steps, (pm - 0.5) / 7, rtol=0, atol=2e-7)


def test_tail_level_is_between_the_two_halves_of_32_and_30():
    # p_max = 1 − (1/32 + 1/30)/2 lies halfway between 1 − 1/32 and 1 − 1/30.
    assert math.isclose(nf4.P_MAX, 0.5 * ((1 - 1 / 32) + (1 - 1 / 30)), rel_tol=0, abs_tol=1e-16)
