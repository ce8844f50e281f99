"""Pins of the AdamW oracle (fp32 steps) against the textbook fp64 update and
closed forms: the first step from zero state moves each parameter by about
lr·sign(g); with no momentum the update is g/|g|-like; a zero gradient leaves
pure decoupled decay; the bias corrections are the fp64 formula's."""

import numpy as np

from bounds import adamw_magnitudes, adamw_param_bound, adamw_state_bounds
from oracle import adamw, nf4


def _bf16(x):
    return nf4.bf16_bits_to_f64(nf4.bf16_rne_bits(np.asarray(x, np.float32))).astype(np.float32)


def _state(n=4096, seed=1):
    g = np.random.default_rng(seed)
    p = (g.standard_normal(n) * 0.02).astype(np.float32)
    grad = _bf16(g.standard_normal(n) * 1e-3)
    m = (g.standard_normal(n) * 1e-4).astype(np.float32)
    v = (np.abs(g.standard_normal(n)) * 1e-7).astype(np.float32)
    return p, grad, m, v


def test_matches_textbook_fp64_over_several_steps():
    p, g, m, v = _state()
    p64, m64, v64 = p.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    Mabs, Vabs = np.abs(m64), v64.copy()
    for t in range(1, 6):
        p, m, v, _ = adamw.step(p, g, m, v, t, lr=2e-4, wd=0.01)
        p64, m64, v64 = adamw.step_fp64(p64, g, m64, v64, t, lr=2e-4, wd=0.01)
        # the states carry fp32 rounding from each step: a few u per step of
        # the magnitudes the moments accumulate
        Mabs, Vabs = adamw_magnitudes(Mabs, Vabs, g)
        bm, bv = adamw_state_bounds(t, Mabs, Vabs)
        assert np.all(np.abs(m - m64) <= bm)
        assert np.all(np.abs(v - v64) <= bv)
        # p (|p| < 0.1) is rounded to fp32 once or twice per step
        assert np.max(np.abs(p - p64)) < adamw_param_bound(t)


def test_first_step_from_zero_state_is_lr_times_sign():
    p, g, _, _ = _state(seed=2)
    z = np.zeros_like(p)
    g[g == 0] = np.float32(1e-3)
    p2, m2, v2, _ = adamw.step(p, g, z, z, 1, lr=1e-3, eps=1e-12)
    np.testing.assert_allclose(p - p2, 1e-3 * np.sign(g), rtol=1e-5,
                               atol=2 * float(np.spacing(np.float32(0.1))))


def test_no_momentum_is_normalised_gradient():
    p, g, m, v = _state(seed=3)
    p2, m2, v2, _ = adamw.step(p, g, m, v, 7, lr=1e-3, b1=0.0, b2=0.0, eps=0.0)
    assert np.array_equal(m2, g) and np.array_equal(v2, g * g)
    nz = g != 0
    # p − p2 in fp32 carries the rounding of p (|p| ~ 0.02): two ulps
    np.testing.assert_allclose((p - p2)[nz], 1e-3 * np.sign(g[nz]), rtol=1e-6,
                               atol=2 * float(np.spacing(np.float32(0.1))))


def test_zero_gradient_and_state_is_pure_decay():
    p, _, _, _ = _state(seed=4)
    z = np.zeros_like(p)
    p2, _, _, b = adamw.step(p, z, z, z, 3, lr=0.1, wd=0.5)
    assert np.array_equal(p2, p * np.float32(1.0 - np.float32(0.1) * np.float32(0.5)))
    assert np.array_equal(b, nf4.bf16_rne_bits(p2))


def test_bias_corrections():
    c1, c2, rs, keep, lr1, e = adamw.constants(1e-3, 0.9, 0.999, 1e-8, 0.0, 3)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    assert np.isclose(lr1, np.float32(1e-3) / (1 - b1 ** 3), rtol=1e-7)
    assert np.isclose(rs, 1 / np.sqrt(1 - b2 ** 3), rtol=1e-7)
    assert keep == 1.0 and c1 == np.float32(1 - b1)


def test_state_bound_catches_a_wrong_update():
    """The state bound is tight enough that a wrong coefficient or a dropped
    term of the update breaks it."""
    p, g, m, v = _state(seed=5)
    Mabs, Vabs = adamw_magnitudes(np.abs(m.astype(np.float64)), v.astype(np.float64), g)
    bm, bv = adamw_state_bounds(1, Mabs, Vabs)
    _, m64, v64 = adamw.step_fp64(p.astype(np.float64), g, m.astype(np.float64), v.astype(np.float64), 1)
    _, m_bad, v_bad, _ = adamw.step(p, g, m, v, 1, b1=0.91)          # wrong beta1
    assert np.any(np.abs(m_bad - m64) > bm)
    _, m_ok, v_bad, _ = adamw.step(p, g, m, np.zeros_like(v), 1)     # v's carried term dropped
    assert np.any(np.abs(v_bad - v64) > bv)
