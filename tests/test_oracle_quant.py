"""Pins of the oracle's blockwise NF4 encode, double quantization and dequant.

Pinned against: the pages' worked example and bit accounting (golden files),
exact rational brute force (Python Fractions, an arithmetic independent of
the oracle's fp64 thresholds), an exact correctly-rounded fp32 division, the
exact-zero round trip, endpoint invariants and a closed-form error bound.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nf4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        return json.load(f)


@pytest.fixture(scope="module")
def V():
    return nf4.codebook()


# ---------------------------------------------------------------- exact helpers

def round_to_f32(x: Fraction) -> float:
    """Exact nearest-even rounding of a rational to fp32 (normal or subnormal)."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    e = max(e, -126)
    scale = Fraction(2) ** (e - 23)
    m = x / scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * scale)


def brute_code(w: float, c1: float, V) -> int:
    """argmin_k |w/c1 − V[k]| in exact rationals, ties to the lower index."""
    if c1 == 0:
        return 7
    x = Fraction(w) / Fraction(c1)
    dists = [abs(x - Fraction(float(v))) for v in V]
    best = min(dists)
    return dists.index(best)


def brute_q8(c1: float, step: float) -> int:
    if step == 0:
        return 0
    dists = [abs(q * Fraction(step) - Fraction(c1)) for q in range(256)]
    return dists.index(min(dists))


# ---------------------------------------------------------------- page pins

def test_worked_example_sizes():
    g = gold("worked_example.json")
    codes, s8, s2 = nf4.sizes(g["weights"])
    assert codes == g["code_bytes"]
    assert s8 == g["scale8_bytes"] and s2 == g["scale2_bytes"]
    assert s8 + s2 == g["dq_scale_bytes"]
    nb = -(-g["weights"] // nf4.BLOCK)
    assert nb == g["blocks"] and 4 * nb == g["fp32_scale_bytes"]
    assert 4 * nb - (s8 + s2) == g["saved_bytes"]
    # and the quantizer really emits buffers of those sizes
    w = np.random.default_rng(0).standard_normal(g["weights"]).astype(np.float32) * 0.02
    c, q8, st = nf4.quantize(w)
    assert c.nbytes == g["code_bytes"] and q8.nbytes == g["scale8_bytes"] and st.nbytes == g["scale2_bytes"]


def test_bit_accounting():
    g = gold("accounting.json")
    nd = g["printed_decimals"]
    for k in (1, 3, 1024):
        n = 16384 * k
        c, s8, s2 = nf4.sizes(n)
        fp32_bits = Fraction(32 * (n // 64), n)
        dq_bits = Fraction(8 * (s8 + s2), n)
        total = Fraction(8 * (c + s8 + s2), n)
        assert fp32_bits == Fraction(1, 2) == Fraction(g["fp32_scale_bits_per_param"])
        assert dq_bits == Fraction(8, 64) + Fraction(32, 64 * 256) == Fraction(130, 1024)
        assert total == Fraction(4) + dq_bits
        assert round(float(dq_bits), nd) == g["dq_bits_per_param_approx"]
        assert round(float(fp32_bits - dq_bits), nd) == g["saving_bits_per_param_approx"]
        assert round(float(total), nd) == g["total_bits_per_param_approx"]
    assert float(Fraction(4) + Fraction(130, 1024)) == 4.126953125


def test_layer_4096_example():
    g = gold("layer_4096.json")
    n = g["rows"] * g["cols"]
    assert round(n / 1e6, 2) == g["params_millions_approx"]
    assert n * 2 == g["bf16_mib"] * 2**20
    codes, _, _ = nf4.sizes(n)
    assert codes == g["nf4_code_mib"] * 2**20
    r = g["lora_rank"]
    lora = r * g["rows"] + r * g["cols"]
    assert lora == g["lora_params"]
    assert 100.0 * lora / n == g["lora_percent"]


# ---------------------------------------------------------------- encode pins

def _random_weights(n, seed, std=0.02):
    return (np.random.default_rng(seed).standard_normal(n) * std).astype(np.float32)


def test_encode_matches_exact_brute_force_random(V):
    w = _random_weights(64 * 6, 1)
    w[5] = 0.0
    w[70] = -0.0
    c1 = nf4.block_absmax(w)
    k = nf4.nf4_encode(w, c1, V)
    for i, wi in enumerate(w):
        assert k[i] == brute_code(float(wi), float(c1[i // 64]), V), i


def test_encode_ties_go_to_lower_index(V):
    """Weights placed exactly on the midpoints between codebook values."""
    vd = V.astype(np.float64)
    mids = (vd[:-1] + vd[1:]) / 2
    rows = []
    for scale_exp in (0, -5, -20):
        c1 = 2.0 ** scale_exp
        blk = np.zeros(64, dtype=np.float64)
        blk[0] = c1
        j = 1
        for t, m in enumerate(mids):
            x = m * c1
            if np.float32(x) == x:       # midpoint representable: an exact tie
                blk[j] = x
                j += 1
            xf = np.float32(x)
            blk[j] = np.nextafter(xf, np.float32(np.inf))
            blk[j + 1] = np.nextafter(xf, np.float32(-np.inf))
            j += 2
        rows.append(blk[:64])
    w = np.concatenate(rows).astype(np.float32)
    c1 = nf4.block_absmax(w)
    k = nf4.nf4_encode(w, c1, V)
    n_ties = 0
    for i, wi in enumerate(w):
        b = brute_code(float(wi), float(c1[i // 64]), V)
        assert k[i] == b, (i, float(wi))
        x = Fraction(float(wi)) / Fraction(float(c1[i // 64]))
        if any(x == (Fraction(float(V[t])) + Fraction(float(V[t + 1]))) / 2 for t in range(15)):
            n_ties += 1
    assert n_ties >= 3


def test_endpoints_and_zero_block(V):
    w = _random_weights(64 * 256 * 2, 2)
    w[64 * 3: 64 * 4] = 0.0                        # an all-zero block
    c1 = nf4.block_absmax(w)
    k = nf4.nf4_encode(w, c1, V)
    kb = k.reshape(-1, 64)
    wb = w.reshape(-1, 64)
    for b in range(kb.shape[0]):
        if c1[b] == 0:
            assert np.all(kb[b] == 7)
            continue
        imax = int(np.argmax(np.abs(wb[b])))
        assert kb[b, imax] == (15 if wb[b, imax] > 0 else 0)


# ---------------------------------------------------------------- double quant pins

def test_step_is_correctly_rounded_division():
    rng = np.random.default_rng(3)
    c1 = np.abs(rng.standard_normal(256 * 40) * rng.choice([1e-3, 1, 1e30, 1e-38], 256 * 40)).astype(np.float32)
    step = nf4.second_level_step(c1)
    c2 = c1.reshape(-1, 256).max(axis=1)
    for g in range(c2.size):
        assert float(step[g]) == round_to_f32(Fraction(float(c2[g])) / 255)


def test_scale_code_matches_exact_brute_force():
    rng = np.random.default_rng(4)
    c1 = (np.abs(rng.standard_normal(256 * 3)) * 0.05).astype(np.float32)
    # group 1: c1 exactly on half-steps (ties → lower q)
    step_exact = 2.0 ** -10
    c1[256] = np.float32(255 * step_exact)         # group max → step exactly 2^-10
    for j in range(1, 200):
        c1[256 + j] = np.float32((j % 250 + 0.5) * step_exact)
    # group 2 is all zero
    c1[512:] = 0.0
    step = nf4.second_level_step(c1)
    assert step[1] == np.float32(step_exact) and step[2] == 0.0
    q8 = nf4.scale_encode(c1, step)
    for b in range(c1.size):
        assert q8[b] == brute_q8(float(c1[b]), float(step[b // 256])), b
    # the largest constant of each non-zero group maps to the top code
    for g in (0, 1):
        assert q8[g * 256 + int(np.argmax(c1[g * 256:(g + 1) * 256]))] == 255


# ---------------------------------------------------------------- dequant pins

def test_exact_zero_round_trip():
    w = _random_weights(16384 * 2 + 100, 5)
    zi = np.random.default_rng(6).choice(w.size, 500, replace=False)
    w[zi] = 0.0
    w[16384: 16384 + 64] = 0.0     # whole zero block
    c, q8, st = nf4.quantize(w)
    wh = nf4.dequant_f32(c, q8, st, w.size)
    assert np.all(wh[zi] == 0.0)
    assert np.all(wh[16384: 16384 + 64] == 0.0)
    assert not np.signbit(wh[zi]).any()


def test_dequant_is_two_fp32_products(V):
    """Dequant written per element in exact rationals, then rounded once per product."""
    w = _random_weights(16384 + 640, 7)
    c, q8, st = nf4.quantize(w)
    wh = nf4.dequant_f32(c, q8, st, w.size)
    k = nf4.unpack_nibbles(c, w.size)
    idx = np.random.default_rng(8).choice(w.size, 300, replace=False)
    for i in idx:
        b, g = i // 64, i // (64 * 256)
        chat = round_to_f32(Fraction(int(q8[b])) * Fraction(float(st[g])))
        ref = round_to_f32(Fraction(float(V[k[i]])) * Fraction(chat))
        assert float(wh[i]) == ref


def test_error_bound():
    """|w − ŵ| ≤ (largest half-gap)·c1 + |c1 − ĉ| + ½ulp, with |c1 − ĉ| ≤ d/2 + ½ulp(ĉ)."""
    V = nf4.codebook().astype(np.float64)
    half_gap = np.max(np.diff(V)) / 2
    for std in (0.02, 1.0, 1e-6):
        w = _random_weights(16384 * 3, 9, std)
        c, q8, st = nf4.quantize(w)
        wh = nf4.dequant_f32(c, q8, st, w.size).astype(np.float64)
        c1 = nf4.block_absmax(w).astype(np.float64)
        step = np.repeat(st.astype(np.float64), 256)
        chat = q8.astype(np.float32) * np.repeat(st, 256)
        assert np.all(np.abs(c1 - chat) <= step / 2 + np.spacing(np.abs(chat).astype(np.float32)) / 2 + 0)
        bound = half_gap * np.repeat(c1, 64) + np.repeat(np.abs(c1 - chat), 64) \
            + np.spacing(np.abs(wh).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(w.astype(np.float64) - wh) <= bound)


def test_bf16_rounding_against_torch_and_ties():
    x = np.array([1.0, 1.00390625, 1.01171875, -1.00390625, 3.0e-39, 1e30, 0.1, -0.0],
                 dtype=np.float32)
    bits = nf4.bf16_rne_bits(x)
    assert bits[1] == 0x3F80          # tie → even (1.0)
    assert bits[2] == 0x3F82          # tie → even (1.015625)
    rnd = np.random.default_rng(10).standard_normal(100000).astype(np.float32)
    allx = np.concatenate([x, rnd, rnd * 1e-39, rnd * 1e20])
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.bf16_rne_bits(allx), ref)


# ---------------------------------------------------------------- layout pins

def test_tails_and_padding():
    for n in (1, 63, 65, 127, 16383, 16385, 16384 * 2 + 7):
        w = _random_weights(n, n)
        c, q8, st = nf4.quantize(w)
        cb, s8b, s2b = nf4.sizes(n)
        assert c.nbytes == cb and q8.nbytes == s8b and st.nbytes == s2b
        assert np.all(nf4.unpack_nibbles(c, cb * 2)[n:] == 7)
        wh = nf4.dequant_f32(c, q8, st, n)
        c1 = nf4.block_absmax(w)
        assert np.all(np.abs(wh - w) <= 0.16 * np.repeat(c1, 64)[:n] + 1e-30)


def test_chunked_equals_whole():
    w = _random_weights(16384 * 5 + 300, 11)
    a = nf4.quantize(w)
    b = nf4.quantize_chunked(w, chunk=16384 * 2)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


def test_nibble_order():
    k = np.arange(16, dtype=np.uint8)
    packed = nf4.pack_nibbles(k)
    assert packed.tolist() == [0x40, 0x51, 0x62, 0x73, 0xC8, 0xD9, 0xEA, 0xFB]
    assert nf4.unpack_nibbles(packed, 16).tolist() == k.tolist()
    # 4 bits per code: two codes per byte whenever 8 divides n; a ragged tail is padded with 7
    p3 = nf4.pack_nibbles(np.array([1, 2, 3], dtype=np.uint8))
    assert p3.tolist() == [0x71, 0x72, 0x73, 0x77]
    for n in (8, 16384, 4096 * 4096):
        assert nf4.sizes(n)[0] * 2 == n
