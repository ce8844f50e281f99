"""Oracle: second-level (double) quantization variants with a tensor offset.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[QLoRA-074 §二] stores the first-level constants in 8 bits with one fp32
constant per 256 of them and notes that offsets also exist but are left out
of its accounting; the LoRA-PyTorch page (garbled) speaks of an FP8 code of
the constants.  The default scheme (oracle.nf4) is an unsigned linear code
with no offset.  These variants centre the constants on their tensor mean
first, which is how the QLoRA paper's double quantization is usually
described; the pages fix neither variant, so every step below is a reading:

  μ   = fl32(S / nb): S sums the fp32 constants in fp64, each 256-block group
        in increasing block order, then the group sums in increasing order.
  c'  = fl32(c1 − μ) per block.
  int8_mean: per group step = fl32(max|c'| / 127); q ∈ [−127, 127] the
        integer nearest to c'/step, ties to the smaller magnitude; stored as
        the byte of the two's-complement int8.  ĉ = fl32(fl32(q·step) + μ).
  fp8_mean:  per group step = fl32(max|c'| / 448); q the FP8 E4M3 value
        (bias 7, subnormals, no infinities, largest finite 448) nearest to
        c'/step, ties to the even mantissa; stored as its bit pattern.
        ĉ = fl32(fl32(value(q)·step) + μ).
  A group with max|c'| = 0 has step 0 and codes 0.

The first-level codes are the NF4 codes computed with the exact c1, as in the
default scheme [QLoRA-074 §三 order].  scale2 holds the ng steps followed by μ.
"""

from __future__ import annotations

import numpy as np

from . import nf4

VARIANTS = ("uint8", "int8_mean", "fp8_mean")


def tensor_mean(c1: np.ndarray) -> np.float32:
    c1 = np.asarray(c1, np.float32)
    nb = c1.size
    ng = -(-nb // nf4.GROUP)
    padded = np.zeros(ng * nf4.GROUP, np.float64)
    padded[:nb] = c1
    blocks = padded.reshape(ng, nf4.GROUP)
    psum = np.zeros(ng)
    for b in range(nf4.GROUP):               # increasing block order in each group
        psum += blocks[:, b]
    total = 0.0
    for g in range(ng):                      # then the groups in order
        total += float(psum[g])
    return np.float32(total / nb)


def e4m3_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, indexed by their 7-bit code."""
    vals = []
    for code in range(127):                  # 0x7F is NaN
        e, m = code >> 3, code & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def _group_absmax(x: np.ndarray, ng: int) -> np.ndarray:
    padded = np.zeros(ng * nf4.GROUP, np.float32)
    padded[: x.size] = np.abs(x)
    return padded.reshape(ng, nf4.GROUP).max(axis=1)


def second_level(c1: np.ndarray, variant: str):
    """(scale8 u8[nb], scale2 f32[ng + 1]) of a variant (the last float is μ)."""
    c1 = np.asarray(c1, np.float32)
    nb = c1.size
    ng = -(-nb // nf4.GROUP)
    mu = tensor_mean(c1)
    cp = (c1 - mu).astype(np.float32)                       # one fp32 rounding
    a = _group_absmax(cp, ng)
    top = 127.0 if variant == "int8_mean" else 448.0
    step = (a.astype(np.float64) / top).astype(np.float32)
    stepd = np.repeat(step.astype(np.float64), nf4.GROUP)[:nb]
    x = np.abs(cp.astype(np.float64))
    if variant == "int8_mean":
        q = np.zeros(nb, np.int64)
        for j in range(127):                                # half-steps strictly below |c'|
            q += x > (2 * j + 1) * stepd / 2.0
        q[stepd == 0.0] = 0
        q = np.where(cp < 0, -q, q)
        s8 = (q & 0xFF).astype(np.uint8)
    elif variant == "fp8_mean":
        V = e4m3_values()
        mids = (V[:-1] + V[1:]) / 2.0
        k = np.zeros(nb, np.int64)
        for t, mval in enumerate(mids):
            thr = mval * stepd                              # exact in fp64
            above = x > thr
            tie = x == thr
            # at a tie keep the even mantissa: the upper code if it is even
            k += above | (tie & (((t + 1) & 1) == 0))
        k[stepd == 0.0] = 0
        s8 = (k | np.where(cp < 0, 0x80, 0)).astype(np.uint8)
        s8[(k == 0)] = 0                                    # +0, never −0
    else:
        raise ValueError(variant)
    return s8, np.concatenate([step, [mu]]).astype(np.float32)


def chat(scale8: np.ndarray, scale2: np.ndarray, nb: int, variant: str) -> np.ndarray:
    """fp32 ĉ per block."""
    ng = -(-nb // nf4.GROUP)
    step = np.repeat(np.asarray(scale2[:ng], np.float32), nf4.GROUP)[:nb]
    mu = np.float32(scale2[ng])
    s8 = np.asarray(scale8[:nb], np.uint8)
    if variant == "int8_mean":
        qv = s8.view(np.int8).astype(np.float32)
    else:
        V = e4m3_values()
        mag = V[np.minimum(s8 & 0x7F, 126)].astype(np.float32)
        qv = np.where(s8 & 0x80, -mag, mag).astype(np.float32)
    return (qv * step).astype(np.float32) + mu             # two fp32 roundings


def quantize(w: np.ndarray, variant: str, V: np.ndarray | None = None):
    """(codes, scale8, scale2 with μ appended) of the NF4 codes with a DQ variant."""
    w = np.asarray(w, np.float32).ravel()
    codes, _, _ = nf4.quantize_chunked(w, V=V)
    s8, s2 = second_level(nf4.block_absmax(w), variant)
    return codes, s8, s2


def dequant_f32(codes, scale8, scale2, n: int, variant: str, V=None) -> np.ndarray:
    if V is None:
        V = nf4.codebook()
    nb = -(-n // nf4.BLOCK)
    c = chat(scale8, scale2, nb, variant)
    k = nf4.unpack_nibbles(codes, n)
    return V.astype(np.float32)[k] * c[np.arange(n) // nf4.BLOCK]


def quantization_mse(w: np.ndarray, variant: str) -> float:
    w = np.asarray(w, np.float32).ravel()
    c, s8, s2 = quantize(w, variant)
    d = dequant_f32(c, s8, s2, w.size, variant).astype(np.float64)
    return float(np.mean((d - w.astype(np.float64)) ** 2))
