"""Oracle: other 4-bit codebooks run through the same blockwise + double-quant path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  [QLoRA-074 §四, Table 2]
compares NF4 with plain 4-bit integers and two 4-bit float layouts, E2M1 and
E3M0.  All four are used the same way: a 16-entry table of values in
[-1, 1] scaled by the block absmax, nearest value with ties to the lower
index.  The pages name the formats but do not give their tables; the
readings taken are written out with each function below, built from the
bit layout of each format, not from any library.

The encode is oracle.nf4.nf4_encode: k = number of midpoints strictly below
w/c1.  With distinct values that is the nearest value with ties to the
lower index; the FP4 tables hold both −0 and +0 (midpoint 0), so a weight
that rounds to zero keeps its sign (+0 for w > 0, −0 for w ≤ 0).
"""

from __future__ import annotations

import numpy as np

from . import nf4

FORMATS = ("nf4", "int4", "fp4_e2m1", "fp4_e3m0")


def int4_values() -> list[float]:
    """Signed 4-bit integers -8..7, scaled so that the absmax maps to 7.

    Reading: absmax scaling to 7 (a symmetric range), so the code -8 lies at
    -8/7 < -1 and is never the nearest value of a weight with |w| ≤ c1.
    """
    return [(i - 8) / 7.0 for i in range(16)]


def _minifloat(sign: int, e: int, m: int, ebits: int, mbits: int, bias: int) -> float:
    """Value of an IEEE-style minifloat with subnormals and no inf/NaN codes."""
    s = -1.0 if sign else 1.0
    if e == 0:                                    # subnormal (or zero)
        return s * (m / (1 << mbits)) * 2.0 ** (1 - bias)
    return s * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)


def e2m1_values() -> list[float]:
    """FP4 E2M1 (1 sign, 2 exponent, 1 mantissa bit, bias 1): ±{0, .5, 1,
    1.5, 2, 3, 4, 6}; divided by 6 so the largest magnitude is 1.  Both
    zeros are kept, giving 16 entries."""
    vals = []
    for code in range(16):
        sign, e, m = code >> 3, (code >> 1) & 3, code & 1
        vals.append(_minifloat(sign, e, m, 2, 1, 1) / 6.0)
    return sorted(vals, key=lambda v: (v, 0 if np.copysign(1.0, v) < 0 else 1))


def e3m0_values() -> list[float]:
    """FP4 E3M0 (1 sign, 3 exponent bits, no mantissa): exponent field 0 is
    zero, fields 1..7 are 2^(e-7), so the magnitudes are 0 and 1/64 .. 1.
    Reading: the bias is chosen so that the largest magnitude is 1."""
    vals = []
    for code in range(16):
        sign, e = code >> 3, code & 7
        mag = 0.0 if e == 0 else 2.0 ** (e - 7)
        vals.append(-mag if sign else mag)
    return sorted(vals, key=lambda v: (v, 0 if np.copysign(1.0, v) < 0 else 1))


def codebook(fmt: str) -> np.ndarray:
    """16 ascending fp32 values of a format (NF4 from oracle.nf4)."""
    if fmt == "nf4":
        return nf4.codebook()
    table = {"int4": int4_values, "fp4_e2m1": e2m1_values, "fp4_e3m0": e3m0_values}[fmt]()
    return np.array(table, dtype=np.float64).astype(np.float32)


def quantize(w: np.ndarray, fmt: str):
    """Blockwise 4-bit + double quantization with the format's table."""
    return nf4.quantize_chunked(w, V=codebook(fmt))


def dequant_f32(codes, scale8, scale2, n: int, fmt: str) -> np.ndarray:
    return nf4.dequant_f32(codes, scale8, scale2, n, codebook(fmt))


def quantization_mse(w: np.ndarray, fmt: str) -> float:
    """Mean squared error of the fp32 dequantized weights against w."""
    w = np.asarray(w, dtype=np.float32).ravel()
    c, s8, s2 = quantize(w, fmt)
    d = dequant_f32(c, s8, s2, w.size, fmt).astype(np.float64)
    return float(np.mean((d - w.astype(np.float64)) ** 2))
