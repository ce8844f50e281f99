"""Oracle: NF4 codebook, blockwise NF4 encode, double quantization, dequant.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy / Python,
fp64 or exact arithmetic; written from the pages, not from any library.

Layout (reading of the pages): the tensor is a flat array of n fp32 weights.
Element i lies in block b = i // 64 and double-quant group g = b // 256.
For a linear layer stored row-major as Wq[o][d], i = row*d + col, so blocks
run along d.  The pages fix 4 bits per code (two per byte) but not their
order; the reading taken packs each run of 8 consecutive codes into one
little-endian 32-bit word, byte j (j = 0..3) holding code j in bits 3:0 and
code j+4 in bits 7:4.  Missing codes past n are padded with code 7 (the zero
code), so the code buffer is 4·ceil(n/8) bytes (n/2 whenever 8 divides n).
"""

from __future__ import annotations

import math
import statistics

import numpy as np

BLOCK = 64      # weights per first-level absmax block  [QLoRA-074 §二]
GROUP = 256     # first-level constants per second-level constant  [QLoRA-074 §二]

# Tail quantile of the codebook.  The pages only say the 16 values follow
# normal quantiles with an exact zero [QLoRA-074 §二]; the offset below is the
# one of the QLoRA paper that page summarises: p_max = 1 - (1/32 + 1/30) / 2.
P_MAX = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


# --------------------------------------------------------------------------
# Φ⁻¹ by two independent routes
# --------------------------------------------------------------------------

def inv_cdf_wichura(p: float) -> float:
    """Standard normal quantile via Python's NormalDist (Wichura's AS241)."""
    return statistics.NormalDist().inv_cdf(p)


def inv_cdf_bisect(p: float) -> float:
    """Standard normal quantile by bisection on Φ(x) = erfc(-x/√2)/2, in fp64.

    Runs until the bracket can no longer shrink, so the result is the fp64
    number where the computed Φ crosses p.
    """
    lo, hi = -40.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# --------------------------------------------------------------------------
# Codebook  [QLoRA-074 §二: 16 values from normal quantiles, finer near 0,
# coarser in the tails, exact zero, absmax-normalised; QLoRA-glossary:
# the normal curve cut into 16 quantile intervals]
# --------------------------------------------------------------------------

def codebook_f64(route: str = "wichura") -> list[float]:
    """The 16 NF4 values in fp64, ascending.

    One exact zero and 16 values force an asymmetric split; the reading taken
    is 8 positive and 7 negative values:
      positive  q_j = Φ⁻¹(1/2 + j·(p_max − 1/2)/8),   j = 1..8
      negative  −Φ⁻¹(1/2 + j·(p_max − 1/2)/7),         j = 1..7
    all divided by Φ⁻¹(p_max) so the ends are exactly −1 and +1.
    """
    inv = {"wichura": inv_cdf_wichura, "bisect": inv_cdf_bisect}[route]
    half_span = P_MAX - 0.5
    z_max = inv(P_MAX)
    pos = [inv(0.5 + half_span * (j / 8.0)) / z_max for j in range(1, 9)]
    neg = [-inv(0.5 + half_span * (j / 7.0)) / z_max for j in range(1, 8)]
    vals = sorted(neg + [0.0] + pos)
    return vals


def codebook(route: str = "wichura") -> np.ndarray:
    """The NF4 codebook as 16 fp32 values (fp64 construction, then RNE)."""
    return np.array(codebook_f64(route), dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# Sizes  [QLoRA-074, boxed note on the compression ratio]
# --------------------------------------------------------------------------

def sizes(n: int) -> tuple[int, int, int]:
    """Bytes of (codes, 8-bit scales, fp32 second-level scales) for n weights."""
    nb = -(-n // BLOCK)
    ng = -(-nb // GROUP)
    return 4 * (-(-n // 8)), nb, 4 * ng


# --------------------------------------------------------------------------
# Quantization  [QLoRA-074 §三 procedure: blockwise NF4 quantize with block
# 64, then quantize the first-level scales with block 256]
# --------------------------------------------------------------------------

def block_absmax(w: np.ndarray) -> np.ndarray:
    """c1_b = max |w_i| over the valid elements of each 64-block (fp32, exact)."""
    w = np.asarray(w, dtype=np.float32).ravel()
    nb = -(-w.size // BLOCK)
    padded = np.zeros(nb * BLOCK, dtype=np.float32)  # |0| never raises a max
    padded[: w.size] = np.abs(w)
    return padded.reshape(nb, BLOCK).max(axis=1)


def nf4_encode(w: np.ndarray, c1: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Index of the nearest codebook value to w/c1, ties to the lower index.

    Exact: w is closer to V[t+1] than to V[t] iff w > c1·(V[t]+V[t+1])/2, and
    every quantity here is exact in fp64 (the midpoint of two fp32 values
    needs at most 26 significant bits, its product with an fp32 c1 at most
    50).  So k = number of midpoints strictly below w/c1.  A block with
    c1 = 0 holds only zeros and gets the zero code 7.
    """
    w = np.asarray(w, dtype=np.float32).ravel()
    n = w.size
    nb = c1.size
    padded = np.zeros(nb * BLOCK, dtype=np.float64)
    padded[:n] = w
    blocks = padded.reshape(nb, BLOCK)
    Vd = V.astype(np.float64)
    mids = (Vd[:-1] + Vd[1:]) / 2.0                       # 15 midpoints
    thr = c1.astype(np.float64)[:, None] * mids[None, :]  # nb × 15, exact
    k = np.zeros((nb, BLOCK), dtype=np.int64)
    for t in range(15):
        k += blocks > thr[:, t : t + 1]
    k[c1 == 0, :] = 7
    return k.reshape(-1)[:n].astype(np.uint8)


def pack_nibbles(k: np.ndarray) -> np.ndarray:
    """4-bit codes -> bytes: per 8 codes one 32-bit word, byte j = k_j | k_{j+4} << 4."""
    k = np.asarray(k, dtype=np.uint8).ravel()
    pad = (-k.size) % 8
    if pad:
        k = np.concatenate([k, np.full(pad, 7, dtype=np.uint8)])
    g = k.reshape(-1, 8)
    return (g[:, :4] | (g[:, 4:] << 4)).astype(np.uint8).ravel()


def unpack_nibbles(codes: np.ndarray, n: int) -> np.ndarray:
    b = np.asarray(codes, dtype=np.uint8).reshape(-1, 4)
    k = np.concatenate([b & 0x0F, b >> 4], axis=1)
    return k.ravel()[:n]


def second_level_step(c1: np.ndarray) -> np.ndarray:
    """d_g = fl32(c2_g / 255) with c2_g = max of the group's first-level c1.

    The 8-bit scale code q means q·d_g, an unsigned linear code whose top
    level 255 lands on the group's largest constant.  The fp64 quotient of two
    fp32 numbers rounded again to fp32 is the correctly rounded fp32 quotient
    (53 ≥ 2·24 + 2 bits), so this is IEEE fp32 division.
    """
    nb = c1.size
    ng = -(-nb // GROUP)
    padded = np.zeros(ng * GROUP, dtype=np.float32)
    padded[:nb] = c1
    c2 = padded.reshape(ng, GROUP).max(axis=1)
    return (c2.astype(np.float64) / 255.0).astype(np.float32)


def scale_encode(c1: np.ndarray, step: np.ndarray) -> np.ndarray:
    """q8_b = the q in 0..255 minimising |q·d_g − c1_b|, ties to the lower q.

    Exact: q·d_g is nearer than (q+1)·d_g iff c1 ≤ (2q+1)·d_g/2, a product of
    a ≤ 9-bit integer and an fp32 number, exact in fp64.  So q8 counts the
    half-steps strictly below c1.  A group whose step is 0 gets q8 = 0.
    """
    c1d = c1.astype(np.float64)
    stepd = np.repeat(step.astype(np.float64), GROUP)[: c1.size]
    q = np.zeros(c1.size, dtype=np.int64)
    for j in range(255):
        q += c1d > (2 * j + 1) * stepd / 2.0
    q[stepd == 0.0] = 0
    return q.astype(np.uint8)


def quantize(w: np.ndarray, V: np.ndarray | None = None):
    """Blockwise NF4 + double quantization of a flat fp32 tensor.

    Returns (codes u8[ceil(n/2)], scale8 u8[nb], scale2 f32[ng]).  Following
    the procedure of [QLoRA-074 §三], the weights are encoded with the exact
    fp32 first-level constants; only afterwards are those constants
    themselves quantized to 8 bits with one fp32 step per 256 of them.
    """
    if V is None:
        V = codebook()
    w = np.asarray(w, dtype=np.float32).ravel()
    c1 = block_absmax(w)
    k = nf4_encode(w, c1, V)
    step = second_level_step(c1)
    q8 = scale_encode(c1, step)
    return pack_nibbles(k), q8, step


def quantize_chunked(w: np.ndarray, chunk: int = 1 << 20, V: np.ndarray | None = None):
    """Same result as quantize(), processed in whole 16384-weight groups."""
    if V is None:
        V = codebook()
    w = np.asarray(w, dtype=np.float32).ravel()
    gw = BLOCK * GROUP
    chunk = max(gw, (chunk // gw) * gw)
    parts = [quantize(w[i : i + chunk], V) for i in range(0, w.size, chunk)]
    return (np.concatenate([p[0] for p in parts]),
            np.concatenate([p[1] for p in parts]),
            np.concatenate([p[2] for p in parts]))


# --------------------------------------------------------------------------
# Dequantization  [QLoRA-074 §一: Ŵ = Dequant(W4bit, scales); §三: on demand,
# dequantize the required weights to BF16]
# --------------------------------------------------------------------------

def dequant_f32(codes: np.ndarray, scale8: np.ndarray, scale2: np.ndarray, n: int,
                V: np.ndarray | None = None) -> np.ndarray:
    """ŵ_i = fl32(V[k_i] · ĉ_b) with ĉ_b = fl32(q8_b · d_g): two fp32 products."""
    if V is None:
        V = codebook()
    k = unpack_nibbles(codes, n)
    b = np.arange(n) // BLOCK
    g = b // GROUP
    chat = scale8.astype(np.float32)[b] * scale2.astype(np.float32)[g]   # fp32 product
    return V.astype(np.float32)[k] * chat                                 # fp32 product


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns u16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_bf16_bits(codes, scale8, scale2, n, V=None) -> np.ndarray:
    """The bf16 operand of the linear layer: RNE_bf16(ŵ), as u16 bit patterns."""
    return bf16_rne_bits(dequant_f32(codes, scale8, scale2, n, V))
