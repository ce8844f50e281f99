"""Oracle: the AdamW update of the adapter parameters, in the kernels' fp32 steps.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[QLoRA-074 §三] updates only the LoRA parameters, with a paged optimizer;
[QLoRA-074 §二] and the weimeta glossary describe the paging: the optimizer
states (Adam's m and v) live in CPU memory and move to the GPU when an update
needs them.  The update itself is AdamW with decoupled weight decay
(Loshchilov and Hutter), the optimizer the pages' training configuration
names.  The pages fix neither the precision nor the order of operations;
reading: fp32 master parameters and fp32 states, a bf16 gradient, and per
element, with every operation rounded to fp32:

    m' = b1·m + c1·g                   c1 = 1 − b1
    v' = b2·v + c2·(g·g)               c2 = 1 − b2
    den = sqrt(v')·rs + eps            rs = 1 / sqrt(1 − b2^t)
    p' = p·keep − (lr1·m') / den       keep = 1 − lr·wd,  lr1 = lr / (1 − b1^t)

The per-step constants are computed in fp64 from the fp32 hyper-parameters
(b^t by t successive multiplications) and rounded once to fp32; sqrt and the
division are correctly rounded.  The bf16 copy of p' is its nearest-even
rounding.
"""

from __future__ import annotations

import math

import numpy as np

from . import nf4


def constants(lr, b1, b2, eps, wd, t):
    """fp32 (c1, c2, rs, keep, lr1, eps) for step t >= 1 from fp32 hyper-parameters."""
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    p1 = p2 = 1.0
    for _ in range(int(t)):
        p1 *= b1
        p2 *= b2
    f = lambda x: np.float32(x)            # noqa: E731  (one rounding of an fp64 value)
    return (f(1.0 - b1), f(1.0 - b2), f(1.0 / math.sqrt(1.0 - p2)), f(1.0 - lr * wd),
            f(lr / (1.0 - p1)), f(eps))


def step(p, g, m, v, t, lr=1e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """One AdamW step.  p, m, v fp32 arrays; g the bf16 gradient as float values.
    Returns (p', m', v', bf16 bits of p')."""
    p = np.asarray(p, np.float32)
    g = np.asarray(g, np.float32)
    m = np.asarray(m, np.float32)
    v = np.asarray(v, np.float32)
    c1, c2, rs, keep, lr1, e = constants(lr, b1, b2, eps, wd, t)
    f32 = np.float32
    m2 = f32(b1) * m + c1 * g
    v2 = f32(b2) * v + c2 * (g * g)
    den = np.sqrt(v2) * rs + e
    p2 = p * keep - (lr1 * m2) / den
    return p2, m2, v2, nf4.bf16_rne_bits(p2)


def step_fp64(p, g, m, v, t, lr=1e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """The textbook AdamW step in fp64 (for the pins, not for parity)."""
    p, g, m, v = (np.asarray(x, np.float64) for x in (p, g, m, v))
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    p = p * (1.0 - lr * wd)
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    mh = m / (1.0 - b1 ** t)
    vh = v / (1.0 - b2 ** t)
    return p - lr * mh / (np.sqrt(vh) + eps), m, v
