"""Helpers of the GPU parity tests: device transfer, the tolerance rule and
adversarial weight blocks for the quantizer."""

from __future__ import annotations

import numpy as np

# Floating-point parity bar for the bf16 products (fp32 accumulation):
# relative Frobenius error and a per-element bound scaled by the result's rms.
REL_FRO = 5e-3
ELEM = 2e-2


def check_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    err = got - ref
    nref = np.linalg.norm(ref)
    rms = nref / np.sqrt(ref.size)
    if nref == 0:
        assert np.all(got == 0), f"{what}: expected exact zeros"
        return
    rel = np.linalg.norm(err) / nref
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    bound = ELEM * (np.abs(ref) + rms)
    bad = np.abs(err) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements outside |err| <= {ELEM}(|ref|+rms); "
                           f"worst at {np.unravel_index(np.argmax(np.abs(err) - bound), ref.shape)}")


def bf16_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def bf16_host_f64(t) -> np.ndarray:
    import torch
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (u << 16).view(np.float32).astype(np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def grid_and_scale_blocks(V, seed: int) -> np.ndarray:
    """Blocks of weights with w/c1 on a fine uniform grid ((j + 1/2)/128 for
    every j with the value in [-1, 1]) and one ulp either side, at
    power-of-two absmax (so the grid points are exact fp32 values); then
    blocks whose absmax sits at the edges of the fp32 range: FLT_MAX, 2^-100
    and its fp32 neighbours, small subnormals down to 2^-149.  V: the table,
    whose decision points are added too."""
    rng = np.random.default_rng(seed)
    V = np.asarray(V, dtype=np.float64)
    pts = [(j + 0.5) / 128 for j in range(-129, 129) if abs((j + 0.5) / 128) <= 1]
    pts += [float(m) for m in (V[:-1] + V[1:]) / 2 if abs(m) <= 1]
    blocks = []
    for e in (0, -7, -40, -110):
        c1 = np.float32(2.0 ** e)
        vals = []
        for x in pts:
            w = np.float32(x * float(c1))
            for u in (w, np.nextafter(w, np.float32(np.inf)), np.nextafter(w, np.float32(-np.inf))):
                if abs(float(u)) <= float(c1):
                    vals.append(u)
        vals = np.array(vals, dtype=np.float32)
        for i in range(0, vals.size, 63):
            blk = np.zeros(64, np.float32)
            blk[0] = c1 if (i // 63) % 2 else -c1
            part = vals[i:i + 63]
            blk[1:1 + part.size] = part
            blocks.append(blk)
    fmax = np.finfo(np.float32).max
    t = np.float32(2.0 ** -100)
    for c1 in (fmax, np.float32(2.0 ** 127), t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1)),
               np.float32(1e-40), np.float32(2.0 ** -149)):
        blk = (rng.uniform(-1, 1, 64) * float(c1)).astype(np.float32)
        blk[rng.integers(64)] = c1
        blocks.append(blk)
    return np.concatenate(blocks)
