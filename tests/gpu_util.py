"""Helpers of the GPU parity tests: device transfer and the tolerance rule."""

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
