"""Seeded synthetic inputs for the QLoRA linear layer.

The one module that both the oracle's tests and the HIP path's tests and
benchmark draw from.  It holds none of the method's arithmetic: it only draws
Gaussian numbers and stores them as fp32 or bfloat16.

Recipe: numpy.random.default_rng([workload, projection, tensor]) with tensor
ids W = 0, X = 1, A = 2, B = 3, dY = 4; fp64 normal draws rounded to fp32,
and for bf16 tensors rounded once more (nearest-even) by torch's CPU cast.
Weights follow N(0, 0.02) (N(0, 0.015) at the 65B-style shapes), activations
and output gradients N(0, 1), LoRA factors N(0, 0.02), s = 2.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

T_W, T_X, T_A, T_B, T_DY = 0, 1, 2, 3, 4
T_A_STACK, T_B_STACK = 7, 8        # stacked adapters [n][d][r], [n][r][o] (one per token)


def normal_f32(shape, std: float, seed) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (u16) of fp32 data, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, std: float, seed) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(shape, std, seed))


@dataclass(frozen=True)
class Proj:
    name: str
    o: int
    d: int


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    projs: tuple
    M: int
    r: int
    w_std: float
    s: float = 2.0
    backward: bool = True


_H7, _F7, _H65, _F65 = 4096, 11008, 8192, 22016


def _block(h: int, f: int):
    return (Proj("q", h, h), Proj("k", h, h), Proj("v", h, h), Proj("o", h, h),
            Proj("gate", f, h), Proj("up", f, h), Proj("down", h, f))


WORKLOADS = {
    # 128×128 linear: 16384 weights = 256 blocks = one double-quant group.
    "tiny_128": Workload(0, "tiny_128", (Proj("w", 128, 128),), M=8, r=8, w_std=0.02),
    # One 4096×4096 linear, 4096 tokens (2 × 2048), rank 64.
    "linear_4096": Workload(1, "linear_4096", (Proj("w", 4096, 4096),), M=4096, r=64, w_std=0.02),
    # Decode shapes on 7B-style MLP weights, rank 16, forward only.
    "decode_mlp_7b": Workload(2, "decode_mlp_7b",
                              (Proj("gate", _F7, _H7), Proj("up", _F7, _H7), Proj("down", _H7, _F7)),
                              M=1, r=16, w_std=0.02, backward=False),
    # All 7 projections of a 7B-style block, 4096 tokens, rank 64.
    "block_7b": Workload(3, "block_7b", _block(_H7, _F7), M=4096, r=64, w_std=0.02),
    # All 7 projections of a 65B-style block, 2048 tokens, rank 64.
    "block_65b": Workload(4, "block_65b", _block(_H65, _F65), M=2048, r=64, w_std=0.015),
}

PROJ_IDS = {"w": 0, "q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


def layer_inputs(wl: Workload, proj: Proj, M: int | None = None):
    """Host inputs of one projection: W fp32 [o][d]; X, A, B, dY as bf16 bits."""
    M = wl.M if M is None else M
    pid = PROJ_IDS[proj.name]
    seed = lambda t: [wl.wid, pid, t]  # noqa: E731
    W = normal_f32((proj.o, proj.d), wl.w_std, seed(T_W))
    X = normal_bf16((M, proj.d), 1.0, seed(T_X))
    A = normal_bf16((proj.d, wl.r), 0.02, seed(T_A))
    B = normal_bf16((wl.r, proj.o), 0.02, seed(T_B))
    dY = normal_bf16((M, proj.o), 1.0, seed(T_DY))
    return W, X, A, B, dY
