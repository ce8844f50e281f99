"""Python binding of libqlora.so, the MI355X (gfx950) QLoRA NF4 + double-quant layer.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/qlora.h.  PyTorch provides device memory
and the current HIP stream.  There is no CPU fallback: if the library is not
built, or a tensor is not on a HIP device, the calls raise.

Functions carry the C names:
  qlora_quant_sizes, qlora_codebook, qlora_workspace_bytes,
  qlora_quantize_nf4_dq, qlora_dequant, qlora_linear_fwd, qlora_linear_bwd,
  qlora_linear_bwd_noalloc, qlora_linear_fwd_multi, qlora_merge_adapter, qlora_adamw_step,
  qlora_paged_adamw_step.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlora.so")

QLORA_OK, QLORA_E_NONFINITE, QLORA_E_SCRATCH = 0, 7, 8
QLORA_NOALLOC_SCRATCH_BYTES = 64 << 20
QLORA_F32, QLORA_BF16 = 0, 1
QLORA_OP_FWD, QLORA_OP_BWD = 0, 1
QLORA_BLOCK, QLORA_GROUP = 64, 256     # weights per block, blocks per double-quant group
# Tables of the 4-bit codes (qlora_fmt) and codes of the constants (qlora_dq).
FORMATS = {"nf4": 0, "int4": 1, "fp4_e2m1": 2, "fp4_e3m0": 3}
DQ_VARIANTS = {"uint8": 0, "int8_mean": 1, "fp8_mean": 2}

_lib = None


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class _AdamW(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64)]


class _NF4DQ(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale8", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("n", ctypes.c_int64), ("fmt", ctypes.c_int32),
                ("dq", ctypes.c_int32)]


def lib() -> ctypes.CDLL:
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c "
                           f"'import __graft_entry__ as g; g.build()'` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, sz, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER
    L.qlora_quant_sizes.argtypes = [i64, P(i64), P(i64), P(i64)]
    L.qlora_codebook.argtypes = [i32, P(ctypes.c_float)]
    L.qlora_workspace_bytes.argtypes = [i32, i64, i64, i64, i64]
    L.qlora_workspace_bytes.restype = sz
    L.qlora_strerror.argtypes = [i32]
    L.qlora_strerror.restype = ctypes.c_char_p
    L.qlora_version.restype = ctypes.c_char_p
    L.qlora_quantize_nf4_dq.argtypes = [vp, i64, P(_NF4DQ), vp, vp]
    L.qlora_quantize_nf4_dq_ws.argtypes = [vp, i64, P(_NF4DQ), vp, vp, sz, vp]
    L.qlora_quantize_nf4_dq_grouped.argtypes = [P(vp), P(_NF4DQ), i32, vp, vp]
    L.qlora_quant_sizes_dq.argtypes = [i64, i32, P(i64), P(i64), P(i64), P(i64)]
    L.qlora_dequant.argtypes = [P(_NF4DQ), i32, vp, vp]
    L.qlora_linear_fwd.argtypes = [vp, i64, i64, P(_NF4DQ), i64, vp, vp, i64, ctypes.c_float,
                                   vp, vp, vp, sz, vp]
    L.qlora_linear_bwd.argtypes = [vp, vp, vp, i64, i64, P(_NF4DQ), i64, vp, vp, i64,
                                   ctypes.c_float, vp, vp, vp, vp, sz, vp]
    L.qlora_linear_bwd_noalloc.argtypes = [vp, vp, vp, i64, i64, P(_NF4DQ), i64, vp, vp, i64,
                                           ctypes.c_float, vp, vp, vp, vp]
    L.qlora_adamw_step.argtypes = [vp, vp, vp, vp, vp, i64, P(_AdamW), vp]
    L.qlora_paged_adamw_step.argtypes = [vp, vp, vp, vp, vp, i64, P(_AdamW), vp, sz, vp]
    L.qlora_merge_adapter.argtypes = [P(_NF4DQ), i64, i64, vp, vp, i64, ctypes.c_float, vp, vp]
    L.qlora_linear_fwd_multi.argtypes = [vp, i64, i64, P(_NF4DQ), i64, vp, vp, i64, i64,
                                         P(ctypes.c_float), vp, vp, vp, vp, sz, vp]
    L.qlora_timing_begin.argtypes = [ctypes.c_uint32]
    L.qlora_timing_read.argtypes = [i32, P(ctypes.c_double), P(i64)]
    for name in ("qlora_quant_sizes", "qlora_quant_sizes_dq", "qlora_quantize_nf4_dq_ws",
                 "qlora_codebook", "qlora_quantize_nf4_dq", "qlora_quantize_nf4_dq_grouped",
                 "qlora_dequant",
                 "qlora_linear_fwd", "qlora_linear_bwd", "qlora_linear_bwd_noalloc",
                 "qlora_linear_fwd_multi",
                 "qlora_merge_adapter", "qlora_adamw_step", "qlora_paged_adamw_step",
                 "qlora_timing_begin", "qlora_timing_end",
                 "qlora_timing_read"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().qlora_strerror(int(status)).decode()


def _check(status: int, where: str):
    if status != QLORA_OK:
        raise QloraError(status, where)


# ------------------------------------------------------------------ host helpers

def qlora_quant_sizes_dq(n: int, dq="uint8") -> tuple[int, int, int, int]:
    """(codes, scale8, scale2, workspace) bytes for a second-level variant."""
    c, s8, s2, w = (ctypes.c_int64() for _ in range(4))
    code = DQ_VARIANTS[dq] if isinstance(dq, str) else int(dq)
    _check(lib().qlora_quant_sizes_dq(n, code, ctypes.byref(c), ctypes.byref(s8), ctypes.byref(s2),
                                      ctypes.byref(w)), "qlora_quant_sizes_dq")
    return c.value, s8.value, s2.value, w.value


def qlora_quant_sizes(n: int) -> tuple[int, int, int]:
    c, s8, s2 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().qlora_quant_sizes(n, ctypes.byref(c), ctypes.byref(s8), ctypes.byref(s2)),
           "qlora_quant_sizes")
    return c.value, s8.value, s2.value


def _fmt_code(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown 4-bit format {fmt!r}; one of {sorted(FORMATS)}")
        return FORMATS[fmt]
    return int(fmt)


def qlora_codebook(fmt="nf4") -> list[float]:
    """The 16 ascending values of a code table ("nf4", "int4", "fp4_e2m1", "fp4_e3m0")."""
    buf = (ctypes.c_float * 16)()
    _check(lib().qlora_codebook(_fmt_code(fmt), buf), "qlora_codebook")
    return list(buf)


def qlora_workspace_bytes(op: int, M: int, d: int, o: int, r: int) -> int:
    return int(lib().qlora_workspace_bytes(op, M, d, o, r))


# Kernel classes of the launch-timing diagnostics (qlora_kernel_class).
K_MAIN_GEMM, K_QUANTIZE, K_GEMV, K_DEQUANT, K_ADAPTER, K_GRADS = range(6)
KERNEL_CLASSES = {"main_gemm": K_MAIN_GEMM, "quantize": K_QUANTIZE, "gemv": K_GEMV,
                  "dequant": K_DEQUANT, "adapter": K_ADAPTER, "grads": K_GRADS}


def qlora_timing_begin(classes=None):
    """Start recording launch events for the given kernel classes (default: all)."""
    mask = 0xFFFFFFFF if classes is None else sum(1 << c for c in classes)
    _check(lib().qlora_timing_begin(mask), "qlora_timing_begin")


def qlora_timing_end():
    _check(lib().qlora_timing_end(), "qlora_timing_end")


def qlora_timing_read(kernel_class: int) -> tuple[float, int]:
    """(summed milliseconds, launches) of one kernel class since qlora_timing_begin()."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().qlora_timing_read(kernel_class, ctypes.byref(ms), ctypes.byref(n)),
           "qlora_timing_read")
    return ms.value, n.value


# ------------------------------------------------------------------ device calls

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, device=None):
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a HIP device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _tensor(t, name):
    torch = _torch()
    if t is not None and not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")


def _shape(t, shape, name):
    """ValueError unless tensor t (if given) has exactly `shape`.  Checked
    before anything reaches the library: the C ABI receives sizes only, so a
    mis-shaped buffer would otherwise be read or written past its end."""
    if t is None:
        return
    _tensor(t, name)
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _numel(t, n, name):
    if t is None:
        return
    _tensor(t, name)
    if t.numel() != n:
        raise ValueError(f"{name} holds {t.numel()} elements, expected {n}")


def _linear_dims(q, name="q"):
    shape = getattr(q, "shape", None)
    if shape is None or len(shape) != 2 or int(shape[0]) * int(shape[1]) != q.n:
        raise ValueError(f"{name} must be a quantized 2-D weight [o][d]")
    q.check_buffers()
    return int(shape[0]), int(shape[1])


@dataclass
class QuantizedWeight:
    """Device buffers of a quantized tensor: codes, 8-bit scales, fp32 steps."""
    codes: object
    scale8: object
    scale2: object
    n: int
    shape: tuple
    fmt: int = 0
    dq: int = 0

    def view(self) -> _NF4DQ:
        self.check_buffers()
        return _NF4DQ(self.codes.data_ptr(), self.scale8.data_ptr(), self.scale2.data_ptr(), self.n,
                      self.fmt, self.dq)

    def check_buffers(self):
        """ValueError unless every buffer holds at least the bytes the layout
        of n weights needs (4 bits per weight, one byte per 64, one fp32 per
        16384, plus the mean for the centred second levels)."""
        n = int(self.n)
        nb = -(-n // QLORA_BLOCK)
        need = {"codes": 4 * -(-n // 8), "scale8": nb,
                "scale2": 4 * -(-nb // QLORA_GROUP) + (4 if self.dq and n > 0 else 0)}
        for name, nbytes in need.items():
            t = getattr(self, name)
            have = t.numel() * t.element_size()
            if have < nbytes:
                raise ValueError(f"quantized {name} holds {have} bytes, {nbytes} needed for n={n}")

    @property
    def device(self):
        return self.codes.device


def _alloc_quantized(n: int, shape, device, fmt: int, dq: int = 0) -> QuantizedWeight:
    torch = _torch()
    c, s8, s2, _ = qlora_quant_sizes_dq(n, dq)
    return QuantizedWeight(torch.empty(max(c, 1), dtype=torch.uint8, device=device),
                           torch.empty(max(s8, 1), dtype=torch.uint8, device=device),
                           torch.empty(max(s2 // 4, 1), dtype=torch.float32, device=device),
                           n, tuple(shape), fmt, dq)


def qlora_quantize_nf4_dq(W, check_finite: bool = True, out: QuantizedWeight | None = None,
                          fmt="nf4", dq="uint8") -> QuantizedWeight:
    """Blockwise 4-bit + double quantization of an fp32 device tensor (any shape, flattened).

    `fmt` picks the code table (NF4 by default) and `dq` the code of the
    constants ("uint8" by default, or "int8_mean" / "fp8_mean", which run the
    workspace quantizer).  `out` reuses the buffers of an earlier result of
    the same size (and keeps its table and variant).  With check_finite the
    call waits for the kernel and raises on NaN/Inf input.
    """
    torch = _torch()
    _need(W, torch.float32, "W")
    _tensor(W, "W")
    if out is not None and out.n != W.numel():
        raise ValueError("out holds a different number of weights")
    dq_code = DQ_VARIANTS[dq] if isinstance(dq, str) else int(dq)
    q = _alloc_quantized(W.numel(), W.shape, W.device, _fmt_code(fmt), dq_code) if out is None else out
    flags = getattr(q, "flags", None)
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=W.device)
    elif check_finite:
        flags.zero_()
    if q.dq == 0:
        _check(lib().qlora_quantize_nf4_dq(_ptr(W), W.numel(), ctypes.byref(q.view()), _ptr(flags),
                                           _stream(W.device)), "qlora_quantize_nf4_dq")
    else:
        nws = qlora_quant_sizes_dq(W.numel(), q.dq)[3]
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=W.device)
        _check(lib().qlora_quantize_nf4_dq_ws(_ptr(W), W.numel(), ctypes.byref(q.view()), _ptr(flags),
                                              _ptr(ws), ws.numel(), _stream(W.device)),
               "qlora_quantize_nf4_dq_ws")
    if check_finite and int(flags.item()) & 1:
        raise QloraError(QLORA_E_NONFINITE, "qlora_quantize_nf4_dq")
    q.flags = flags
    return q


QLORA_MAX_GROUPED = 16


def qlora_quantize_nf4_dq_grouped(Ws, check_finite: bool = True, outs=None,
                                  fmt="nf4") -> list:
    """Blockwise 4-bit + double quantization of several fp32 device tensors
    (one table, the default code of the constants) in one launch; the result
    for each equals qlora_quantize_nf4_dq of that tensor.  `outs` reuses
    earlier results of the same sizes.  With check_finite the call waits and
    raises on NaN/Inf in any input."""
    torch = _torch()
    Ws = list(Ws)
    if len(Ws) > QLORA_MAX_GROUPED:
        raise ValueError(f"at most {QLORA_MAX_GROUPED} tensors per grouped call")
    if outs is not None and len(outs) != len(Ws):
        raise ValueError("outs must match Ws one to one")
    if not Ws:
        return []
    dev = Ws[0].device
    qs = []
    for k, W in enumerate(Ws):
        _need(W, torch.float32, f"Ws[{k}]", dev)
        _tensor(W, f"Ws[{k}]")
        if outs is None:
            qs.append(_alloc_quantized(W.numel(), W.shape, W.device, _fmt_code(fmt)))
        else:
            o = outs[k]
            if o.n != W.numel():
                raise ValueError(f"outs[{k}] holds a different number of weights")
            if o.dq != 0:
                raise ValueError("the grouped quantizer writes the default code of the constants")
            qs.append(o)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    views = (_NF4DQ * len(qs))(*[q.view() for q in qs])
    ptrs = (ctypes.c_void_p * len(Ws))(*[_ptr(W) for W in Ws])
    _check(lib().qlora_quantize_nf4_dq_grouped(ptrs, views, len(Ws), _ptr(flags), _stream(dev)),
           "qlora_quantize_nf4_dq_grouped")
    if check_finite and int(flags.item()) & 1:
        raise QloraError(QLORA_E_NONFINITE, "qlora_quantize_nf4_dq_grouped")
    for q in qs:
        q.flags = flags
    return qs


def qlora_stack_rows(parts) -> QuantizedWeight:
    """Quantized weights of one row length stacked by rows into one quantized
    tensor, e.g. projections that read the same input run as one layer.  The
    result is exactly what quantizing the stacked fp32 rows gives, which holds
    when every part covers whole double-quant groups (16384 weights), so that
    no group spans two parts; other parts raise ValueError.  Buffer copies only."""
    torch = _torch()
    parts = list(parts)
    if not parts:
        raise ValueError("no parts")
    d = parts[0].shape[-1]
    for q in parts:
        if q.n % (QLORA_BLOCK * QLORA_GROUP) != 0:
            raise ValueError("each part must hold whole double-quant groups (16384 weights)")
        if q.shape[-1] != d or q.fmt != parts[0].fmt or q.dq != 0 or parts[0].dq != 0:
            raise ValueError("parts need one row length, one code table and the default second level")
    sizes = [qlora_quant_sizes(q.n) for q in parts]
    codes = torch.cat([q.codes[:c] for q, (c, _, _) in zip(parts, sizes)])
    scale8 = torch.cat([q.scale8[:s8] for q, (_, s8, _) in zip(parts, sizes)])
    scale2 = torch.cat([q.scale2[:s2 // 4] for q, (_, _, s2) in zip(parts, sizes)])
    rows = sum(q.n // d for q in parts)
    return QuantizedWeight(codes, scale8, scale2, sum(q.n for q in parts), (rows, d), parts[0].fmt, 0)


def qlora_dequant(q: QuantizedWeight, dtype=None):
    """Ŵ as fp32 (default) or bf16, shaped like the original tensor."""
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    code = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}[dtype]
    out = torch.empty(q.shape, dtype=dtype, device=q.device)
    _check(lib().qlora_dequant(ctypes.byref(q.view()), code, _ptr(out), _stream(q.device)),
           "qlora_dequant")
    return out


class Workspace:
    """Grow-only device scratch buffer reused across calls on one stream.

    Calls that share a Workspace must be ordered (one stream, or streams
    synchronised by the caller): a later call may overwrite, or regrow and
    free, the buffer while an earlier call's kernels still use it.  The
    default workspaces are kept per (device, stream) for that reason."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, device):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws: dict = {}


def _workspace(ws, device, nbytes):
    if ws is None:
        torch = _torch()
        key = (str(device), torch.cuda.current_stream(device).cuda_stream)
        ws = _default_ws.setdefault(key, Workspace())
    return ws.get(nbytes, device)


def qlora_linear_fwd(X, q: QuantizedWeight, A, B, s: float, want_T: bool = True, ws=None,
                     out=None):
    """Y = X·Ŵ + s·(X·A)·B.  X bf16 [M][d]; q of Wq [o][d]; A bf16 [d][r]; B bf16 [r][o].

    Returns (Y, T) with T = X·A in fp32 (None if want_T is False or r == 0).
    """
    torch = _torch()
    o, d = _linear_dims(q)
    _tensor(X, "X")
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M][d], got shape {tuple(X.shape)}")
    M = X.shape[0]
    _shape(X, (M, d), "X")
    if (A is None) != (B is None):
        raise ValueError("A and B are given together or not at all")
    _tensor(A, "A")
    r = 0 if A is None else (A.shape[1] if A.dim() == 2 else -1)
    _shape(A, (d, r), "A")
    _shape(B, (r, o), "B")
    _shape(out, (M, o), "out")
    for t, nm in ((X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm, X.device)
    Y = torch.empty((M, o), dtype=torch.bfloat16, device=X.device) if out is None else out
    _need(Y, torch.bfloat16, "Y", X.device)
    T = torch.empty((M, r), dtype=torch.float32, device=X.device) if (want_T and r > 0) else None
    nbytes = qlora_workspace_bytes(QLORA_OP_FWD, M, d, o, r)
    buf = _workspace(ws, X.device, nbytes)
    _check(lib().qlora_linear_fwd(_ptr(X), M, d, ctypes.byref(q.view()), o, _ptr(A), _ptr(B), r,
                                  float(s), _ptr(Y), _ptr(T), _ptr(buf), buf.numel(),
                                  _stream(X.device)), "qlora_linear_fwd")
    return Y, T


def qlora_linear_bwd(dY, X, T, q: QuantizedWeight, A, B, s: float, need_dX: bool = True,
                     ws=None):
    """(dX, dA, dB) of the layer; no gradient for the 4-bit weight.  T may be None."""
    torch = _torch()
    o, d = _linear_dims(q)
    _tensor(dY, "dY")
    if dY.dim() != 2:
        raise ValueError(f"dY must be 2-D [M][o], got shape {tuple(dY.shape)}")
    M = dY.shape[0]
    _shape(dY, (M, o), "dY")
    if (A is None) != (B is None):
        raise ValueError("A and B are given together or not at all")
    _tensor(A, "A")
    r = 0 if A is None else (A.shape[1] if A.dim() == 2 else -1)
    _shape(A, (d, r), "A")
    _shape(B, (r, o), "B")
    _shape(X, (M, d), "X")
    _shape(T, (M, r), "T")
    for t, nm in ((dY, "dY"), (X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm, dY.device)
    _need(T, torch.float32, "T", dY.device)
    dev = dY.device
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=dev) if need_dX else None
    dA = torch.empty((d, r), dtype=torch.bfloat16, device=dev) if r > 0 else None
    dB = torch.empty((r, o), dtype=torch.bfloat16, device=dev) if r > 0 else None
    nbytes = qlora_workspace_bytes(QLORA_OP_BWD, M, d, o, r)
    buf = _workspace(ws, dev, nbytes)
    _check(lib().qlora_linear_bwd(_ptr(dY), _ptr(X), _ptr(T), M, d, ctypes.byref(q.view()), o,
                                  _ptr(A), _ptr(B), r, float(s), _ptr(dX), _ptr(dA), _ptr(dB),
                                  _ptr(buf), buf.numel(), _stream(dev)), "qlora_linear_bwd")
    return dX, dA, dB


def qlora_linear_bwd_noalloc(dY, X, T, q: QuantizedWeight, A, B, s: float, dX, dA, dB):
    """qlora_linear_bwd into caller-given outputs (dX may be None; dA, dB
    None only with r == 0), with the library's static device scratch instead
    of a workspace: nothing is allocated, in this function or the library.
    Calls that overlap on one GPU race on that scratch."""
    o, d = _linear_dims(q)
    _tensor(dY, "dY")
    if dY.dim() != 2:
        raise ValueError(f"dY must be 2-D [M][o], got shape {tuple(dY.shape)}")
    M = dY.shape[0]
    _shape(dY, (M, o), "dY")
    if (A is None) != (B is None):
        raise ValueError("A and B are given together or not at all")
    _tensor(A, "A")
    r = 0 if A is None else (A.shape[1] if A.dim() == 2 else -1)
    _shape(A, (d, r), "A")
    _shape(B, (r, o), "B")
    _shape(X, (M, d), "X")
    _shape(T, (M, r), "T")
    _shape(dX, (M, d), "dX")
    _shape(dA, (d, r), "dA")
    _shape(dB, (r, o), "dB")
    if r > 0 and (dA is None or dB is None):
        raise ValueError("dA and dB are required when r > 0")
    torch = _torch()
    dev = dY.device
    for t, nm in ((dY, "dY"), (X, "X"), (A, "A"), (B, "B"), (dX, "dX"), (dA, "dA"), (dB, "dB")):
        _need(t, torch.bfloat16, nm, dev)
    _need(T, torch.float32, "T", dev)
    _check(lib().qlora_linear_bwd_noalloc(_ptr(dY), _ptr(X), _ptr(T), M, d, ctypes.byref(q.view()), o,
                                          _ptr(A), _ptr(B), r, float(s), _ptr(dX), _ptr(dA),
                                          _ptr(dB), _stream(dev)), "qlora_linear_bwd_noalloc")
    return dX, dA, dB


def qlora_linear_fwd_multi(X, q: QuantizedWeight, A, B, s, adapter, want_T: bool = False,
                           ws=None, out=None):
    """Few-token forward with one adapter per token over one shared base.

    X bf16 [M][d] (M <= 16); A bf16 [n][d][r]; B bf16 [n][r][o]; s: n floats;
    adapter: int32 device tensor [M], an index outside [0, n) selecting the
    base alone.  Returns (Y, T) with T = X[m]·A[adapter[m]] in fp32 (or None).
    """
    torch = _torch()
    o, d = _linear_dims(q)
    _tensor(X, "X")
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M][d], got shape {tuple(X.shape)}")
    M = X.shape[0]
    _shape(X, (M, d), "X")
    _tensor(A, "A")
    if A is None or B is None or A.dim() != 3:
        raise ValueError("A must be [n][d][r] and B [n][r][o]")
    n, r = A.shape[0], A.shape[2]
    _shape(A, (n, d, r), "A")
    _shape(B, (n, r, o), "B")
    _shape(adapter, (M,), "adapter")
    _shape(out, (M, o), "out")
    for t, nm in ((X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm, X.device)
    _need(adapter, torch.int32, "adapter", X.device)
    svals = [float(v) for v in s]
    if len(svals) != n:
        raise ValueError("s must hold one scale per adapter")
    Y = torch.empty((M, o), dtype=torch.bfloat16, device=X.device) if out is None else out
    _need(Y, torch.bfloat16, "Y", X.device)
    T = torch.empty((M, r), dtype=torch.float32, device=X.device) if want_T else None
    nbytes = qlora_workspace_bytes(QLORA_OP_FWD, M, d, o, r)
    buf = _workspace(ws, X.device, nbytes)
    s_arr = (ctypes.c_float * n)(*svals)
    _check(lib().qlora_linear_fwd_multi(_ptr(X), M, d, ctypes.byref(q.view()), o, _ptr(A), _ptr(B),
                                        n, r, s_arr, _ptr(adapter), _ptr(Y), _ptr(T), _ptr(buf),
                                        buf.numel(), _stream(X.device)), "qlora_linear_fwd_multi")
    return Y, T


def qlora_merge_adapter(q: QuantizedWeight, A, B, s: float, out=None):
    """fp32 [o][d] merged weight ŵ + s·(A·B)ᵀ, ready for qlora_quantize_nf4_dq."""
    torch = _torch()
    o, d = _linear_dims(q)
    if (A is None) != (B is None):
        raise ValueError("A and B are given together or not at all")
    _tensor(A, "A")
    r = 0 if A is None else (A.shape[1] if A.dim() == 2 else -1)
    _shape(A, (d, r), "A")
    _shape(B, (r, o), "B")
    _shape(out, (o, d), "out")
    for t, nm in ((A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm, q.device)
    W = torch.empty((o, d), dtype=torch.float32, device=q.device) if out is None else out
    _need(W, torch.float32, "out", q.device)
    _check(lib().qlora_merge_adapter(ctypes.byref(q.view()), o, d, _ptr(A), _ptr(B), r, float(s),
                                     _ptr(W), _stream(q.device)), "qlora_merge_adapter")
    return W


def _adamw(step, lr, beta1, beta2, eps, weight_decay):
    return _AdamW(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))


def qlora_adamw_step(p, p16, g, m, v, step, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.0):
    """AdamW on device tensors: p, m, v fp32 (in place), g bf16, p16 bf16 or None."""
    torch = _torch()
    _tensor(p, "p")
    n = p.numel()
    for t, nm in ((m, "m"), (v, "v"), (g, "g"), (p16, "p16")):
        _numel(t, n, nm)
    if m is None or v is None or g is None:
        raise ValueError("m, v and g are required")
    _need(p, torch.float32, "p")
    for t, nm, dt in ((m, "m", torch.float32), (v, "v", torch.float32), (g, "g", torch.bfloat16),
                      (p16, "p16", torch.bfloat16)):
        _need(t, dt, nm, p.device)
    h = _adamw(step, lr, beta1, beta2, eps, weight_decay)
    _check(lib().qlora_adamw_step(_ptr(p), _ptr(p16), _ptr(g), _ptr(m), _ptr(v), n, ctypes.byref(h),
                                  _stream(p.device)), "qlora_adamw_step")


def pinned_state(n, device=None):
    """A pinned host fp32 buffer for the paged optimizer states (zeros)."""
    torch = _torch()
    return torch.zeros(n, dtype=torch.float32, pin_memory=True)


def qlora_paged_adamw_step(p, p16, g, m_host, v_host, step, pool, lr=1e-4, beta1=0.9,
                           beta2=0.999, eps=1e-8, weight_decay=0.0):
    """AdamW with the states in pinned host tensors, paged through `pool` (a
    device uint8 tensor of at least 4096 bytes)."""
    torch = _torch()
    _tensor(p, "p")
    for t, nm in ((g, "g"), (p16, "p16"), (m_host, "m_host"), (v_host, "v_host")):
        _numel(t, p.numel(), nm)
    if g is None or m_host is None or v_host is None or pool is None:
        raise ValueError("g, m_host, v_host and pool are required")
    _need(p, torch.float32, "p")
    for t, nm, dt in ((g, "g", torch.bfloat16), (p16, "p16", torch.bfloat16),
                      (pool, "pool", torch.uint8)):
        _need(t, dt, nm, p.device)
    for t, nm in ((m_host, "m_host"), (v_host, "v_host")):
        if t.device.type != "cpu" or not t.is_pinned() or t.dtype != torch.float32:
            raise TypeError(f"{nm} must be a pinned host fp32 tensor")
    n = p.numel()
    h = _adamw(step, lr, beta1, beta2, eps, weight_decay)
    _check(lib().qlora_paged_adamw_step(_ptr(p), _ptr(p16), _ptr(g), _ptr(m_host), _ptr(v_host), n,
                                        ctypes.byref(h), _ptr(pool), pool.numel(), _stream(p.device)),
           "qlora_paged_adamw_step")
