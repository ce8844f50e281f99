"""GPU parity of the other 4-bit tables (int4, FP4 E2M1, FP4 E3M0).

[QLoRA-074 §四, Table 2] compares NF4 with these formats under the same
blockwise scheme.  The library runs them through the same kernels as NF4
with another 16-entry table, so the same bar applies: codes, 8-bit scales,
fp32 steps and the dequantized weights bit-exact against oracle.formats;
the linear layer (fused GEMM path and few-token path) within the bf16
tolerance of gpu_util against the fp64 oracle on the format's Ŵ.
"""

import numpy as np
import pytest

import synth
from gpu_util import bf16_dev, bf16_host_f64, bf16_to_f64, check_close, grid_and_scale_blocks
from oracle import formats, linear, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")

OTHER = ("int4", "fp4_e2m1", "fp4_e3m0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_quantize(w: np.ndarray, fmt: str):
    W = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).ravel()).cuda()
    q = qb.qlora_quantize_nf4_dq(W, fmt=fmt)
    c, s8, s2 = qb.qlora_quant_sizes(w.size)
    torch.cuda.synchronize()
    return (q, q.codes.cpu().numpy()[:c], q.scale8.cpu().numpy()[:s8],
            q.scale2.cpu().numpy()[: s2 // 4])


def assert_exact(w: np.ndarray, fmt: str, what: str):
    q, c, s8, s2 = gpu_quantize(w, fmt)
    rc, rs8, rs2 = formats.quantize(w.ravel(), fmt)
    assert np.array_equal(s2.view(np.uint32), rs2.view(np.uint32)), f"{what}: scale2"
    assert np.array_equal(s8, rs8), f"{what}: scale8"
    assert np.array_equal(c, rc), f"{what}: codes ({np.count_nonzero(c != rc)} bytes differ)"
    ref = formats.dequant_f32(rc, rs8, rs2, w.size, fmt)
    got = qb.qlora_dequant(q, torch.float32).cpu().numpy().ravel()
    # bitwise, so the sign of the FP4 tables' −0 entries is checked too
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{what}: dequant f32"
    got16 = qb.qlora_dequant(q, torch.bfloat16).view(torch.int16).cpu().numpy().ravel()
    assert np.array_equal(got16.view(np.uint16), nf4.bf16_rne_bits(ref)), f"{what}: dequant bf16"
    return q


def _with_ties(fmt: str, seed: int) -> np.ndarray:
    """Gaussian blocks, signed zeros, and weights exactly on the table's
    midpoints (the ties go to the lower index; at the duplicated zero of the
    FP4 tables the sign decides)."""
    w = synth.normal_f32((64 * 40 + 17,), 0.02, [seed, 0, 0])
    w[5], w[6], w[64 * 7: 64 * 8] = 0.0, -0.0, 0.0          # one all-zero block
    V = formats.codebook(fmt).astype(np.float64)
    mids = (V[:-1] + V[1:]) / 2
    c1 = float(np.max(np.abs(w[64 * 3: 64 * 4])))
    for t, m in enumerate(mids):
        x = np.float32(m * c1)
        if abs(m) < 1 and float(x) == m * c1:           # (int4's lowest midpoint lies below -1)
            w[64 * 3 + 1 + t] = x
    w[64 * 9 + 2] = np.float32(1e-30)                        # both round to a zero entry
    w[64 * 9 + 3] = np.float32(-1e-30)
    return w


@pytest.mark.parametrize("fmt", OTHER)
def test_table_bytes_match_oracle(fmt):
    assert np.array_equal(np.array(qb.qlora_codebook(fmt), dtype=np.float32).view(np.uint32),
                          formats.codebook(fmt).view(np.uint32))


@pytest.mark.parametrize("fmt", OTHER)
@pytest.mark.parametrize("n", [1, 65, 16385, 3 * 16384 + 1037])
def test_ragged_exact(fmt, n):
    w = synth.normal_f32((n,), 0.02, [40 + n % 97, 0, 0])
    assert_exact(w, fmt, f"{fmt} n={n}")


@pytest.mark.parametrize("fmt", OTHER)
def test_ties_and_zeros_exact(fmt):
    assert_exact(_with_ties(fmt, 9), fmt, f"{fmt} ties")


@pytest.mark.parametrize("fmt", OTHER)
def test_grid_points_and_extreme_scales_exact(fmt):
    assert_exact(grid_and_scale_blocks(formats.codebook(fmt), 33), fmt, f"{fmt} grid")


@pytest.mark.parametrize("fmt", OTHER)
def test_4096_layer_exact(fmt):
    w = synth.normal_f32((4096, 4096), 0.02, [77, 0, 0])
    assert_exact(w, fmt, f"{fmt} 4096x4096")


def _parity(fmt, M, d, o, r, s, seed):
    W = synth.normal_f32((o, d), 0.02, [seed, 0, 0])
    X = synth.normal_bf16((M, d), 1.0, [seed, 0, 1])
    A = synth.normal_bf16((d, r), 0.02, [seed, 0, 2])
    B = synth.normal_bf16((r, o), 0.02, [seed, 0, 3])
    dY = synth.normal_bf16((M, o), 1.0, [seed, 0, 4])
    c, s8, s2 = formats.quantize(W.ravel(), fmt)
    Wh = nf4.bf16_bits_to_f64(nf4.dequant_bf16_bits(c, s8, s2, W.size,
                                                    formats.codebook(fmt))).reshape(o, d)
    Xf, Af, Bf, dYf = map(bf16_to_f64, (X, A, B, dY))
    Yr, Tr = linear.forward(Xf, Wh, Af, Bf, s)
    dXr, dAr, dBr = linear.backward(dYf, Xf, Wh, Af, Bf, s)

    q = qb.qlora_quantize_nf4_dq(torch.from_numpy(W).cuda(), fmt=fmt)
    Xd, Ad, Bd, dYd = bf16_dev(X), bf16_dev(A), bf16_dev(B), bf16_dev(dY)
    Y, T = qb.qlora_linear_fwd(Xd, q, Ad, Bd, s)
    dX, dA, dB = qb.qlora_linear_bwd(dYd, Xd, T, q, Ad, Bd, s)
    torch.cuda.synchronize()
    tag = f"{fmt} M={M} d={d} o={o} r={r}"
    check_close(bf16_host_f64(Y), Yr, "Y " + tag)
    check_close(T.cpu().numpy(), Tr, "T " + tag)
    check_close(bf16_host_f64(dX), dXr, "dX " + tag)
    check_close(bf16_host_f64(dA), dAr, "dA " + tag)
    check_close(bf16_host_f64(dB), dBr, "dB " + tag)


@pytest.mark.parametrize("fmt", OTHER)
def test_linear_gemm_path(fmt):
    _parity(fmt, 520, 640, 776, 16, 2.0, seed=61)       # several tiles, ragged in M and o


@pytest.mark.parametrize("fmt", OTHER)
def test_linear_few_token_path(fmt):
    _parity(fmt, 3, 192, 264, 16, 2.0, seed=62)         # the GEMV forward


def test_quantization_error_order_on_gpu():
    """The GPU-quantized weights give the same MSE ordering as the oracle:
    NF4 lowest on Gaussian weights, E3M0 highest."""
    w = synth.normal_f32((1 << 20,), 0.02, [12, 1, 0])
    Wd = torch.from_numpy(w).cuda()
    mse = {}
    for fmt in formats.FORMATS:
        q = qb.qlora_quantize_nf4_dq(Wd, fmt=fmt)
        mse[fmt] = float(((qb.qlora_dequant(q).double() - Wd.double()) ** 2).mean())
    assert mse["nf4"] < min(mse["int4"], mse["fp4_e2m1"], mse["fp4_e3m0"])
    assert mse["fp4_e3m0"] > max(mse["int4"], mse["fp4_e2m1"])
    for fmt in formats.FORMATS:
        assert mse[fmt] == pytest.approx(formats.quantization_mse(w, fmt), rel=1e-9)
