"""Bit-exact parity of the dequantized weights the fused kernels consume.

The GEMM and GEMV kernels never write Ŵ to memory: each expands codes and
scales into bf16 operands on the fly ("074｜QLoRA：把大模型放进显存，再用小适配器
改变它" §一, Ŵ = Dequant(W4bit, scales); §三, dequantize the needed weights to
BF16 on demand).  One-hot activations read those operands back exactly:
with rank 0, a token row X[m] = e_k gives Y[m][n] = Ŵ[k][n] = Wq[n][k] (one
product 1·w, the rest 0·w', summed in fp32, then one bf16 rounding of a bf16
value), and an output-gradient row dY[m] = e_n gives dX[m][k] = Wq[n][k].
Every value is compared with the oracle's bf16 dequantization (values, so
+0 and −0 compare equal), for the four code tables:
  * k_qgemm forward with X = I_d and backward with dY = I_o (every weight),
    on the 4096×4096 layer and on a ragged 264×640 one;
  * k_gemv (M <= 16; the 1-, 2-, 4- and 16-token instances) with one-hot
    rows whose columns cover every position of a 64-weight block, several
    blocks and several double-quant groups, including the 7B-style
    11008×4096 gate weight.
"""

import numpy as np
import pytest

import synth
from gpu_util import bf16_to_f64
from oracle import formats, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_bf16(W, fmt):
    """Oracle bf16 Ŵ [o][d] as fp64 values, from its own quantization of W."""
    o, d = W.shape
    V = formats.codebook(fmt)
    c, s8, s2 = nf4.quantize_chunked(W.ravel(), V=V)
    return c, bf16_to_f64(nf4.dequant_bf16_bits(c, s8, s2, W.size, V)).reshape(o, d)


def _quantize(W, fmt, codes_ref):
    q = qb.qlora_quantize_nf4_dq(torch.from_numpy(W).cuda(), fmt=fmt)
    n_c = qb.qlora_quant_sizes(W.size)[0]
    assert np.array_equal(q.codes.cpu().numpy()[:n_c], codes_ref), f"{fmt}: codes differ"
    return q


def _vals(t):
    return t.float().cpu().numpy().astype(np.float64)


def _same(got, want, what):
    bad = got != want            # value comparison: +0 == -0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} dequantized values differ, "
                           f"first at {np.argwhere(bad)[0].tolist()}")


def _gemm_identity(W, fmt):
    o, d = W.shape
    codes, ref = _oracle_bf16(W, fmt)
    q = _quantize(W, fmt, codes)
    Xi = torch.eye(d, dtype=torch.bfloat16, device="cuda")
    Y, _ = qb.qlora_linear_fwd(Xi, q, None, None, 0.0, want_T=False)     # Y = Ŵ = Wqᵀ
    dYi = torch.eye(o, dtype=torch.bfloat16, device="cuda")
    dX, _, _ = qb.qlora_linear_bwd(dYi, None, None, q, None, None, 0.0)  # dX = Wq
    torch.cuda.synchronize()
    _same(_vals(Y), ref.T, f"k_qgemm forward {o}x{d} {fmt}")
    _same(_vals(dX), ref, f"k_qgemm backward {o}x{d} {fmt}")


@pytest.mark.parametrize("fmt", list(qb.FORMATS))
def test_gemm_ragged_identity_all_tables(fmt):
    W = synth.normal_f32((264, 640), 0.02, [501, 0, 0])
    _gemm_identity(W, fmt)


def test_gemm_linear_4096_identity():
    wl = synth.WORKLOADS["linear_4096"]
    W = synth.layer_inputs(wl, wl.projs[0], M=1)[0]
    _gemm_identity(W, "nf4")


def _one_hot(cols, d):
    X = torch.zeros((len(cols), d), dtype=torch.bfloat16)
    X[torch.arange(len(cols)), torch.tensor(cols)] = 1.0
    return X.cuda()


def _gemv_columns(W, fmt, M, cols):
    """Y rows of one-hot tokens through the few-token kernel, M at a time."""
    o, d = W.shape
    codes, ref = _oracle_bf16(W, fmt)
    q = _quantize(W, fmt, codes)
    for i in range(0, len(cols), M):
        cs = cols[i:i + M]
        Y, _ = qb.qlora_linear_fwd(_one_hot(cs, d), q, None, None, 0.0, want_T=False)
        torch.cuda.synchronize()
        _same(_vals(Y), ref[:, cs].T, f"k_gemv {o}x{d} {fmt} M={len(cs)} columns {cs}")


@pytest.mark.parametrize("fmt", list(qb.FORMATS))
@pytest.mark.parametrize("M", [1, 2, 4, 16])
def test_gemv_one_hot_every_block_position(fmt, M):
    # d = 640: 10 blocks per row; 264 rows: 165 groups, ragged output tile
    W = synth.normal_f32((264, 640), 0.02, [502, M, 0])
    # positions 0..63 of a block, spread over the 10 blocks of a row
    cols = [64 * ((7 * j) % 10) + j for j in range(64)]
    if M < 16:
        cols = cols[: 8 * M]       # fewer launches for the small instances
    _gemv_columns(W, fmt, M, cols)


def test_gemv_decode_gate_weight_one_hot():
    wl = synth.WORKLOADS["decode_mlp_7b"]
    p = next(x for x in wl.projs if x.name == "gate")
    W = synth.normal_f32((p.o, p.d), wl.w_std, [wl.wid, synth.PROJ_IDS[p.name], synth.T_W])
    cols = [0, 1, 63, 64, 511, 512, 1000, 1023, 1024, 2047, 2048, 2989, 3071, 4032, 4094, 4095]
    _gemv_columns(W, "nf4", 16, cols)
    _gemv_columns(W, "nf4", 13, cols[:13])
    _gemv_columns(W, "nf4", 1, cols[::5])


def test_gemv_decode_down_weight_one_hot():
    """The down projection (d = 11008: 172 blocks per row, 43 groups of four):
    one-hot columns at the first, last and group-boundary positions."""
    wl = synth.WORKLOADS["decode_mlp_7b"]
    p = next(x for x in wl.projs if x.name == "down")
    W = synth.normal_f32((p.o, p.d), wl.w_std, [wl.wid, synth.PROJ_IDS[p.name], synth.T_W])
    cols = [0, 63, 4095, 4096, 4159, 8191, 8192, 8255, 10943, 10944, 11007]
    _gemv_columns(W, "nf4", 1, cols)
