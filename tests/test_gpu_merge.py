"""GPU parity of the adapter merge and the re-quantization that follows.

The merged fp32 weight W' = fl32(ŵ + fl32(s·Δ)), Δ = A·B summed in fp32 in
increasing rank order, is compared bit for bit with oracle.merge, and with
the exact fp64 ŵ + s·(A·B)ᵀ within the rounding bound of such a sum, and so are
the codes and scales of quantizing it again (same fp32 input on both sides).
Shapes cover partial 128 × 128 tiles, ranks across the 64-wide rank chunks,
r = 0, and the full 4096 × 4096, r = 64 layer.
"""

import numpy as np
import pytest

import synth
from bounds import merge_bound
from gpu_util import bf16_dev, bf16_to_f64
from oracle import merge, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check(o, d, r, s, seed):
    W = synth.normal_f32((o, d), 0.02, [seed, 0, 0])
    A = synth.normal_bf16((d, r), 0.02, [seed, 0, 2])
    B = synth.normal_bf16((r, o), 0.02, [seed, 0, 3])
    c, s8, s2 = nf4.quantize_chunked(W.ravel())
    w_hat = nf4.dequant_f32(c, s8, s2, W.size).reshape(o, d)
    ref = merge.merge(w_hat, bf16_to_f64(A), bf16_to_f64(B), s)

    q = qb.qlora_quantize_nf4_dq(torch.from_numpy(W).cuda())
    got = qb.qlora_merge_adapter(q, bf16_dev(A) if r else None, bf16_dev(B) if r else None, s)
    q2 = qb.qlora_quantize_nf4_dq(got)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), \
        f"o={o} d={d} r={r}: {np.count_nonzero(g != ref)} merged weights differ"
    # the plain definition, independent of the order of the fp32 rank sum:
    # the exact ŵ + s·(A·B)ᵀ within the rounding bound of any such order
    bound, exact = merge_bound(w_hat, bf16_to_f64(A), bf16_to_f64(B), s, r)
    far = np.abs(g.astype(np.float64) - exact) > bound
    assert not far.any(), f"o={o} d={d} r={r}: {int(far.sum())} merged weights outside the bound"
    rc, rs8, rs2 = nf4.quantize_chunked(ref.ravel())
    n_c, n_s8, n_s2 = qb.qlora_quant_sizes(o * d)
    assert np.array_equal(q2.codes.cpu().numpy()[:n_c], rc)
    assert np.array_equal(q2.scale8.cpu().numpy()[:n_s8], rs8)
    assert np.array_equal(q2.scale2.cpu().numpy()[: n_s2 // 4].view(np.uint32), rs2.view(np.uint32))
    return q, q2


@pytest.mark.parametrize("o,d,r,s", [
    (136, 192, 8, 2.0),       # partial tiles in both directions
    (264, 640, 24, -0.5),
    (128, 128, 64, 2.0),      # exactly one rank chunk
    (256, 384, 136, 0.25),    # three rank chunks, the last partial
])
def test_merge_and_requantize_bit_exact(o, d, r, s):
    check(o, d, r, s, seed=o + d + r)


def test_rank_zero_is_the_dequantized_base():
    W = synth.normal_f32((64, 256), 0.02, [3, 0, 0])
    q = qb.qlora_quantize_nf4_dq(torch.from_numpy(W).cuda())
    got = qb.qlora_merge_adapter(q, None, None, 2.0)
    deq = qb.qlora_dequant(q, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), deq.view(torch.int32))


def test_full_4096_layer_rank_64():
    check(4096, 4096, 64, 2.0, seed=41)
