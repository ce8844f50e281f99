"""GPU parity of the second-level variants centred on the tensor mean
(int8 and FP8 E4M3 codes of the constants): codes, scale8, scale2 (with the
mean) and the dequantized weights bit for bit against oracle.dq, on ragged
lengths, zero groups, an all-zero tensor and the 4096 x 4096 weight."""

import numpy as np
import pytest

import synth
from oracle import dq, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")

VARIANTS = ("int8_mean", "fp8_mean")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check(w, variant, what):
    W = torch.from_numpy(np.ascontiguousarray(w, np.float32).ravel()).cuda()
    q = qb.qlora_quantize_nf4_dq(W, dq=variant)
    c, s8, s2, _ = qb.qlora_quant_sizes_dq(w.size, variant)
    torch.cuda.synchronize()
    gc, g8, g2 = q.codes.cpu().numpy()[:c], q.scale8.cpu().numpy()[:s8], q.scale2.cpu().numpy()[: s2 // 4]
    rc, r8, r2 = dq.quantize(w.ravel(), variant)
    assert np.array_equal(gc, rc), what + ": codes"
    assert np.array_equal(g2.view(np.uint32), r2.view(np.uint32)), \
        f"{what}: scale2 ({np.count_nonzero(g2 != r2)} differ; mean {g2[-1]!r} vs {r2[-1]!r})"
    assert np.array_equal(g8, r8), f"{what}: scale8 ({np.count_nonzero(g8 != r8)} differ)"
    ref = dq.dequant_f32(rc, r8, r2, w.size, variant)
    got = qb.qlora_dequant(q, torch.float32).cpu().numpy().ravel()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), what + ": dequant f32"
    g16 = qb.qlora_dequant(q, torch.bfloat16).view(torch.int16).cpu().numpy().ravel()
    assert np.array_equal(g16.view(np.uint16), nf4.bf16_rne_bits(ref)), what + ": dequant bf16"


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n", [1, 1000, 16384 * 3 + 777])
def test_ragged(variant, n):
    check(synth.normal_f32((n,), 0.02, [60 + n % 89, 0, 0]), variant, f"{variant} n={n}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_zero_group_and_zero_tensor(variant):
    w = synth.normal_f32((16384 * 3,), 0.02, [61, 0, 0])
    w[16384: 2 * 16384] = 0.0                    # a whole group of zero blocks: c' = −μ there
    w[100:164] = 0.0
    check(w, variant, f"{variant} zero group")
    check(np.zeros(20000, np.float32), variant, f"{variant} zero tensor")


@pytest.mark.parametrize("variant", VARIANTS)
def test_4096_layer(variant):
    check(synth.normal_f32((4096, 4096), 0.02, [77, 0, 0]), variant, f"{variant} 4096x4096")
