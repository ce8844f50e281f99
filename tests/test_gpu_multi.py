"""GPU parity of the multi-adapter few-token forward against oracle.multi.

One frozen 4-bit base, several LoRA adapters, an adapter index per token
([LoRA-PyTorch §四.5]; the weimeta glossary FAQ on serving many adapters over
one base).  Y and T are compared with the bf16 tolerance rule of gpu_util;
rows whose index selects no adapter must give T = 0 exactly; and a batch in
which every row uses adapter a must reproduce qlora_linear_fwd with
(A[a], B[a], s[a]) bit for bit.
"""

import numpy as np
import pytest

import synth
from gpu_util import bf16_dev, bf16_host_f64, bf16_to_f64, check_close
from oracle import multi, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make(M, d, o, r, n, seed):
    W = synth.normal_f32((o, d), 0.02, [seed, 0, 0])
    X = synth.normal_bf16((M, d), 1.0, [seed, 0, 1])
    A = synth.normal_bf16((n, d, r), 0.02, [seed, 0, 2])
    B = synth.normal_bf16((n, r, o), 0.02, [seed, 0, 3])
    s = [float(v) for v in np.random.default_rng(seed).choice([2.0, 0.5, -1.0, 1.5, 0.25], size=n)]
    return W, X, A, B, s


def oracle_weight(W):
    o, d = W.shape
    c, s8, s2 = nf4.quantize(W.ravel())
    return nf4.bf16_bits_to_f64(nf4.dequant_bf16_bits(c, s8, s2, W.size)).reshape(o, d)


def run(W, X, A, B, s, idx, want_T=True):
    q = qb.qlora_quantize_nf4_dq(torch.from_numpy(W).cuda())
    ad = torch.tensor(np.asarray(idx, np.int32), device="cuda")
    Y, T = qb.qlora_linear_fwd_multi(bf16_dev(X), q, bf16_dev(A), bf16_dev(B), s, ad, want_T=want_T)
    torch.cuda.synchronize()
    return q, Y, T


@pytest.mark.parametrize("M,d,o,r,n", [
    (1, 256, 264, 16, 3),
    (5, 640, 136, 8, 4),
    (16, 1024, 520, 24, 16),
    (3, 192, 40, 64, 2),
])
def test_parity_with_oracle(M, d, o, r, n):
    W, X, A, B, s = make(M, d, o, r, n, seed=M * 31 + n)
    rng = np.random.default_rng(M + d)
    idx = rng.integers(0, n, size=M).astype(np.int32)
    if M >= 3:
        idx[1], idx[2] = -1, n + 3            # no adapter, out of range
    q, Y, T = run(W, X, A, B, s, idx)
    Yr, Tr = multi.forward(bf16_to_f64(X), oracle_weight(W), bf16_to_f64(A), bf16_to_f64(B), s,
                           np.where((idx >= 0) & (idx < n), idx, -1))
    tag = f"M={M} d={d} o={o} r={r} n={n}"
    check_close(bf16_host_f64(Y), Yr, "Y " + tag)
    Th = T.cpu().numpy()
    check_close(Th, Tr, "T " + tag)
    for m in range(M):
        if not 0 <= idx[m] < n:
            assert not Th[m].any(), f"row {m} has no adapter but T != 0"


@pytest.mark.parametrize("a", [0, 2])
def test_shared_adapter_matches_single_adapter_bitwise(a):
    M, d, o, r, n = 7, 512, 264, 16, 3
    W, X, A, B, s = make(M, d, o, r, n, seed=17)
    q, Y, T = run(W, X, A, B, s, [a] * M)
    Ys, Ts = qb.qlora_linear_fwd(bf16_dev(X), q, bf16_dev(A[a]), bf16_dev(B[a]), s[a])
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Ys.view(torch.int16))
    assert torch.equal(T, Ts)


def test_decode_7b_gate_sixteen_adapters():
    """Full 7B gate projection (11008×4096), 16 tokens on 16 different adapters."""
    M, d, o, r, n = 16, 4096, 11008, 16, 16
    W, X, A, B, s = make(M, d, o, r, n, seed=23)
    idx = np.arange(M, dtype=np.int32)[::-1].copy()
    q, Y, T = run(W, X, A, B, s, idx)
    Yr, Tr = multi.forward(bf16_to_f64(X), oracle_weight(W), bf16_to_f64(A), bf16_to_f64(B), s, idx)
    check_close(bf16_host_f64(Y), Yr, "Y gate 16 adapters")
    check_close(T.cpu().numpy(), Tr, "T gate 16 adapters")
