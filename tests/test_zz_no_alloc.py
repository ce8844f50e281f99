"""The allocation-free backward (qlora_linear_bwd_noalloc, static device
scratch) against the workspace entry point qlora_linear_bwd: two calls in a
row on one GPU, the second smaller than the first (the scratch keeps the
first call's contents), each compared bit for bit (same kernels, same order,
no atomics), and the size limit reported as an error before any launch.
Neither the binding nor the library allocates device memory in the call."""

import pytest

import synth
from gpu_util import bf16_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(M, d, o, r, seed):
    W = synth.normal_f32((o, d), 0.02, [seed, 0, 0])
    X = bf16_dev(synth.normal_bf16((M, d), 1.0, [seed, 0, 1]))
    A = bf16_dev(synth.normal_bf16((d, r), 0.02, [seed, 0, 2]))
    B = bf16_dev(synth.normal_bf16((r, o), 0.02, [seed, 0, 3]))
    dY = bf16_dev(synth.normal_bf16((M, o), 1.0, [seed, 0, 4]))
    q = qb.qlora_quantize_nf4_dq(torch.from_numpy(W).cuda())
    return q, X, A, B, dY


def _compare(M, d, o, r, seed, given_T):
    q, X, A, B, dY = _case(M, d, o, r, seed)
    T = qb.qlora_linear_fwd(X, q, A, B, 2.0)[1] if given_T else None
    want = qb.qlora_linear_bwd(dY, X, T, q, A, B, 2.0)
    outs = (torch.empty((M, d), dtype=torch.bfloat16, device="cuda"),
            torch.empty((d, r), dtype=torch.bfloat16, device="cuda"),
            torch.empty((r, o), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = qb.qlora_linear_bwd_noalloc(dY, X, T, q, A, B, 2.0, *outs)
    assert torch.cuda.memory_allocated() == before, "the call allocated device memory"
    torch.cuda.synchronize()
    for name, a, b in zip(("dX", "dA", "dB"), got, want):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} M={M} d={d} o={o} r={r}"


def test_two_calls_second_smaller():
    # first the 4096x4096 layer at 4096 tokens, rank 64 (33 MiB of scratch),
    # then a ragged small layer with T recomputed inside the call
    _compare(4096, 4096, 4096, 64, seed=61, given_T=True)
    _compare(130, 256, 200, 16, seed=62, given_T=False)


def test_rank_zero_and_too_large():
    q, X, _, _, dY = _case(40, 128, 96, 8, seed=64)
    want = qb.qlora_linear_bwd(dY, X, None, q, None, None, 2.0)[0]
    dX = torch.empty((40, 128), dtype=torch.bfloat16, device="cuda")
    qb.qlora_linear_bwd_noalloc(dY, X, None, q, None, None, 2.0, dX, None, None)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), want.view(torch.int16))
    # 4096 tokens on an 8192x8192 layer at rank 128 need 98 MiB of scratch
    M, d, o, r = 4096, 8192, 8192, 128
    assert qb.qlora_workspace_bytes(qb.QLORA_OP_BWD, M, d, o, r) > qb.QLORA_NOALLOC_SCRATCH_BYTES
    qz = qb.QuantizedWeight(*(torch.zeros(n, dtype=dt, device="cuda") for n, dt in
                              ((o * d // 2, torch.uint8), (o * d // 64, torch.uint8),
                               (o * d // 16384, torch.float32))), o * d, (o, d))
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    with pytest.raises(qb.QloraError) as e:
        qb.qlora_linear_bwd_noalloc(z(M, o), z(M, d), None, qz, z(d, r), z(r, o), 2.0, z(M, d),
                                    z(d, r), z(r, o))
    assert e.value.status == qb.QLORA_E_SCRATCH
