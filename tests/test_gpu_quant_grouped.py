"""GPU parity of the grouped quantizer: several tensors in one launch give
exactly the bytes of one call per tensor, and the oracle's bytes.

Cases: ragged lengths (partial blocks, partial groups, a single weight, an
empty tensor) mixed in one call, every code table, the largest count of
tensors, the seven 65B-style block shapes on sampled groups, and non-finite
input in one tensor of the group.
"""

import numpy as np
import pytest

import synth
from oracle import formats, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")

GE = nf4.BLOCK * nf4.GROUP


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bytes(q):
    c, s8, s2 = qb.qlora_quant_sizes(q.n)
    return (q.codes.cpu().numpy()[:c], q.scale8.cpu().numpy()[:s8],
            q.scale2.cpu().numpy()[: s2 // 4].view(np.uint32))


def _same(qa, qb_, tag):
    for name, a, b in zip(("codes", "scale8", "scale2"), _bytes(qa), _bytes(qb_)):
        assert np.array_equal(a, b), f"{tag}: {name} differs"


SIZES = [GE, 1, 65, 0, 3 * GE + 4097, 64 * 100 + 7, GE + 1, 2 * GE]


@pytest.mark.parametrize("fmt", list(qb.FORMATS))
def test_grouped_equals_separate_calls(fmt):
    Ws = [torch.from_numpy(synth.normal_f32((n,), 0.02, [611, k, len(fmt)])).cuda()
          for k, n in enumerate(SIZES)]
    grouped = qb.qlora_quantize_nf4_dq_grouped(Ws, fmt=fmt)
    torch.cuda.synchronize()
    for k, W in enumerate(Ws):
        single = qb.qlora_quantize_nf4_dq(W, fmt=fmt)
        torch.cuda.synchronize()
        _same(grouped[k], single, f"{fmt} tensor {k} (n = {SIZES[k]})")


def test_grouped_matches_oracle():
    """Against the oracle directly, on the ragged members of a group."""
    Ws = [synth.normal_f32((n,), 0.02, [612, k]) for k, n in enumerate(SIZES)]
    grouped = qb.qlora_quantize_nf4_dq_grouped([torch.from_numpy(w).cuda() for w in Ws])
    torch.cuda.synchronize()
    for k, w in enumerate(Ws):
        if w.size == 0:
            continue
        c, s8, s2 = nf4.quantize(w)
        got = _bytes(grouped[k])
        assert np.array_equal(got[0], c), f"codes of tensor {k}"
        assert np.array_equal(got[1], s8), f"scale8 of tensor {k}"
        assert np.array_equal(got[2], np.asarray(s2, dtype=np.float32).view(np.uint32)), f"scale2 of tensor {k}"


def test_grouped_other_table_matches_oracle():
    w = synth.normal_f32((GE + 777,), 0.02, [613, 0])
    (q,) = qb.qlora_quantize_nf4_dq_grouped([torch.from_numpy(w).cuda()], fmt="fp4_e2m1")
    torch.cuda.synchronize()
    c, s8, s2 = formats.quantize(w, "fp4_e2m1")
    got = _bytes(q)
    assert np.array_equal(got[0], c) and np.array_equal(got[1], s8)
    assert np.array_equal(got[2], np.asarray(s2, dtype=np.float32).view(np.uint32))


def test_grouped_largest_count_and_reuse():
    n = [GE * (1 + k % 3) + 64 * k for k in range(qb.QLORA_MAX_GROUPED)]
    Ws = [torch.from_numpy(synth.normal_f32((m,), 0.02, [614, k])).cuda() for k, m in enumerate(n)]
    first = qb.qlora_quantize_nf4_dq_grouped(Ws)
    copies = [tuple(x.copy() for x in _bytes(q)) for q in first]
    again = qb.qlora_quantize_nf4_dq_grouped(Ws, outs=first)      # same buffers, rewritten
    torch.cuda.synchronize()
    for k, q in enumerate(again):
        assert q is first[k]
        for a, b in zip(_bytes(q), copies[k]):
            assert np.array_equal(a, b)
        single = qb.qlora_quantize_nf4_dq(Ws[k])
        _same(q, single, f"tensor {k}")
    with pytest.raises(ValueError):
        qb.qlora_quantize_nf4_dq_grouped(Ws + Ws[:1])


def test_grouped_65b_block_shapes_sampled():
    """The seven 65B-style tensors in one launch, checked on sampled groups of each."""
    wl = synth.WORKLOADS["block_65b"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(615)
    Ws = []
    for p in wl.projs:
        W = torch.empty((p.o, p.d), dtype=torch.float32, device="cuda")
        W.normal_(0.0, wl.w_std, generator=gen)
        Ws.append(W)
    qs = qb.qlora_quantize_nf4_dq_grouped(Ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(616)
    for W, q in zip(Ws, qs):
        ng = (W.numel() + GE - 1) // GE
        for g in sorted(set(rng.integers(0, ng, 3).tolist()) | {0, ng - 1}):
            lo, hi = g * GE, min(W.numel(), (g + 1) * GE)
            w = W.view(-1)[lo:hi].cpu().numpy()
            c, s8, s2 = nf4.quantize(w)
            assert np.array_equal(q.codes[lo // 2: lo // 2 + c.size].cpu().numpy(), c)
            assert np.array_equal(q.scale8[lo // 64: lo // 64 + s8.size].cpu().numpy(), s8)
            assert q.scale2[g].item() == np.float32(s2[0])
        del W
    del Ws


def test_grouped_flags_non_finite():
    Ws = [torch.from_numpy(synth.normal_f32((GE,), 0.02, [617, k])).cuda() for k in range(3)]
    Ws[1][5000] = float("nan")
    with pytest.raises(qb.QloraError):
        qb.qlora_quantize_nf4_dq_grouped(Ws)
    Ws[1][5000] = 0.0
    qb.qlora_quantize_nf4_dq_grouped(Ws)
