"""GPU parity of the quantizer and dequantizer: bit-exact against the oracle.

Cases: the 128×128 workload, ragged lengths (partial blocks and groups),
adversarial values (exact ties between codebook values and between scale
levels, zero blocks and groups, subnormals, huge magnitudes), weights on a
fine grid of w/c1 and at the edges of the fp32 range, non-finite
input, determinism, and the full-size weight shapes of the 4096×4096 layer,
the 7B-style MLP (11008×4096) and the 65B-style MLP (22016×8192), the last
two checked on sampled double-quant groups (quantization is group-local),
and a ragged tensor large enough for the streaming launch configuration.
"""

import numpy as np
import pytest

import synth
from gpu_util import grid_and_scale_blocks
from oracle import nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")

GE = nf4.BLOCK * nf4.GROUP


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_quantize(w: np.ndarray):
    W = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).ravel()).cuda()
    q = qb.qlora_quantize_nf4_dq(W)
    c, s8, s2 = qb.qlora_quant_sizes(w.size)
    torch.cuda.synchronize()
    return (q, q.codes.cpu().numpy()[:c], q.scale8.cpu().numpy()[:s8],
            q.scale2.cpu().numpy()[: s2 // 4])


def assert_quant_exact(w: np.ndarray, what: str):
    q, c, s8, s2 = gpu_quantize(w)
    rc, rs8, rs2 = nf4.quantize(w.ravel())
    assert np.array_equal(s2.view(np.uint32), rs2.view(np.uint32)), f"{what}: scale2"
    assert np.array_equal(s8, rs8), f"{what}: scale8 ({np.count_nonzero(s8 != rs8)} differ)"
    assert np.array_equal(c, rc), f"{what}: codes ({np.count_nonzero(c != rc)} bytes differ)"
    return q


def test_tiny_128_exact_and_dequant():
    wl = synth.WORKLOADS["tiny_128"]
    W = synth.layer_inputs(wl, wl.projs[0])[0]
    q = assert_quant_exact(W, "tiny_128")
    ref = nf4.dequant_f32(*nf4.quantize(W.ravel()), W.size)
    got32 = qb.qlora_dequant(q, torch.float32).cpu().numpy().ravel()
    assert np.array_equal(got32.view(np.uint32), ref.view(np.uint32))
    got16 = qb.qlora_dequant(q, torch.bfloat16).view(torch.int16).cpu().numpy().ravel().view(np.uint16)
    assert np.array_equal(got16, nf4.bf16_rne_bits(ref))


@pytest.mark.parametrize("n", [1, 2, 7, 63, 64, 65, 1000, 16383, 16384, 16385, 3 * 16384 + 1037])
def test_ragged_lengths(n):
    w = (np.random.default_rng(n).standard_normal(n) * 0.02).astype(np.float32)
    assert_quant_exact(w, f"n={n}")


def _adversarial():
    V = nf4.codebook().astype(np.float64)
    mids = (V[:-1] + V[1:]) / 2
    rng = np.random.default_rng(123)
    parts = []
    # blocks whose weights sit exactly on (and one ulp around) the decision points
    for e in (0, -3, -17, -60):
        c1 = 2.0 ** e
        blk = [c1]
        for m in mids:
            x = np.float32(m * c1)
            blk += [x, np.nextafter(x, np.float32(1)), np.nextafter(x, np.float32(-1))]
        blk = (blk + [0.0] * 64)[:64]
        parts.append(np.array(blk, dtype=np.float32))
    parts.append(np.zeros(64, np.float32))                       # zero block
    parts.append(-np.zeros(64, np.float32))                      # negative zeros
    parts.append((rng.standard_normal(64) * 1e-41).astype(np.float32))   # subnormals
    parts.append((rng.standard_normal(64) * 1e37).astype(np.float32))    # huge
    g0 = np.concatenate(parts)
    g0 = np.concatenate([g0, (rng.standard_normal(GE - g0.size) * 0.02).astype(np.float32)])
    # group whose block maxima sit exactly on half-steps of an exact step 2^-10
    g1 = np.zeros(GE, np.float32)
    step = 2.0 ** -10
    g1[0] = np.float32(255 * step)
    for b in range(1, 256):
        c1 = np.float32(((b * 7) % 255 + 0.5) * step)
        blk = (rng.uniform(-1, 1, 64) * c1).astype(np.float32)
        blk[b % 64] = c1 if b % 2 else -c1
        g1[b * 64:(b + 1) * 64] = blk
    g2 = np.zeros(GE, np.float32)                                # zero group
    g3 = (rng.standard_normal(GE) * 1e-39).astype(np.float32)    # subnormal group
    return np.concatenate([g0, g1, g2, g3, g0[:777]])


def test_adversarial_values():
    w = _adversarial()
    q = assert_quant_exact(w, "adversarial")
    ref = nf4.dequant_f32(*nf4.quantize(w), w.size)
    got = qb.qlora_dequant(q, torch.float32).cpu().numpy().ravel()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_grid_points_and_extreme_scales():
    w = grid_and_scale_blocks(nf4.codebook(), 31)
    w = np.concatenate([w, (np.random.default_rng(32).standard_normal(GE - w.size % GE) * 0.02)
                        .astype(np.float32)])
    q = assert_quant_exact(w, "grid and extreme scales")
    ref = nf4.dequant_f32(*nf4.quantize(w), w.size)
    got = qb.qlora_dequant(q, torch.float32).cpu().numpy().ravel()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_exact_zero_round_trip_on_gpu():
    w = (np.random.default_rng(5).standard_normal(GE * 2) * 0.02).astype(np.float32)
    zi = np.random.default_rng(6).choice(w.size, 999, replace=False)
    w[zi] = 0.0
    q, *_ = gpu_quantize(w)
    got = qb.qlora_dequant(q, torch.float32).cpu().numpy().ravel()
    assert np.all(got[zi] == 0.0)


def test_nonfinite_sets_flag():
    for bad in (np.nan, np.inf, -np.inf):
        w = (np.random.default_rng(1).standard_normal(GE + 100) * 0.02).astype(np.float32)
        w[GE + 17] = bad
        W = torch.from_numpy(w).cuda()
        with pytest.raises(qb.QloraError) as ei:
            qb.qlora_quantize_nf4_dq(W)
        assert ei.value.status == qb.QLORA_E_NONFINITE
        q = qb.qlora_quantize_nf4_dq(torch.from_numpy(w[:GE].copy()).cuda())   # clean part passes
        assert int(q.flags.item()) == 0


def test_deterministic():
    w = (np.random.default_rng(9).standard_normal(GE * 7 + 5) * 0.02).astype(np.float32)
    a = gpu_quantize(w)[1:]
    b = gpu_quantize(w)[1:]
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


def test_dequant_of_oracle_buffers():
    """The GPU dequantizer fed the oracle's own quantized buffers."""
    n = GE * 3 + 4321
    w = (np.random.default_rng(11).standard_normal(n) * 0.02).astype(np.float32)
    rc, rs8, rs2 = nf4.quantize(w)
    q = qb.QuantizedWeight(torch.from_numpy(rc).cuda(), torch.from_numpy(rs8).cuda(),
                           torch.from_numpy(rs2).cuda(), n, (n,))
    ref = nf4.dequant_f32(rc, rs8, rs2, n)
    got = qb.qlora_dequant(q, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    got16 = qb.qlora_dequant(q, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, nf4.bf16_rne_bits(ref))


def test_full_4096_layer_exact():
    wl = synth.WORKLOADS["linear_4096"]
    W = synth.normal_f32((4096, 4096), wl.w_std, [wl.wid, 0, synth.T_W])
    assert_quant_exact(W, "linear_4096")


@pytest.mark.parametrize("wname,proj", [("decode_mlp_7b", "gate"), ("decode_mlp_7b", "down"),
                                        ("block_65b", "gate"), ("block_65b", "down")])
def test_full_size_sampled_groups(wname, proj):
    wl = synth.WORKLOADS[wname]
    p = [x for x in wl.projs if x.name == proj][0]
    W = synth.normal_f32((p.o, p.d), wl.w_std, [wl.wid, synth.PROJ_IDS[p.name], synth.T_W]).ravel()
    q, c, s8, s2 = gpu_quantize(W)
    ng = s2.size
    groups = sorted(set(np.random.default_rng(0).choice(ng, 24, replace=False).tolist()) | {0, ng - 1})
    for g in groups:
        rc, rs8, rs2 = nf4.quantize(W[g * GE:(g + 1) * GE])
        assert rs2[0].view(np.uint32) == s2[g].view(np.uint32), g
        assert np.array_equal(rs8, s8[g * 256:(g + 1) * 256]), g
        assert np.array_equal(rc, c[g * GE // 2:(g + 1) * GE // 2]), g
    del q


def test_streaming_instance_ragged():
    """A tensor past the size where the quantizer streams from HBM (its other
    launch configuration, with non-temporal code stores), with a length that
    ends inside a block and inside a code word: sampled groups and the partial
    last group against the oracle, alone and as a member of a grouped launch
    with a small ragged tensor."""
    n = 84_000_000 + 4097
    assert n * 4 > 320 << 20
    W = synth.normal_f32((n,), 0.02, [631, 0])
    small = synth.normal_f32((3 * GE + 4097,), 0.02, [631, 1])
    q, c, s8, s2 = gpu_quantize(W)
    ng = s2.size
    assert ng == (n + GE - 1) // GE
    grouped = qb.qlora_quantize_nf4_dq_grouped([torch.from_numpy(W).cuda(), torch.from_numpy(small).cuda()])
    torch.cuda.synchronize()
    gc = grouped[0].codes.cpu().numpy()[: c.size]
    gs8 = grouped[0].scale8.cpu().numpy()[: s8.size]
    gs2 = grouped[0].scale2.cpu().numpy()[: s2.size]
    assert np.array_equal(gc, c) and np.array_equal(gs8, s8) and np.array_equal(gs2.view(np.uint32), s2.view(np.uint32))
    groups = sorted(set(np.random.default_rng(1).choice(ng - 1, 8, replace=False).tolist()) | {0, ng - 1})
    for g in groups:
        rc, rs8, rs2 = nf4.quantize(W[g * GE:(g + 1) * GE])
        assert rs2[0].view(np.uint32) == s2[g].view(np.uint32), g
        assert np.array_equal(rs8, s8[g * 256: g * 256 + rs8.size]), g
        assert np.array_equal(rc, c[g * GE // 2: g * GE // 2 + rc.size]), g
    rc, rs8, rs2 = nf4.quantize(small)
    got = (grouped[1].codes.cpu().numpy()[: rc.size], grouped[1].scale8.cpu().numpy()[: rs8.size],
           grouped[1].scale2.cpu().numpy()[: rs2.size])
    assert np.array_equal(got[0], rc) and np.array_equal(got[1], rs8)
    assert np.array_equal(got[2].view(np.uint32), np.asarray(rs2, dtype=np.float32).view(np.uint32))
    del q, grouped
