"""GPU parity of the AdamW step of the adapter parameters, device-resident and
paged from host memory, against oracle.adamw bit for bit (fp32 p, m, v and the
bf16 copy of p), over consecutive steps, ragged lengths and pools small enough
to force many pages; and against the textbook fp64 AdamW update within the
rounding bounds of an fp32 evaluation, independent of the operation order."""

import numpy as np
import pytest

import synth
from bounds import adamw_magnitudes, adamw_param_bound, adamw_state_bounds
from oracle import adamw, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(n, seed):
    p = synth.normal_f32((n,), 0.02, [seed, 0, 2])
    gbits = synth.normal_bf16((n,), 1e-3, [seed, 0, 4])
    return p, gbits


def oracle_steps(p, gbits_list, steps):
    g_vals = [nf4.bf16_bits_to_f64(b).astype(np.float32) for b in gbits_list]
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    out = []
    for t in range(1, steps + 1):
        p, m, v, b = adamw.step(p, g_vals[t - 1], m, v, t, lr=HP["lr"], b1=HP["beta1"],
                                b2=HP["beta2"], eps=HP["eps"], wd=HP["weight_decay"])
        out.append((p.copy(), m.copy(), v.copy(), b.copy()))
    return out


def grads(n, seed, steps):
    return [synth.normal_bf16((n,), 1e-3, [seed, t, 4]) for t in range(steps)]


def dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def assert_same(tag, p, m, v, p16, ref):
    rp, rm, rv, rb = ref
    assert np.array_equal(p.cpu().numpy().view(np.uint32), rp.view(np.uint32)), tag + ": p"
    assert np.array_equal(m.cpu().numpy().view(np.uint32) if m.is_cuda else m.numpy().view(np.uint32),
                          rm.view(np.uint32)), tag + ": m"
    assert np.array_equal(v.cpu().numpy().view(np.uint32) if v.is_cuda else v.numpy().view(np.uint32),
                          rv.view(np.uint32)), tag + ": v"
    assert np.array_equal(p16.view(torch.int16).cpu().numpy().view(np.uint16), rb), tag + ": p16"


@pytest.mark.parametrize("n", [5, 4096 * 64 + 37])
def test_device_step_bit_exact(n):
    p0, _ = inputs(n, seed=n % 1000)
    gl = grads(n, n % 1000, 3)
    ref = oracle_steps(p0, gl, 3)
    p = torch.from_numpy(p0.copy()).cuda()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    p16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for t in range(1, 4):
        qb.qlora_adamw_step(p, p16, dev_bf16(gl[t - 1]), m, v, t, lr=HP["lr"], beta1=HP["beta1"],
                            beta2=HP["beta2"], eps=HP["eps"], weight_decay=HP["weight_decay"])
        torch.cuda.synchronize()
        assert_same(f"n={n} t={t}", p, m, v, p16, ref[t - 1])


@pytest.mark.parametrize("n,pool_bytes", [(300_005, 64 << 10), (1000, 1 << 20), (4096 * 3, 8192),
                                          (4 * 256 * 5 + 3, 8192)])
def test_paged_step_bit_exact(n, pool_bytes):
    p0, _ = inputs(n, seed=7)
    gl = grads(n, 7, 2)
    ref = oracle_steps(p0, gl, 2)
    p = torch.from_numpy(p0.copy()).cuda()
    p16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    m = qb.pinned_state(n)
    v = qb.pinned_state(n)
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    for t in range(1, 3):
        qb.qlora_paged_adamw_step(p, p16, dev_bf16(gl[t - 1]), m, v, t, pool, lr=HP["lr"],
                                  beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"],
                                  weight_decay=HP["weight_decay"])
        torch.cuda.synchronize()
        assert_same(f"paged n={n} pool={pool_bytes} t={t}", p, m, v, p16, ref[t - 1])


@pytest.mark.parametrize("paged", [False, True])
def test_steps_within_bounds_of_fp64_definition(paged):
    n = 4096 * 64 + 37
    p0, _ = inputs(n, seed=11)
    gl = grads(n, 11, 5)
    p = torch.from_numpy(p0.copy()).cuda()
    p16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    if paged:
        m, v = qb.pinned_state(n), qb.pinned_state(n)
        pool = torch.empty(256 << 10, dtype=torch.uint8, device="cuda")
    else:
        m, v = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    p64, m64, v64 = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    Mabs, Vabs = np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        g = nf4.bf16_bits_to_f64(gl[t - 1])
        kw = dict(lr=HP["lr"], beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"],
                  weight_decay=HP["weight_decay"])
        if paged:
            qb.qlora_paged_adamw_step(p, p16, dev_bf16(gl[t - 1]), m, v, t, pool, **kw)
        else:
            qb.qlora_adamw_step(p, p16, dev_bf16(gl[t - 1]), m, v, t, **kw)
        torch.cuda.synchronize()
        p64, m64, v64 = adamw.step_fp64(p64, g, m64, v64, t, lr=HP["lr"], b1=HP["beta1"],
                                        b2=HP["beta2"], eps=HP["eps"], wd=HP["weight_decay"])
        gp, gm, gv = (x.cpu().numpy() for x in (p, m, v))
        Mabs, Vabs = adamw_magnitudes(Mabs, Vabs, g, HP["beta1"], HP["beta2"])
        bm, bv = adamw_state_bounds(t, Mabs, Vabs)
        assert np.all(np.abs(gm - m64) <= bm), f"t={t}: m outside the bound"
        assert np.all(np.abs(gv - v64) <= bv), f"t={t}: v outside the bound"
        assert np.max(np.abs(gp - p64)) < adamw_param_bound(t), f"t={t}: p outside the bound"
