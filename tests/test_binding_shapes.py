"""The Python binding checks every operand's shape before anything reaches the
C ABI, which receives sizes only: a mis-shaped tensor raises ValueError and no
kernel is launched.  CPU tensors stand in for device tensors here: with
shapes right, the same calls fail on the device check instead (TypeError),
which shows the shape check ran first and passed."""

import pytest

torch = pytest.importorskip("torch")
qb = pytest.importorskip("nf4_double_quant_amd")


def qweight(o, d, dq=0, short=None):
    n = o * d
    nb = -(-n // 64)
    sizes = {"codes": 4 * -(-n // 8), "scale8": nb, "scale2": 4 * -(-nb // 256) + (4 if dq else 0)}
    if short:
        sizes[short] -= 1
    return qb.QuantizedWeight(torch.zeros(sizes["codes"], dtype=torch.uint8),
                              torch.zeros(sizes["scale8"], dtype=torch.uint8),
                              torch.zeros(-(-sizes["scale2"] // 4), dtype=torch.float32)
                              if short != "scale2" else torch.zeros(0, dtype=torch.float32),
                              n, (o, d), 0, dq)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


M, d, o, r = 5, 128, 64, 8


def fwd(**kw):
    a = dict(X=bf(M, d), q=qweight(o, d), A=bf(d, r), B=bf(r, o), s=2.0)
    a.update(kw)
    return qb.qlora_linear_fwd(a["X"], a["q"], a["A"], a["B"], a["s"], out=a.get("out"))


def bwd(**kw):
    a = dict(dY=bf(M, o), X=bf(M, d), T=torch.zeros(M, r), q=qweight(o, d), A=bf(d, r), B=bf(r, o))
    a.update(kw)
    return qb.qlora_linear_bwd(a["dY"], a["X"], a["T"], a["q"], a["A"], a["B"], 2.0)


def test_forward_shapes_right_reach_the_device_check():
    with pytest.raises(TypeError):
        fwd()


@pytest.mark.parametrize("kw", [
    dict(X=bf(M, d + 64)), dict(X=bf(M, d, 1)), dict(A=bf(d, r + 8)[:, :r].contiguous().T),
    dict(A=bf(d + 1, r)), dict(B=bf(r, o + 8)), dict(B=bf(r + 8, o)), dict(out=bf(M, o + 8)),
    dict(out=bf(M + 1, o)), dict(A=None), dict(q=qweight(o, d, short="codes")),
    dict(q=qweight(o, d, short="scale8")), dict(q=qweight(o, d, short="scale2")),
])
def test_forward_rejects_wrong_shapes(kw):
    with pytest.raises(ValueError):
        fwd(**kw)


def test_backward_shapes_right_reach_the_device_check():
    with pytest.raises(TypeError):
        bwd()


@pytest.mark.parametrize("kw", [
    dict(dY=bf(M, o + 8)), dict(X=bf(M + 1, d)), dict(X=bf(M, d - 64)), dict(T=torch.zeros(M, r + 1)),
    dict(T=torch.zeros(M + 1, r)), dict(A=bf(d, r + 8)), dict(B=bf(r, o - 8)), dict(B=None),
])
def test_backward_rejects_wrong_shapes(kw):
    with pytest.raises(ValueError):
        bwd(**kw)


def test_multi_adapter_rejects_wrong_shapes():
    n = 3
    good = dict(X=bf(M, d), A=bf(n, d, r), B=bf(n, r, o), idx=torch.zeros(M, dtype=torch.int32))

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return qb.qlora_linear_fwd_multi(a["X"], qweight(o, d), a["A"], a["B"], [2.0] * n, a["idx"],
                                         out=a.get("out"))

    with pytest.raises(TypeError):
        call()
    for kw in (dict(A=bf(n, d, r + 8)), dict(B=bf(n + 1, r, o)), dict(B=bf(n, r, o + 8)),
               dict(idx=torch.zeros(M + 1, dtype=torch.int32)), dict(out=bf(M, o - 8)),
               dict(A=bf(d, r))):
        with pytest.raises(ValueError):
            call(**kw)


def test_merge_and_optimizer_reject_wrong_shapes():
    with pytest.raises(TypeError):
        qb.qlora_merge_adapter(qweight(o, d), bf(d, r), bf(r, o), 2.0)
    for A, B, out in ((bf(d, r), bf(r + 8, o), None), (bf(d + 64, r), bf(r, o), None),
                      (bf(d, r), bf(r, o), torch.zeros(d, o))):
        with pytest.raises(ValueError):
            qb.qlora_merge_adapter(qweight(o, d), A, B, 2.0, out=out)
    n = 100
    p, g, p16, m, v = torch.zeros(n), bf(n), bf(n), torch.zeros(n), torch.zeros(n)
    with pytest.raises(TypeError):
        qb.qlora_adamw_step(p, p16, g, m, v, 1)
    for args in ((p, p16, bf(n - 1), m, v), (p, bf(n + 1), g, m, v), (p, p16, g, torch.zeros(n + 4), v)):
        with pytest.raises(ValueError):
            qb.qlora_adamw_step(*args, 1)
    with pytest.raises(ValueError):
        qb.qlora_paged_adamw_step(p, p16, g, torch.zeros(n - 1), v, 1, torch.zeros(4096, dtype=torch.uint8))
