"""GPU parity of the softmax attention decode over an explicit K/V history (the
comparator of the fixed-state measurement) against the FP64 oracle, through the C
ABI: histories inside one 256-row piece and across several (so the combine kernel
runs), the bf16 vector path and the element-wise path (f32, f64, widths that are not
multiples of 8), the new row written to the caches and nothing else touched, steps in
sequence, and the 8-head, 64-wide, 8,192-row shape of the measurement."""
import math

import numpy as np
import pytest

import oracle
import recurrent_state_chunkwise_amd as la

from helpers import BF16_Y_ABS, F32_REL, max_abs, maxnorm_rel, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _case(torch, H, d, dv, pos, cap, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sdt = torch.float64 if dtype == torch.float64 else torch.float32
    sc = 1.0 / math.sqrt(d)
    mk = lambda *shape: (torch.randn(shape, generator=g, device="cuda", dtype=sdt) * sc * 4).to(dtype)
    Kc, Vc = mk(H, cap, d), mk(H, cap, dv)
    q, k, v = mk(H, d), mk(H, d), mk(H, dv)
    return q, k, v, Kc, Vc


def _oracle_y(q, k, v, Kc0, Vc0, pos):
    K = to_f64(Kc0)[:, :pos + 1].copy()
    V = to_f64(Vc0)[:, :pos + 1].copy()
    K[:, pos] = to_f64(k)
    V[:, pos] = to_f64(v)
    return oracle.softmax_decode_heads(to_f64(q), K, V, scale=1.0 / math.sqrt(q.shape[1]), threads=8)


def _check(torch, y, ref, dt, label):
    yg = to_f64(y)
    assert np.isfinite(yg).all(), label
    yr = maxnorm_rel(yg, ref, 1)
    ya = max_abs(yg, ref)
    print("%s: y abs %.2e y rel %.2e" % (label, ya, yr))
    if dt == "bf16":
        assert ya <= BF16_Y_ABS and yr <= 2.0 ** -8, (label, ya, yr)
    elif dt == "f32":
        assert yr <= F32_REL, (label, yr)
    else:
        assert yr <= 1e-11, (label, yr)


CASES = [
    # H, d, dv, pos, dtype
    (3, 64, 64, 0, "bf16"),
    (3, 64, 64, 5, "bf16"),
    (2, 64, 64, 255, "bf16"),     # exactly one piece
    (2, 64, 64, 256, "bf16"),     # two pieces, the new row alone in the second
    (4, 128, 128, 1000, "bf16"),
    (2, 64, 16, 700, "bf16"),
    (2, 64, 24, 300, "bf16"),     # dv / 8 not a power of two: element-wise path
    (3, 40, 24, 600, "f32"),
    (2, 8, 8, 300, "f64"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H%d_d%d_dv%d_pos%d_%s" % c)
def test_softmax_decode_parity(torch, case):
    H, d, dv, pos, dt = case
    dtype = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[dt]
    cap = pos + 7
    q, k, v, Kc, Vc = _case(torch, H, d, dv, pos, cap, dtype, 900 + CASES.index(case))
    Kc0, Vc0 = Kc.clone(), Vc.clone()
    y = torch.empty((H, dv), device="cuda", dtype=dtype)
    la.la_softmax_decode_step(q, k, v, pos, Kc, Vc, y)
    torch.cuda.synchronize()
    _check(torch, y, _oracle_y(q, k, v, Kc0, Vc0, pos), dt, str(case))
    # the new row went into the caches; no other row changed
    assert torch.equal(Kc[:, pos], k) and torch.equal(Vc[:, pos], v)
    keep = [i for i in range(cap) if i != pos]
    assert torch.equal(Kc[:, keep], Kc0[:, keep]) and torch.equal(Vc[:, keep], Vc0[:, keep])


def test_softmax_decode_steps_in_sequence(torch):
    H, d, dv, cap = 4, 64, 64, 600
    q, k, v, Kc, Vc = _case(torch, H, d, dv, 0, cap, torch.bfloat16, 950)
    g = torch.Generator(device="cuda")
    g.manual_seed(951)
    for pos in (250, 251, 252, 511, 512):
        qs, ks, vs = [(torch.randn((H, w), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
                      for w in (d, d, dv)]
        Kc0, Vc0 = Kc.clone(), Vc.clone()
        y = torch.empty((H, dv), device="cuda", dtype=torch.bfloat16)
        la.la_softmax_decode_step(qs, ks, vs, pos, Kc, Vc, y)
        torch.cuda.synchronize()
        _check(torch, y, _oracle_y(qs, ks, vs, Kc0, Vc0, pos), "bf16", "step pos %d" % pos)


def test_softmax_decode_measurement_shape(torch):
    """8 heads x 64, bf16, 8,192 history rows: the longest history of the measurement."""
    H, d, dv, L = 8, 64, 64, 8192
    q, k, v, Kc, Vc = _case(torch, H, d, dv, L - 1, L, torch.bfloat16, 960)
    Kc0, Vc0 = Kc.clone(), Vc.clone()
    y = torch.empty((H, dv), device="cuda", dtype=torch.bfloat16)
    la.la_softmax_decode_step(q, k, v, L - 1, Kc, Vc, y)
    torch.cuda.synchronize()
    _check(torch, y, _oracle_y(q, k, v, Kc0, Vc0, L - 1), "bf16", "H8 d64 L8192")


def test_softmax_decode_sharp_scores(torch):
    """A key aligned with the query at large scale takes nearly all the weight: the
    piece maxima and the rescaling in the combine must keep that exact."""
    H, d, dv, pos = 2, 64, 64, 700
    q, k, v, Kc, Vc = _case(torch, H, d, dv, pos, pos + 1, torch.bfloat16, 970)
    Kc[:, 333] = q * 8  # score 64 |q|^2 / 8 above the rest
    Kc0, Vc0 = Kc.clone(), Vc.clone()
    y = torch.empty((H, dv), device="cuda", dtype=torch.bfloat16)
    la.la_softmax_decode_step(q, k, v, pos, Kc, Vc, y)
    torch.cuda.synchronize()
    ref = _oracle_y(q, k, v, Kc0, Vc0, pos)
    _check(torch, y, ref, "bf16", "sharp")
