"""The allocation-free softmax decode, la_softmax_decode_step_static, against
la_softmax_decode_step with a caller workspace, through the C ABI.  Both run the same
kernels, so y and the caches must agree bitwise; each output is also checked against
the FP64 oracle's softmax row.  The calls come in a row, larger then smaller, so later
calls run on the fixed scratch that earlier ones left behind."""
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


def _inputs(torch, H, L, d, dv, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sdt = torch.float64 if dtype == torch.float64 else torch.float32
    sc = 4.0 / math.sqrt(d)
    mk = lambda *shape: (torch.randn(shape, generator=g, device="cuda", dtype=sdt) * sc).to(dtype)
    cap = L + 5
    return mk(H, d), mk(H, d), mk(H, dv), mk(H, cap, d), mk(H, cap, dv)


# (H, L, d, dv): the first needs 64 x 16 pieces of partials, the later ones fewer
CALLS = [(64, 4096, 128, 128), (8, 1000, 64, 64), (3, 300, 40, 24)]


@pytest.mark.parametrize("io", ["bf16", "f32", "f64"])
def test_static_scratch_matches_caller_workspace(torch, io):
    dtype = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[io]
    for n, (H, L, d, dv) in enumerate(CALLS):
        code = {"bf16": la.LA_BF16, "f32": la.LA_F32, "f64": la.LA_F64}[io]
        need = la.la_softmax_decode_workspace_bytes(code, H, L, dv)
        assert 0 < need <= la.LA_SOFTMAX_STATIC_WORKSPACE_BYTES
        q, k, v, Kc, Vc = _inputs(torch, H, L, d, dv, dtype, 9000 + 31 * n + len(io))
        Kc0, Vc0 = Kc.clone(), Vc.clone()
        K1, V1, K2, V2 = Kc.clone(), Vc.clone(), Kc.clone(), Vc.clone()
        y1 = torch.empty((H, dv), device="cuda", dtype=dtype)
        y2 = torch.full((H, dv), float("nan"), device="cuda", dtype=dtype)
        ws = torch.empty(need, device="cuda", dtype=torch.uint8)
        la.la_softmax_decode_step(q, k, v, L - 1, K1, V1, y1, workspace=ws)
        la.la_softmax_decode_step_static(q, k, v, L - 1, K2, V2, y2)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), (io, n)
        assert torch.equal(K1, K2) and torch.equal(V1, V2), (io, n)
        # the oracle: the new row joins the history, then the softmax row over L rows
        K = to_f64(Kc0)[:, :L].copy()
        V = to_f64(Vc0)[:, :L].copy()
        K[:, L - 1] = to_f64(k)
        V[:, L - 1] = to_f64(v)
        ref = oracle.softmax_decode_heads(to_f64(q), K, V, scale=1.0 / math.sqrt(d), threads=8)
        yg = to_f64(y2)
        assert np.isfinite(yg).all()
        if io == "bf16":
            assert max_abs(yg, ref) <= BF16_Y_ABS and maxnorm_rel(yg, ref, 1) <= 2.0 ** -8
        elif io == "f32":
            assert maxnorm_rel(yg, ref, 1) <= F32_REL
        else:
            assert maxnorm_rel(yg, ref, 1) <= 1e-11


def test_static_scratch_refuses_oversized_call(torch):
    """More partials than the fixed scratch holds: rejected before any launch, outputs untouched."""
    H, L, d, dv = 2100, 8192, 8, 128  # 2100 x 32 pieces x 130 floats x 4 B = 34.9 MB > 32 MiB
    assert la.la_softmax_decode_workspace_bytes(la.LA_BF16, H, L, dv) > la.LA_SOFTMAX_STATIC_WORKSPACE_BYTES
    q = torch.zeros((H, d), device="cuda", dtype=torch.bfloat16)
    v = torch.zeros((H, dv), device="cuda", dtype=torch.bfloat16)
    Kc = torch.zeros((H, L, d), device="cuda", dtype=torch.bfloat16)
    Vc = torch.zeros((H, L, dv), device="cuda", dtype=torch.bfloat16)
    y = torch.full((H, dv), 7.0, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        la.la_softmax_decode_step_static(q, q.clone(), v, L - 1, Kc, Vc, y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
