"""GPU parity of the fp32 MFMA chunked prefill (f32 inputs, d = dv = 128, chunk 64) against
the FP64 oracle, through the C ABI, at the fp32 bar (1e-4: per-head max-norm relative on y
and S, elementwise relative on z): ragged lengths, one to many segments per sequence,
gates including zero gates, a carried state, and the ungated prefill shape
(B=4, H=16, T=4096) in fp32 in full."""
import numpy as np
import pytest

import recurrent_state_chunkwise_amd as la
from recurrent_state_chunkwise_amd import workloads as wl

from helpers import F32_REL, assert_prefill_parity, oracle_prefill

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _inputs(torch, B, H, T, gated, with_state, seed, zero_gates=False):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    mk = lambda s: torch.randn((B, H, T, D), generator=g, device="cuda") * s
    Q, K, V = mk(0.7), mk(0.7), mk(1.0)
    alpha = None
    if gated:
        alpha = torch.sigmoid(torch.randn((B, H, T), generator=g, device="cuda") + 2.0)
        if zero_gates:
            alpha[..., T // 2] = 0.0
            alpha[..., 0] = 0.0
            if T > 700:
                alpha[..., 640] = 0.0  # the first token of a segment when segments are 320 long
    S0 = z0 = None
    if with_state:
        S0 = torch.randn((B, H, D, D), generator=g, device="cuda") * 0.3
        z0 = torch.rand((B, H, D), generator=g, device="cuda") * 5.0 + 0.5
    return Q, K, V, alpha, S0, z0


def _run(torch, Q, K, V, alpha, S0, z0, eps=1e-6):
    B, H, T, _ = Q.shape
    Y = torch.empty_like(V)
    S = torch.empty((B, H, D, D), device="cuda")
    z = torch.empty((B, H, D), device="cuda")
    if S0 is None:
        la.la_state_init(S, z)
    else:
        S.copy_(S0)
        z.copy_(z0)
    la.la_prefill_chunked(Q, K, V, alpha, eps, 64, Y, S, z)
    torch.cuda.synchronize()
    return Y, S, z


CASES = [
    # B, H, T, gated, with_state, zero_gates      (segments per sequence in the comment)
    (1, 2, 1, False, False, False),      # 1
    (1, 2, 63, True, True, False),       # 1, one partial chunk
    (1, 2, 200, True, False, True),      # 1, ragged
    (1, 3, 257, False, True, False),     # 1
    (2, 4, 700, True, True, True),       # 2
    (1, 2, 2000, False, True, False),    # 6
    (1, 2, 2100, True, True, True),      # 6, zero gates inside and at a segment start
    (1, 16, 1300, True, True, False),    # 4
    (1, 1, 4000, True, True, False),     # 12: more maps than the scan reads in one batch
    (2, 64, 96, False, False, False),    # 1, 128 sequences
]


@pytest.mark.parametrize("case", CASES)
def test_f32_mfma_prefill_parity(torch, case):
    B, H, T, gated, with_state, zero_gates = case
    assert la.la_prefill_variant(la.LA_F32, D, D, 64, gated, la.LA_F32) == 2
    Q, K, V, alpha, S0, z0 = _inputs(torch, B, H, T, gated, with_state, 31 * T + H, zero_gates)
    Y, S, z = _run(torch, Q, K, V, alpha, S0, z0)
    m = assert_prefill_parity(Y, S, z, oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0), "f32", str(case))
    print(case, m)


def test_f32_mfma_prefill_full_shape(torch):
    """The ungated prefill shape in fp32: 64 sequences x 4096 tokens, 4 segments each."""
    cfg = wl.PREFILL_UNGATED_F32
    assert la.la_prefill_segments(cfg.B * cfg.H, cfg.T, 64, la.LA_F32) == (4, 1024)
    Q, K, V, A = wl.prefill_inputs(cfg, "cuda")
    Y, S, z = _run(torch, Q, K, V, A, None, None, cfg.eps)
    m = assert_prefill_parity(Y, S, z, oracle_prefill(Q, K, V, A, cfg.eps, threads=16), "f32", cfg.name)
    print(cfg.name, m)


def test_f32_mfma_causality_and_resume(torch):
    """Later tokens leave earlier outputs bitwise unchanged; a prefill resumed from a returned
    state matches one call over the whole sequence within the fp32 bar."""
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 2, 1500, True, True, 808)
    Y1, S1, z1 = _run(torch, Q, K, V, alpha, S0, z0)
    K2, V2 = K.clone(), V.clone()
    K2[:, :, 900:] += 3.0
    V2[:, :, 900:] -= 1.0
    Y2, _, _ = _run(torch, Q, K2, V2, alpha, S0, z0)
    assert torch.equal(Y1[:, :, :900], Y2[:, :, :900])
    cut = 640
    part = lambda t: t[:, :, :cut].contiguous()
    rest = lambda t: t[:, :, cut:].contiguous()
    Ya, Sa, za = _run(torch, part(Q), part(K), part(V), part(alpha), S0, z0)
    Yb, Sb, zb = _run(torch, rest(Q), rest(K), rest(V), rest(alpha), Sa, za)
    Yab = torch.cat([Ya, Yb], dim=2)
    rel = lambda a, b: float((a - b).abs().max() / b.abs().max())
    assert rel(Yab, Y1) <= F32_REL and rel(Sb, S1) <= F32_REL
    assert float(((zb - z1).abs() / z1).max()) <= F32_REL
