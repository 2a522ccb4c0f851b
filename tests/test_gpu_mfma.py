"""GPU parity of the bf16 MFMA chunked prefill (d = dv = 128, chunk 64 or 128)
against the FP64 oracle, through the C ABI: ragged lengths, one to many segments
per sequence, gates (including zero gates), carried state, the page's worked
examples embedded at width 128, causality and chunk invariance."""
import math

import numpy as np
import pytest

import recurrent_state_chunkwise_amd as la

from helpers import BF16_STATE_REL, BF16_Y_ABS, Y_MAXNORM_REL, Z_REL, elem_rel, max_abs, maxnorm_rel, oracle_prefill, to_f64

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _inputs(torch, B, H, T, gated, with_state, seed, zero_gates=False, scale=1 / math.sqrt(128)):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    mk = lambda w: (torch.randn((B, H, T, w), generator=g, device="cuda") * scale).to(torch.bfloat16)
    Q, K, V = mk(D), mk(D), mk(D)
    alpha = None
    if gated:
        alpha = torch.sigmoid(torch.randn((B, H, T), generator=g, device="cuda") + 3.0)
        if zero_gates:
            alpha[..., T // 3] = 0.0
            alpha[..., min(T - 1, 70)] = 0.0
            alpha[..., 0] = 0.0
    S0 = z0 = None
    if with_state:
        S0 = torch.randn((B, H, D, D), generator=g, device="cuda") * 0.05
        z0 = torch.rand((B, H, D), generator=g, device="cuda") * 20.0 + 1.0
    return Q, K, V, alpha, S0, z0


def _run(torch, Q, K, V, alpha, chunk, S0=None, z0=None, eps=1e-6):
    B, H, T, _ = Q.shape
    Y = torch.empty_like(V)
    S = torch.empty((B, H, D, D), device="cuda")
    z = torch.empty((B, H, D), device="cuda")
    if S0 is None:
        la.la_state_init(S, z)
    else:
        S.copy_(S0)
        z.copy_(z0)
    la.la_prefill_chunked(Q, K, V, alpha, eps, chunk, Y, S, z)
    torch.cuda.synchronize()
    return Y, S, z


def _check(Y, S, z, ref, label):
    Yr, Sr, zr, _ = ref
    Yg, Sg, zg = to_f64(Y), to_f64(S), to_f64(z)
    assert np.isfinite(Yg).all() and np.isfinite(Sg).all() and np.isfinite(zg).all(), label
    ya, yr = max_abs(Yg, Yr), maxnorm_rel(Yg, Yr, 2)
    sr, zrel = maxnorm_rel(Sg, Sr, 2), elem_rel(zg, zr)
    print("%s: y abs %.2e y rel %.2e S rel %.2e z rel %.2e" % (label, ya, yr, sr, zrel))
    assert ya <= BF16_Y_ABS and sr <= BF16_STATE_REL and zrel <= BF16_STATE_REL, (label, ya, sr, zrel)
    # tighter internal expectation from bf16 operand rounding
    assert yr <= Y_MAXNORM_REL and sr <= 5e-3 and zrel <= Z_REL, (label, yr, sr, zrel)


CASES = [
    # B, H, T, chunk, gated, with_state   (B*H and T set the segment count: one segment per
    # sequence from 256 sequences up, up to 256 / (B*H) segments below)
    (1, 2, 1, 64, False, False),
    (1, 2, 63, 64, False, True),
    (1, 2, 200, 64, True, False),
    (1, 3, 257, 128, True, True),
    (1, 8, 130, 64, False, True),
    (2, 4, 129, 128, False, False),
    (1, 64, 96, 64, True, True),
    (2, 32, 70, 128, False, True),
    (1, 128, 65, 64, False, False),
    (1, 128, 190, 128, True, True),
    # long enough for several segments (segment scan path)
    (1, 2, 2000, 64, False, True),
    (1, 2, 2100, 64, True, True),
    (1, 3, 1999, 128, True, True),
    (1, 4, 1600, 128, False, False),
    (2, 8, 700, 64, True, False),
    (1, 16, 1300, 128, True, True),
    # more segments than the scan reads in one batch
    (1, 1, 4000, 64, True, True),
    (1, 1, 5000, 128, False, True),
    # chunk 128 at its edges: one token, one chunk short of full and exactly full, and
    # several segments of whole and of ragged chunks
    (1, 2, 1, 128, True, True),
    (1, 2, 127, 128, True, False),
    (1, 2, 128, 128, False, True),
    (1, 2, 2048, 128, False, True),
    (1, 2, 2049, 128, True, True),
]


@pytest.mark.parametrize("case", CASES)
def test_mfma_prefill_parity(torch, case):
    B, H, T, chunk, gated, with_state = case
    assert la.la_prefill_variant(la.LA_BF16, D, D, chunk, gated, la.LA_F32) == 1
    Q, K, V, alpha, S0, z0 = _inputs(torch, B, H, T, gated, with_state, 7 * T + H)
    Y, S, z = _run(torch, Q, K, V, alpha, chunk, S0, z0)
    _check(Y, S, z, oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0), str(case))


@pytest.mark.parametrize("chunk,T", [(64, 300), (128, 300), (64, 2100), (128, 2100)])
def test_mfma_zero_gates_reset(torch, chunk, T):
    """Zero gates wipe the state.  At T=2100 the sequence runs in several segments: zero gates
    fall inside segments and on the first token of a segment (640 at chunk 64, where segments
    are 320 tokens; 768 at chunk 128, where they are 384), so segment maps with G = 0 pass
    through the segment scan."""
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 2, T, True, True, 99 if T == 300 else 99 + T + chunk,
                                     zero_gates=True)
    if T > 1000:
        alpha[..., 640] = 0.0
        alpha[..., 768] = 0.0
    Y, S, z = _run(torch, Q, K, V, alpha, chunk, S0, z0)
    _check(Y, S, z, oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0), "zero gates chunk=%d T=%d" % (chunk, T))


@pytest.mark.parametrize("chunk,T", [(64, 300), (128, 300), (64, 2000), (128, 2100)])
def test_mfma_tiny_gates(torch, chunk, T):
    """Gates spread from about 1 down to the fp32 subnormal range (sigmoid of N(0, 30), a few
    exactly 0): the in-chunk log sums reach thousands below zero, the exponentials above
    the diagonal overflow and must be discarded, and products of gates underflow."""
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 2, T, True, True, 31 + T + chunk)
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + T + chunk)
    alpha = torch.sigmoid(torch.randn(alpha.shape, generator=g, device="cuda") * 30.0)
    assert float(alpha.min()) < 1e-30 and float(alpha.max()) > 0.999
    Y, S, z = _run(torch, Q, K, V, alpha, chunk, S0, z0)
    _check(Y, S, z, oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0), "tiny gates chunk=%d T=%d" % (chunk, T))


def test_mfma_causality_bitwise(torch):
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 2, 256, True, True, 5)
    Y1, _, _ = _run(torch, Q, K, V, alpha, 64, S0, z0)
    Q2, K2, V2, a2 = Q.clone(), K.clone(), V.clone(), alpha.clone()
    Q2[:, :, 130:] *= -3
    K2[:, :, 130:] += 1.0
    V2[:, :, 130:] = 5.0
    a2[:, :, 130:] = 0.25
    Y2, _, _ = _run(torch, Q2, K2, V2, a2, 64, S0, z0)
    assert torch.equal(Y1[:, :, :130], Y2[:, :, :130])


def test_mfma_chunk_invariance(torch):
    """chunk changes only the rounding: 64 and 128 agree within the bf16 operand error."""
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 4, 500, True, True, 6)
    Ya, Sa, za = _run(torch, Q, K, V, alpha, 64, S0, z0)
    Yb, Sb, zb = _run(torch, Q, K, V, alpha, 128, S0, z0)
    assert max_abs(to_f64(Ya), to_f64(Yb)) < 2e-2
    assert maxnorm_rel(to_f64(Sa), to_f64(Sb), 2) < 5e-3
    assert elem_rel(to_f64(za), to_f64(zb)) < 2 * Z_REL  # each side within Z_REL of exact


def test_mfma_deterministic(torch):
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 8, 300, True, True, 8)
    r1 = _run(torch, Q, K, V, alpha, 128, S0, z0)
    r2 = _run(torch, Q, K, V, alpha, 128, S0, z0)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("chunk,gated", [(64, False), (64, True), (128, True)])
def test_mfma_unaligned_state_bitwise(torch, chunk, gated):
    """S and z that are 4- but not 16-byte aligned give the aligned results bit for bit
    (several segments, so the entering states go through the segment scan)."""
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 2, 2048, gated, True, 12)
    Y, S, z = _run(torch, Q, K, V, alpha, chunk, S0, z0)
    nS, nz = S0.numel(), z0.numel()
    buf = torch.empty(1 + nS + 1 + nz, device="cuda")
    Su = buf[1:1 + nS].view(S0.shape)
    zu = buf[2 + nS:2 + nS + nz].view(z0.shape)
    assert Su.data_ptr() % 16 != 0 and zu.data_ptr() % 16 != 0
    Su.copy_(S0)
    zu.copy_(z0)
    Yu = torch.empty_like(V)
    la.la_prefill_chunked(Q, K, V, alpha, 1e-6, chunk, Yu, Su, zu)
    torch.cuda.synchronize()
    assert torch.equal(Yu, Y) and torch.equal(Su, S) and torch.equal(zu, z)


def test_mfma_resume_matches_single_call(torch):
    """Prefill of 192 tokens then 100 more from the returned state = one call of 292 (to rounding)."""
    Q, K, V, alpha, S0, z0 = _inputs(torch, 1, 2, 292, True, True, 10)
    Y, S, z = _run(torch, Q, K, V, alpha, 64, S0, z0)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    Ya, Sa, za = _run(torch, sl(Q, 0, 192), sl(K, 0, 192), sl(V, 0, 192), sl(alpha, 0, 192), 64, S0, z0)
    Yb, Sb, zb = _run(torch, sl(Q, 192, 292), sl(K, 192, 292), sl(V, 192, 292), sl(alpha, 192, 292), 64, Sa, za)
    assert torch.equal(torch.cat([Ya, Yb], dim=2), Y)
    assert torch.equal(Sb, S) and torch.equal(zb, z)


def test_worked_examples_at_width_128(torch):
    """The page's examples embedded at d = dv = 128: features 0, 1, 2 come from raw
    inputs -inf, 0, 1 (exact through ELU+1 and bf16); padded features are -inf and
    padded values 0, which leaves S, z and y unchanged.  Exercise 1: S = [[5,3],[7,5]],
    z = [2,2], y3 = [17/6, 11/6]; 2-D example y2 = [8/3, 5/3]."""
    inf = math.inf
    q = torch.full((1, 1, 3, D), -inf)
    k = torch.full((1, 1, 3, D), -inf)
    v = torch.zeros((1, 1, 3, D))
    q[0, 0, :, 0], q[0, 0, :, 1] = 1.0, 0.0            # phi(q) = [2, 1]
    k[0, 0, 0, 0], k[0, 0, 1, 1] = 0.0, 0.0            # phi(k1) = [1, 0], phi(k2) = [0, 1]
    k[0, 0, 2, 0], k[0, 0, 2, 1] = 0.0, 0.0            # phi(k3) = [1, 1]
    v[0, 0, :, :2] = torch.tensor([[2.0, 1.0], [4.0, 3.0], [3.0, 2.0]])
    bf = lambda t: t.to(torch.bfloat16).cuda()
    for chunk in (64, 128):
        Y, S, z = _run(torch, bf(q), bf(k), bf(v), None, chunk, eps=0.0)
        S, z, Y = S[0, 0].cpu(), z[0, 0].cpu(), Y[0, 0].float().cpu()
        assert torch.equal(S[:2, :2], torch.tensor([[5.0, 3.0], [7.0, 5.0]]))
        assert (S[2:] == 0).all() and (S[:, 2:] == 0).all()
        assert torch.equal(z[:2], torch.tensor([2.0, 2.0])) and (z[2:] == 0).all()
        for t, want in ((1, [8 / 3, 5 / 3]), (2, [17 / 6, 11 / 6])):
            for c in range(2):
                # the output is rounded once to bf16 (8 significant bits)
                assert abs(Y[t, c].item() - want[c]) <= 2.0 ** -8 * abs(want[c])
        assert (Y[:, 2:] == 0).all()


def test_gated_walkthrough_at_width_128(torch):
    """Gate 0.5 at every step, features 1, values 2, 4, 8: S = 2, 5, 10.5, z = 1, 1.5, 1.75
    (checked through the outputs and the final state)."""
    inf = math.inf
    q = torch.full((1, 1, 3, D), -inf)
    k = torch.full((1, 1, 3, D), -inf)
    q[..., 0] = 0.0
    k[..., 0] = 0.0
    v = torch.zeros((1, 1, 3, D))
    v[0, 0, :, 0] = torch.tensor([2.0, 4.0, 8.0])
    alpha = torch.full((1, 1, 3), 0.5).cuda()
    bf = lambda t: t.to(torch.bfloat16).cuda()
    for chunk in (64, 128):
        Y, S, z = _run(torch, bf(q), bf(k), bf(v), alpha, chunk, eps=0.0)
        assert abs(S[0, 0, 0, 0].item() - 10.5) < 1e-5 and abs(z[0, 0, 0].item() - 1.75) < 1e-6
        y = Y[0, 0, :, 0].float().cpu()
        for got, want in zip(y.tolist(), [2.0, 10 / 3, 6.0]):
            assert abs(got - want) <= 2.0 ** -8 * want


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_underflowing_query_row(torch, io, chunk):
    """One query row of -200 in every feature: ELU+1 = exp(x) underflows to 0 in fp32 for all
    of them.  With eps > 0 that output is exactly 0 (the FP64 value is below 1e-70); with
    eps = 0 it is 0 / 0 = NaN, as linattn.h states.  Every other output keeps parity."""
    B, H, T, j = 1, 2, 300, 77
    g = torch.Generator(device="cuda")
    g.manual_seed(515 + chunk)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    mk = lambda: (torch.randn((B, H, T, D), generator=g, device="cuda") / math.sqrt(128)).to(dt)
    Q, K, V = mk(), mk(), mk()
    Q[:, :, j, :] = -200.0
    others = [t for t in range(T) if t != j]
    for eps in (1e-6, 0.0):
        Y, S, z = _run(torch, Q, K, V, None, chunk, eps=eps)
        Yr, Sr, zr, _ = oracle_prefill(Q, K, V, None, eps)
        Yg = to_f64(Y)
        if eps > 0:
            assert (Yg[:, :, j] == 0).all() and np.abs(Yr[:, :, j]).max() < 1e-70
        else:
            assert np.isnan(Yg[:, :, j]).all()
        assert np.isfinite(Yg[:, :, others]).all()
        if io == "bf16":
            assert max_abs(Yg[:, :, others], Yr[:, :, others]) <= BF16_Y_ABS
            assert maxnorm_rel(to_f64(S), Sr, 2) <= 5e-3 and elem_rel(to_f64(z), zr) <= Z_REL
        else:
            assert maxnorm_rel(Yg[:, :, others], Yr[:, :, others], 2) <= 1e-4
            assert maxnorm_rel(to_f64(S), Sr, 2) <= 1e-4 and elem_rel(to_f64(z), zr) <= 1e-4
