"""GPU parity of the general kernels (state init, general chunked prefill, decode)
against the FP64 oracle, called through the C ABI."""
import math

import numpy as np
import pytest

import oracle
import recurrent_state_chunkwise_amd as la
from recurrent_state_chunkwise_amd import workloads as wl

from helpers import assert_prefill_parity, elem_rel, maxnorm_rel, oracle_prefill, to_f64, F32_REL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _run_prefill(torch, Q, K, V, alpha, eps, chunk, S0=None, z0=None):
    B, H, T, d = Q.shape
    dv = V.shape[-1]
    st = torch.float64 if Q.dtype == torch.float64 else torch.float32
    Y = torch.empty_like(V)
    S = torch.empty((B, H, d, dv), device=Q.device, dtype=st)
    z = torch.empty((B, H, d), device=Q.device, dtype=st)
    if S0 is None:
        la.la_state_init(S, z)
    else:
        S.copy_(S0)
        z.copy_(z0)
    la.la_prefill_chunked(Q, K, V, alpha, eps, chunk, Y, S, z)
    torch.cuda.synchronize()
    return Y, S, z


def test_state_init(torch):
    for dt in (torch.float32, torch.float64):
        S = torch.full((3, 5, 7), 3.0, device="cuda", dtype=dt)
        z = torch.full((3, 5), 3.0, device="cuda", dtype=dt)
        la.la_state_init(S, z)
        torch.cuda.synchronize()
        assert (S == 0).all() and (z == 0).all()
    # an unaligned view of a larger buffer: only the view is cleared
    buf = torch.full((1 + 2 * 3 * 4 + 2 * 3 + 1,), 7.0, device="cuda", dtype=torch.float32)
    S = buf[1:1 + 24].view(2, 3, 4)
    z = buf[1 + 24:1 + 24 + 6].view(2, 3)
    la.la_state_init(S, z)
    torch.cuda.synchronize()
    h = buf.cpu()
    assert h[0] == 7.0 and h[-1] == 7.0 and (h[1:-1] == 0).all()
    # both ranges span many blocks, each with an unaligned head and a tail
    n, r, dv = 1000, 33, 17
    buf = torch.full((1 + n * r * dv + n * r + 1,), 7.0, device="cuda", dtype=torch.float32)
    S = buf[1:1 + n * r * dv].view(n, r, dv)
    z = buf[1 + n * r * dv:1 + n * r * dv + n * r].view(n, r)
    la.la_state_init(S, z)
    torch.cuda.synchronize()
    h = buf.cpu()
    assert h[0] == 7.0 and h[-1] == 7.0 and (h[1:-1] == 0).all()


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
def test_single_head_f64(torch, chunk):
    """The single-head FP64 workload (B=1, H=1, T=64, d=dv=16) at several chunk sizes."""
    cfg = wl.SINGLE_HEAD_F64
    Q, K, V, _ = wl.prefill_inputs(cfg, "cuda")
    Y, S, z = _run_prefill(torch, Q, K, V, None, cfg.eps, chunk)
    ref = oracle_prefill(Q, K, V, None, cfg.eps)
    m = assert_prefill_parity(Y, S, z, ref, "f64", "chunk=%d" % chunk)
    print("single_head_f64 chunk=%d" % chunk, m)


GENERAL_CASES = [
    # B, H, T, d, dv, chunk, gated, with_state
    (1, 2, 37, 16, 16, 8, False, False),
    (2, 3, 100, 32, 24, 16, True, True),
    (1, 1, 1, 5, 3, 4, True, True),
    (1, 2, 200, 128, 128, 48, False, True),
    (1, 2, 300, 128, 128, 128, True, False),
    (2, 1, 129, 64, 40, 32, True, True),
    (1, 1, 65, 128, 17, 3, False, False),
]


def _case_inputs(torch, B, H, T, d, dv, gated, with_state, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    st = torch.float64 if dtype == torch.float64 else torch.float32
    Q = torch.randn((B, H, T, d), generator=g, device="cuda", dtype=torch.float32).mul_(0.7).to(dtype)
    K = torch.randn((B, H, T, d), generator=g, device="cuda", dtype=torch.float32).mul_(0.7).to(dtype)
    V = torch.randn((B, H, T, dv), generator=g, device="cuda", dtype=torch.float32).to(dtype)
    alpha = None
    if gated:
        alpha = torch.sigmoid(torch.randn((B, H, T), generator=g, device="cuda") + 2.0).to(st)
        alpha[..., T // 2] = 0.0
        if T > 3:
            alpha[..., 1] = 1.0
    S0 = z0 = None
    if with_state:
        S0 = torch.randn((B, H, d, dv), generator=g, device="cuda", dtype=torch.float32).to(st)
        z0 = torch.rand((B, H, d), generator=g, device="cuda", dtype=torch.float32).add_(0.5).to(st)
    return Q, K, V, alpha, S0, z0


@pytest.mark.parametrize("case", GENERAL_CASES)
@pytest.mark.parametrize("io", ["f32", "f64", "bf16"])
def test_general_prefill_parity(torch, case, io):
    B, H, T, d, dv, chunk, gated, with_state = case
    dtype = wl.torch_dtype(io)
    code = {"f32": la.LA_F32, "f64": la.LA_F64, "bf16": la.LA_BF16}[io]
    state = la.LA_F64 if io == "f64" else la.LA_F32
    if la.la_prefill_variant(code, d, dv, chunk, gated, state) != 0:
        pytest.skip("this shape runs an MFMA kernel (covered by its own tests)")
    Q, K, V, alpha, S0, z0 = _case_inputs(torch, B, H, T, d, dv, gated, with_state, dtype, 1000 + T + d)
    Y, S, z = _run_prefill(torch, Q, K, V, alpha, 1e-6, chunk, S0, z0)
    ref = oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0)
    bar = {"f32": "f32", "f64": "f64", "bf16": "f32"}[io]
    if io == "bf16":
        # the general kernel computes in fp32 on the exact bf16 inputs; only Y is rounded
        Yr, Sr, zr, _ = ref
        assert maxnorm_rel(to_f64(S), Sr, 2) <= F32_REL and elem_rel(to_f64(z), zr) <= F32_REL
        assert np.abs(to_f64(Y) - Yr).max() <= 2e-2
        assert maxnorm_rel(to_f64(Y), Yr, 2) <= 1e-2
    else:
        assert_prefill_parity(Y, S, z, ref, bar, str(case))


@pytest.mark.parametrize("form,gated", [("causal", False), ("causal", True), ("noncausal", False)])
def test_general_many_sequences_nonzero_state(torch, form, gated):
    """f32, d = dv = 128, 2,048 sequences with a nonzero incoming S and z: 8,192 workgroups
    (sequence x value slice), more than the GPU holds at once, so the slices of one sequence
    start at different times.  Every slice must read the caller's z, and the final z must
    be written only after all of them have read it."""
    from helpers import oracle_noncausal
    B, H, T, d, dv = 16, 128, 24, 128, 128
    Q, K, V, alpha, S0, z0 = _case_inputs(torch, B, H, T, d, dv, gated, True, torch.float32, 4242)
    if form == "causal":
        Y, S, z = _run_prefill(torch, Q, K, V, alpha, 1e-6, 16, S0, z0)
        ref = oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0)
    else:
        Y, S, z = torch.empty_like(V), S0.clone(), z0.clone()
        la.la_prefill_noncausal(Q, K, V, 1e-6, Y, S, z)
        torch.cuda.synchronize()
        ref = oracle_noncausal(Q, K, V, 1e-6, S0, z0)
    m = assert_prefill_parity(Y, S, z, ref, "f32", "%s gated=%s" % (form, gated))
    print("many sequences", form, gated, m)


def test_general_prefill_causality_bitwise(torch):
    """Changing later tokens leaves earlier outputs bit-identical."""
    Q, K, V, alpha, S0, z0 = _case_inputs(torch, 1, 2, 90, 32, 16, True, True, torch.float32, 77)
    Y1, _, _ = _run_prefill(torch, Q, K, V, alpha, 1e-6, 16, S0, z0)
    K2, V2, Q2, a2 = K.clone(), V.clone(), Q.clone(), alpha.clone()
    K2[:, :, 50:] += 100.0
    V2[:, :, 50:] -= 30.0
    Q2[:, :, 50:] *= -2.0
    a2[:, :, 50:] = 0.3
    Y2, _, _ = _run_prefill(torch, Q2, K2, V2, a2, 1e-6, 16, S0, z0)
    assert torch.equal(Y1[:, :, :50], Y2[:, :, :50])


def test_general_prefill_resume(torch):
    """Prefill of T1 tokens then T2 more from the returned state matches one call of T1+T2."""
    Q, K, V, alpha, S0, z0 = _case_inputs(torch, 1, 2, 150, 48, 32, True, True, torch.float64, 78)
    Y, S, z = _run_prefill(torch, Q, K, V, alpha, 1e-6, 32, S0, z0)
    Ya, Sa, za = _run_prefill(torch, Q[:, :, :70].contiguous(), K[:, :, :70].contiguous(),
                              V[:, :, :70].contiguous(), alpha[:, :, :70].contiguous(), 1e-6, 32, S0, z0)
    Yb, Sb, zb = _run_prefill(torch, Q[:, :, 70:].contiguous(), K[:, :, 70:].contiguous(),
                              V[:, :, 70:].contiguous(), alpha[:, :, 70:].contiguous(), 1e-6, 32, Sa, za)
    assert maxnorm_rel(to_f64(torch.cat([Ya, Yb], dim=2)), to_f64(Y), 2) < 1e-12
    assert maxnorm_rel(to_f64(Sb), to_f64(S), 2) < 1e-12


def _decode_case(torch, N, d, dv, gated, io, steps, seed):
    dtype = wl.torch_dtype(io)
    st = wl.state_dtype(io)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    S = torch.randn((N, d, dv), generator=g, device="cuda", dtype=torch.float32).to(st)
    z = torch.rand((N, d), generator=g, device="cuda", dtype=torch.float32).add_(0.5).to(st)
    S0, z0 = S.clone(), z.clone()
    qs, ks, vs, As, ys = [], [], [], [], []
    for _ in range(steps):
        q = torch.randn((N, d), generator=g, device="cuda", dtype=torch.float32).mul_(0.5).to(dtype)
        k = torch.randn((N, d), generator=g, device="cuda", dtype=torch.float32).mul_(0.5).to(dtype)
        v = torch.randn((N, dv), generator=g, device="cuda", dtype=torch.float32).to(dtype)
        a = torch.sigmoid(torch.randn((N,), generator=g, device="cuda") + 1.0).to(st) if gated else None
        y = torch.empty((N, dv), device="cuda", dtype=dtype)
        la.la_decode_step(q, k, v, a, 1e-6, y, S, z)
        qs.append(q), ks.append(k), vs.append(v), As.append(a), ys.append(y)
    torch.cuda.synchronize()
    # the oracle sees each state's steps as one sequence of `steps` tokens
    Q = np.stack([to_f64(x) for x in qs], axis=1)
    K = np.stack([to_f64(x) for x in ks], axis=1)
    Vv = np.stack([to_f64(x) for x in vs], axis=1)
    A = np.stack([to_f64(x) for x in As], axis=1) if gated else None
    Yr, Sr, zr, _ = oracle.recurrence_heads(Q, K, Vv, A, eps=1e-6, S0=to_f64(S0), z0=to_f64(z0), threads=8)
    Yg = np.stack([to_f64(x) for x in ys], axis=1)
    return Yg, to_f64(S), to_f64(z), Yr, Sr, zr


@pytest.mark.parametrize("io", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("shape", [(300, 128, 128), (130, 64, 64), (77, 40, 24), (5, 1, 1), (64, 128, 7)])
@pytest.mark.parametrize("gated", [False, True])
def test_decode_parity(torch, io, shape, gated):
    N, d, dv = shape
    Yg, Sg, zg, Yr, Sr, zr = _decode_case(torch, N, d, dv, gated, io, 5, 500 + N + d)
    tol = 1e-12 if io == "f64" else F32_REL
    assert maxnorm_rel(Sg, Sr, 2) <= tol
    assert elem_rel(zg, zr) <= tol
    if io == "bf16":
        assert np.abs(Yg - Yr).max() <= 2e-2 and maxnorm_rel(Yg, Yr, 1) <= 1e-2
    else:
        assert maxnorm_rel(Yg, Yr, 1) <= tol


def test_worked_examples_through_f64_prefill(torch):
    """Page values through the device (f64, ELU+1 on exact preimages -inf, 0, 1, 2):
    exercise 1 gives S = [[5,3],[7,5]], z = [2,2], y3 = [17/6, 11/6]; the gated
    walk-through ends at S = 10.5, z = 1.75; exercise 2 gives y3 = 74/11."""
    inf = math.inf

    def run(q, k, v, alpha, chunk):
        t = lambda a: torch.tensor(a, dtype=torch.float64, device="cuda")[None, None]
        Y, S, z = _run_prefill(torch, t(q), t(k), t(v), None if alpha is None else t(alpha), 0.0, chunk)
        return Y[0, 0].cpu().numpy(), S[0, 0].cpu().numpy(), z[0, 0].cpu().numpy()

    for chunk in (1, 2, 3):
        # phi(x): -inf -> 0, 0 -> 1, 1 -> 2
        Y, S, z = run([[1, 0]] * 3, [[0, -inf], [-inf, 0], [0, 0]], [[2, 1], [4, 3], [3, 2]], None, chunk)
        assert np.allclose(S, [[5, 3], [7, 5]], rtol=0, atol=1e-15) and np.allclose(z, [2, 2], rtol=0, atol=1e-15)
        assert np.allclose(Y[1], [8 / 3, 5 / 3], rtol=1e-15) and np.allclose(Y[2], [17 / 6, 11 / 6], rtol=1e-15)
        Y, S, z = run([[0]] * 3, [[0]] * 3, [[2], [4], [8]], [0.5, 0.5, 0.5], chunk)
        assert abs(S[0, 0] - 10.5) < 1e-14 and abs(z[0] - 1.75) < 1e-15 and abs(Y[0, 0] - 2) < 1e-15
        Y, S, z = run([[0]] * 3, [[0]] * 3, [[2], [4], [8]], [1.0, 0.5, 0.25], chunk)
        assert abs(Y[2, 0] - 74 / 11) < 1e-14
