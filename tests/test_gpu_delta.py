"""GPU parity of the delta-rule decode step (la_delta_decode_step) against the FP64
oracle (oracle.delta_steps), through the C ABI: the page's worked examples embedded in
128 x 128 memories (exact), both kernel paths (d = dv = 128 and other widths) in every
dtype pair over several steps, and sampled memories of the full 65,536-memory workload."""
import numpy as np
import pytest

import oracle
import recurrent_state_chunkwise_amd as la
from recurrent_state_chunkwise_amd import workloads as wl

from helpers import max_abs, maxnorm_rel, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _run_steps(torch, q, k, v, beta, S):
    """q, k: [T, N, d]; v: [T, N, dv]; beta: [T, N]; S: [N, d, dv] updated in place.
    Returns y [T, N, dv]."""
    T, N, _ = q.shape
    ys = []
    for t in range(T):
        y = torch.empty_like(v[t])
        la.la_delta_decode_step(q[t], k[t], v[t], beta[t], y, S)
        ys.append(y)
    torch.cuda.synchronize()
    return torch.stack(ys)


def _oracle(q, k, v, beta, S0):
    Q = np.transpose(to_f64(q), (1, 0, 2))
    K = np.transpose(to_f64(k), (1, 0, 2))
    V = np.transpose(to_f64(v), (1, 0, 2))
    B = np.transpose(to_f64(beta), (1, 0))
    Y, S = oracle.delta_steps_states(Q, K, V, B, to_f64(S0), threads=8)
    return np.transpose(Y, (1, 0, 2)), S


def _one_hot_key(torch, io, scale=1.0):
    k = torch.zeros(1, 128, dtype=io, device="cuda")
    k[0, 0] = scale
    return k


@pytest.mark.parametrize("io_name", ["bf16", "f32"])
def test_delta_worked_examples_at_width_128(torch, io_name):
    io = wl.torch_dtype(io_name)
    # two orthogonal keys answering 2 and 4; write 5 for the first with beta 1/2 -> 7/2, 4 stays
    S = torch.zeros(1, 128, 128, device="cuda")
    S[0, 0, 0], S[0, 1, 0] = 2.0, 4.0
    k = _one_hot_key(torch, io)
    v = torch.zeros(1, 128, dtype=io, device="cuda")
    v[0, 0] = 5.0
    beta = torch.tensor([0.5], device="cuda")
    y = torch.empty_like(v)
    la.la_delta_decode_step(k, k, v, beta, y, S)
    torch.cuda.synchronize()
    assert S[0, 0, 0].item() == 3.5 and S[0, 1, 0].item() == 4.0 and y[0, 0].item() == 3.5
    assert S[0, 2:].abs().max().item() == 0.0 and S[0, :, 1:].abs().max().item() == 0.0
    # the same key three times from memory 2: 7/2, 17/4, 37/8
    S = torch.zeros(1, 128, 128, device="cuda")
    S[0, 0, 0] = 2.0
    got = []
    for _ in range(3):
        la.la_delta_decode_step(k, k, v, beta, y, S)
        got.append(S[0, 0, 0].item())
    assert got == [3.5, 4.25, 4.625]
    # exercise 3: key 2, memory 1, target 5: beta 1/2 overshoots to 8, beta 1/4 lands on 5
    k2 = _one_hot_key(torch, io, 2.0)
    for b, s_new, pred in ((0.5, 4.0, 8.0), (0.25, 2.5, 5.0)):
        S = torch.zeros(1, 128, 128, device="cuda")
        S[0, 0, 0] = 1.0
        la.la_delta_decode_step(k2, k2, v, torch.tensor([b], device="cuda"), y, S)
        torch.cuda.synchronize()
        assert S[0, 0, 0].item() == s_new and y[0, 0].item() == pred


CASES = [
    # io, d, dv  (d = dv = 128 takes the streaming kernel; other widths the general one)
    ("bf16", 128, 128), ("f32", 128, 128), ("f64", 128, 128),
    ("bf16", 48, 80), ("f32", 1, 128), ("f64", 100, 7),
]


@pytest.mark.parametrize("io_name,d,dv", CASES)
def test_delta_parity_small(torch, io_name, d, dv):
    io, st = wl.torch_dtype(io_name), wl.state_dtype(io_name)
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + d + dv)
    T, N = 12, 6
    k = torch.randn((T, N, d), generator=g, device="cuda", dtype=torch.float64)
    k = (k / k.norm(dim=2, keepdim=True)).to(io)
    q = (torch.randn((T, N, d), generator=g, device="cuda", dtype=torch.float64) / np.sqrt(d)).to(io)
    v = torch.randn((T, N, dv), generator=g, device="cuda", dtype=torch.float64).to(io)
    beta = torch.sigmoid(torch.randn((T, N), generator=g, device="cuda", dtype=torch.float64)).to(st)
    S0 = (torch.randn((N, d, dv), generator=g, device="cuda", dtype=torch.float64) * 0.1).to(st)
    S = S0.clone()
    Y = _run_steps(torch, q, k, v, beta, S)
    Yr, Sr = _oracle(q, k, v, beta, S0)
    Yg, Sg = to_f64(Y), to_f64(S)
    assert np.isfinite(Yg).all() and np.isfinite(Sg).all()
    ys, ss = maxnorm_rel(Yg, Yr, 2), maxnorm_rel(Sg, Sr, 2)
    print("%s d=%d dv=%d: y max-norm rel %.2e (abs %.2e)  S max-norm rel %.2e" % (io_name, d, dv, ys, max_abs(Yg, Yr), ss))
    if io_name == "f64":
        assert ys <= 1e-11 and ss <= 1e-11
    elif io_name == "f32":
        assert ys <= 1e-4 and ss <= 1e-4
    else:
        # bf16 inputs are exact in both; the fp32 state carries fp32 rounding, y is rounded to bf16
        assert max_abs(Yg, Yr) <= 2e-2 and ss <= 1e-2
        assert ys <= 2.0 ** -8 + 1e-4 and ss <= 1e-5


def test_delta_full_workload_sampled(torch):
    """65,536 memories of 128 x 128, 32 steps; 512 sampled memories against the oracle at
    every step and at the end."""
    cfg = wl.DELTA_DECODE
    N, T = cfg.n_states, 32
    S = wl.delta_seed_state(cfg, "cuda")
    picks = torch.from_numpy(wl.sampled_states(cfg, 512)).cuda()
    S0 = S[picks].clone()
    qs, ks, vs, bs, ys = [], [], [], [], []
    y = torch.empty((N, cfg.dv), device="cuda", dtype=torch.bfloat16)
    for t in range(T):
        q, k, v, b = wl.delta_step_inputs(cfg, t, "cuda")
        la.la_delta_decode_step(q, k, v, b, y, S)
        qs.append(q[picks]); ks.append(k[picks]); vs.append(v[picks]); bs.append(b[picks]); ys.append(y[picks].clone())
    torch.cuda.synchronize()
    Yr, Sr = _oracle(torch.stack(qs), torch.stack(ks), torch.stack(vs), torch.stack(bs), S0)
    Yg, Sg = to_f64(torch.stack(ys)), to_f64(S[picks])
    ya, yr, sr = max_abs(Yg, Yr), maxnorm_rel(Yg, Yr, 2), maxnorm_rel(Sg, Sr, 2)
    print("delta workload (512 sampled memories, 32 steps): y abs %.2e  y max-norm rel %.2e  S rel %.2e" % (ya, yr, sr))
    assert ya <= 2e-2 and sr <= 1e-2
    assert yr <= 2.0 ** -8 + 1e-4 and sr <= 1e-5
