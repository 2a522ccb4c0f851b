"""HIP graph capture of the library's launches: la_state_init + la_prefill_chunked
(the three-pass bf16 MFMA path and the general path) and a chain of la_decode_step
calls are captured once on a side stream and replayed several times, with eager work
and synchronisations between the replays; every replay must reproduce the eager
results bitwise (the library records no memset nodes: state init is a fill kernel)."""
import math

import pytest

import recurrent_state_chunkwise_amd as la

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _prefill_inputs(torch, B, H, T, d, dv, dtype, gated, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sc = 1 / math.sqrt(128)
    Q = (torch.randn((B, H, T, d), generator=g, device="cuda") * sc).to(dtype)
    K = (torch.randn((B, H, T, d), generator=g, device="cuda") * sc).to(dtype)
    V = (torch.randn((B, H, T, dv), generator=g, device="cuda") * sc).to(dtype)
    A = torch.sigmoid(torch.randn((B, H, T), generator=g, device="cuda") + 3.0) if gated else None
    return Q, K, V, A


@pytest.mark.parametrize("case", [
    (1, 2, 1500, 128, 128, "bf16", 64, False),   # segment maps + scan + chunked prefill
    (1, 2, 700, 128, 128, "bf16", 128, True),
    (2, 2, 90, 16, 24, "f32", 16, True),         # general kernel
], ids=["mfma_c64", "mfma_c128_gated", "general_f32"])
def test_prefill_graph_replays(torch, case):
    B, H, T, d, dv, dt, chunk, gated = case
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    Q, K, V, A = _prefill_inputs(torch, B, H, T, d, dv, dtype, gated, 41)
    Y = torch.empty_like(V)
    S = torch.empty((B, H, d, dv), device="cuda")
    z = torch.empty((B, H, d), device="cuda")

    def run():
        la.la_state_init(S, z)
        la.la_prefill_chunked(Q, K, V, A, 1e-6, chunk, Y, S, z)

    run()
    torch.cuda.synchronize()
    ref = (Y.clone(), S.clone(), z.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        # eager work between replays: scribble over the outputs
        Y.fill_(7.0)
        S.fill_(-3.0)
        z.fill_(11.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref[0]) and torch.equal(S, ref[1]) and torch.equal(z, ref[2]), ("replay", rep)


def test_decode_graph_replays(torch):
    N, d, dv, steps = 200, 128, 128, 4
    g = torch.Generator(device="cuda")
    g.manual_seed(43)
    sc = 1 / math.sqrt(128)
    qs = [(torch.randn((N, d), generator=g, device="cuda") * sc).to(torch.bfloat16) for _ in range(steps)]
    ks = [(torch.randn((N, d), generator=g, device="cuda") * sc).to(torch.bfloat16) for _ in range(steps)]
    vs = [(torch.randn((N, dv), generator=g, device="cuda") * sc).to(torch.bfloat16) for _ in range(steps)]
    S0 = torch.randn((N, d, dv), generator=g, device="cuda") * 0.05
    z0 = torch.rand((N, d), generator=g, device="cuda") * 10 + 1
    S, z = S0.clone(), z0.clone()
    ys = [torch.empty((N, dv), device="cuda", dtype=torch.bfloat16) for _ in range(steps)]

    def run():
        for t in range(steps):
            la.la_decode_step(qs[t], ks[t], vs[t], None, 1e-6, ys[t], S, z)

    run()
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys] + [S.clone(), z.clone()]

    S.copy_(S0)
    z.copy_(z0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        S.copy_(S0)  # eager work between replays: reset the state, scribble over the outputs
        z.copy_(z0)
        for y in ys:
            y.fill_(5.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [y for y in ys] + [S, z]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), ("replay", rep)
