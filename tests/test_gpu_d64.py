"""GPU parity of the fp32-arithmetic MFMA chunked prefill at d = dv = 64 (chunk 64), with bf16
and with fp32 inputs, against the FP64 oracle through the C ABI: ragged lengths, one to many
segments per sequence, gates including zero gates, a carried state, the state builds of the
history-against-state comparison (8 and 1,024 sequences, 64 wide), and rows too misaligned
for the kernel, which take the general kernel.

Bars: fp32 inputs at 1e-4 (per-head max-norm relative on y and S, elementwise relative on z).
bf16 inputs at the bf16 bar, and, since every product runs on fp32 operands and y is rounded
to bf16 only when stored, at a tighter internal bound as well: S and z within the fp32 bar,
and every output within one bf16 rounding (2^-8 relative) plus the fp32 bar of its head's
largest output."""
import numpy as np
import pytest

import recurrent_state_chunkwise_amd as la

from helpers import BF16_U, F32_REL, assert_prefill_parity, oracle_prefill, to_f64

pytestmark = pytest.mark.gpu
D = 64


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _inputs(torch, io, B, H, T, gated, with_state, seed, zero_gates=False):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    mk = lambda s: (torch.randn((B, H, T, D), generator=g, device="cuda") * s).to(dt)
    Q, K, V = mk(0.7), mk(0.7), mk(1.0)
    alpha = None
    if gated:
        alpha = torch.sigmoid(torch.randn((B, H, T), generator=g, device="cuda") + 2.0)
        if zero_gates:
            alpha[..., T // 2] = 0.0
            alpha[..., 0] = 0.0
            if T > 500:
                alpha[..., 384] = 0.0  # a segment's first token: segments of 192 (bf16) or 128 (f32)
    S0 = z0 = None
    if with_state:
        S0 = torch.randn((B, H, D, D), generator=g, device="cuda") * 0.3
        z0 = torch.rand((B, H, D), generator=g, device="cuda") * 5.0 + 0.5
    return Q, K, V, alpha, S0, z0


def _run(torch, Q, K, V, alpha, S0, z0, eps=1e-6, Y=None):
    B, H, T, _ = Q.shape
    Y = torch.empty_like(V) if Y is None else Y
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


def _check(io, Y, S, z, ref, label):
    if io == "f32":
        return assert_prefill_parity(Y, S, z, ref, "f32", label)
    m = assert_prefill_parity(Y, S, z, ref, "bf16", label)
    assert m["S_maxnorm_rel"] <= F32_REL and m["z_rel"] <= F32_REL, (label, m)
    Yr = ref[0]
    Yg = to_f64(Y)
    head_max = np.abs(Yr).max(axis=(2, 3), keepdims=True)
    excess = np.abs(Yg - Yr) - (BF16_U * np.abs(Yr) + F32_REL * head_max)
    assert excess.max() <= 0, (label, float(excess.max()))
    return m


CASES = [
    # B, H, T, gated, with_state, zero_gates      (segments per sequence, bf16 / f32)
    (1, 2, 1, False, False, False),      # 1
    (1, 2, 63, True, True, False),       # 1, one partial chunk
    (1, 3, 200, True, False, True),      # 1, ragged
    (2, 4, 450, True, True, True),       # 2 / 3
    (1, 2, 1000, False, True, False),    # 5 / 7
    (1, 2, 1500, True, True, True),      # 7 / 11, zero gates inside and at a segment start
    (1, 1, 3000, True, True, False),     # 15 / 23: more maps than the scan reads in one batch
    (2, 64, 96, False, False, False),    # 1, 128 sequences
]


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES)
def test_d64_mfma_prefill_parity(torch, io, case):
    B, H, T, gated, with_state, zero_gates = case
    code = la.LA_BF16 if io == "bf16" else la.LA_F32
    assert la.la_prefill_variant(code, D, D, 64, gated, la.LA_F32) == 2
    Q, K, V, alpha, S0, z0 = _inputs(torch, io, B, H, T, gated, with_state, 37 * T + H, zero_gates)
    Y, S, z = _run(torch, Q, K, V, alpha, S0, z0)
    m = _check(io, Y, S, z, oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0), f"{io} {case}")
    print(io, case, la.la_prefill_segments(B * H, T, 64, code, D), m)


@pytest.mark.parametrize("heads,T", [(8, 8191), (1024, 2047)])
def test_d64_state_build_shapes(torch, heads, T):
    """The state builds of the history-against-state comparison: bf16 keys and values of
    8 heads x 8,191 rows (32 segments of 192) and of 1,024 heads x 2,047 rows (one segment),
    keys doubling as queries, from a zero state."""
    g = torch.Generator(device="cuda")
    g.manual_seed(heads + T)
    K = torch.randn((heads, 1, T, D), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((heads, 1, T, D), generator=g, device="cuda").to(torch.bfloat16)
    Y, S, z = _run(torch, K, K, V, None, None, None)
    m = _check("bf16", Y, S, z, oracle_prefill(K, K, V, None, 1e-6, threads=16), f"state build {heads}x{T}")
    print(heads, T, la.la_prefill_segments(heads, T, 64, la.LA_BF16, D), m)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_d64_misaligned_rows_take_general_kernel(torch, io):
    """Q, K, V and Y viewed 2 elements into their buffers (4 or 8 bytes: not 8 or 16 aligned)
    run the general kernel, with the same results within the bars."""
    B, H, T = 1, 2, 300
    Q, K, V, alpha, S0, z0 = _inputs(torch, io, B, H, T, True, True, 5150)
    def shifted(t):  # a copy of t that starts 2 elements into its allocation
        return torch.empty(t.numel() + 2, device="cuda", dtype=t.dtype)[2:].view(t.shape)

    Qs, Ks, Vs, Ys = shifted(Q).copy_(Q), shifted(K).copy_(K), shifted(V).copy_(V), shifted(V)
    assert Qs.data_ptr() % (16 if io == "f32" else 8) != 0
    Y, S, z = _run(torch, Qs, Ks, Vs, alpha, S0, z0, Y=Ys)
    ref = oracle_prefill(Q, K, V, alpha, 1e-6, S0, z0)
    assert_prefill_parity(Y, S, z, ref, "f32" if io == "f32" else "bf16", f"misaligned {io}")
