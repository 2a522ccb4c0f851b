"""GPU parity at the full sizes of the workloads, in the launch configuration the
benchmark times, against the FP64 oracle on the same seeded inputs.

* single head f64 (B=1, H=1, T=64, d=dv=16): every output (general kernel)
* ungated prefill B=4, H=16, T=4096: every output, final S and z
* gated prefill B=2, H=16, T=16384: every output, final S and z
* long gated prefill B=1, H=32, T=131072, chunk 128: 4 sampled heads in full,
  with the error-vs-position report (max |dy| and smallest denominator per window)
* batched decode, 65,536 states seeded by 256 writes, 1024 steps: sampled states
  (every step's output and the final state)
"""
import math
import os

import numpy as np
import pytest

import oracle
import recurrent_state_chunkwise_amd as la
from recurrent_state_chunkwise_amd import workloads as wl

from helpers import BF16_STATE_REL, BF16_Y_ABS, Y_MAXNORM_REL, Z_REL, elem_rel, max_abs, maxnorm_rel, to_f64

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    la.library()
    return _t


def _prefill(torch, cfg, Q, K, V, A):
    Y = torch.empty_like(V)
    st = wl.state_dtype(cfg.io)
    S = torch.empty((cfg.B, cfg.H, cfg.d, cfg.dv), device="cuda", dtype=st)
    z = torch.empty((cfg.B, cfg.H, cfg.d), device="cuda", dtype=st)
    la.la_state_init(S, z)
    la.la_prefill_chunked(Q, K, V, A, cfg.eps, cfg.chunk, Y, S, z)
    torch.cuda.synchronize()
    return Y, S, z


def _report(label, ya, yr, sr, zr):
    print("%s: y max abs %.3e  y max-norm rel %.3e  S rel %.3e  z rel %.3e" % (label, ya, yr, sr, zr), flush=True)


def test_single_head_f64_full(torch):
    cfg = wl.SINGLE_HEAD_F64
    Q, K, V, A = wl.prefill_inputs(cfg, "cuda")
    Y, S, z = _prefill(torch, cfg, Q, K, V, A)
    Yr, Sr, zr, _ = oracle.recurrence_heads(to_f64(Q), to_f64(K), to_f64(V), eps=cfg.eps)
    ya, yr = max_abs(to_f64(Y), Yr), maxnorm_rel(to_f64(Y), Yr, 2)
    sr, zrel = maxnorm_rel(to_f64(S), Sr, 2), elem_rel(to_f64(z), zr)
    _report(cfg.name, ya, yr, sr, zrel)
    assert yr <= 1e-11 and sr <= 1e-11 and zrel <= 1e-11


@pytest.mark.parametrize("name", ["prefill_ungated_b4_h16_t4096", "prefill_gated_b2_h16_t16384"])
def test_prefill_full_config(torch, name):
    cfg = wl.CONFIGS[name]
    assert la.la_prefill_variant(la.LA_BF16, cfg.d, cfg.dv, cfg.chunk, cfg.gated, la.LA_F32) == 1
    Q, K, V, A = wl.prefill_inputs(cfg, "cuda")
    Y, S, z = _prefill(torch, cfg, Q, K, V, A)
    Yr, Sr, zr, den = oracle.recurrence_heads(to_f64(Q), to_f64(K), to_f64(V),
                                              None if A is None else to_f64(A), eps=cfg.eps, threads=THREADS)
    Yg = to_f64(Y)
    ya, yr = max_abs(Yg, Yr), maxnorm_rel(Yg, Yr, 2)
    sr, zrel = maxnorm_rel(to_f64(S), Sr, 2), elem_rel(to_f64(z), zr)
    _report(cfg.name, ya, yr, sr, zrel)
    assert ya <= BF16_Y_ABS and sr <= BF16_STATE_REL and zrel <= BF16_STATE_REL
    assert yr <= Y_MAXNORM_REL and sr <= 5e-3 and zrel <= Z_REL


def test_prefill_long_sampled_heads(torch):
    """4 of the 32 heads of the long gated workload in full; error growth vs T.

    The oracle runs the 4 heads piecewise over [0, 2^10), [2^10, 2^12), ... [2^16, 2^17),
    each piece resuming from the state the previous one returned (the recurrence is
    sequential, so this is the same arithmetic as one run) and so also gives the state
    at every piece end T'.  The GPU state at T' comes from a prefill of the 4 heads'
    prefixes of length T' from a zero state (by causality the state after T' tokens
    depends on those tokens only)."""
    cfg = wl.PREFILL_LONG
    Q, K, V, A = wl.prefill_inputs(cfg, "cuda")
    Y, S, z = _prefill(torch, cfg, Q, K, V, A)
    heads = [0, 11, 22, 31]
    sel = lambda t: to_f64(t[0, heads])
    Qs, Ks, Vs, As = sel(Q), sel(K), sel(V), sel(A)
    ends = [1 << 10, 1 << 12, 1 << 14, 1 << 16, cfg.T]
    Yr = np.empty_like(Vs)
    den = np.empty(As.shape)
    Sr = zr = None
    states = {}
    t0 = 0
    for t1 in ends:
        yp, Sr, zr, dp = oracle.recurrence_heads(Qs[:, t0:t1], Ks[:, t0:t1], Vs[:, t0:t1], As[:, t0:t1],
                                                 eps=cfg.eps, S0=Sr, z0=zr, threads=4)
        Yr[:, t0:t1], den[:, t0:t1] = yp, dp
        states[t1] = (Sr, zr)
        t0 = t1
    Yg = sel(Y)
    ya, yr = max_abs(Yg, Yr), maxnorm_rel(Yg, Yr, 2)
    sr, zrel = maxnorm_rel(sel(S), Sr, 2), elem_rel(sel(z), zr)
    _report(cfg.name + " heads %s" % heads, ya, yr, sr, zrel)
    err = np.abs(Yg - Yr).max(axis=(0, 2))
    ref = np.abs(Yr).max(axis=(0, 2))
    for k in range(0, 18):
        lo, hi = (1 << k) - 1, min((1 << (k + 1)) - 1, cfg.T)
        if lo >= cfg.T:
            break
        print("  tokens [%6d, %6d): max |dy| %.3e  max |y| %.3e  min den %.3e"
              % (lo, hi, err[lo:hi].max(), ref[lo:hi].max(), den[:, lo:hi].min()))
    assert ya <= BF16_Y_ABS and sr <= BF16_STATE_REL and zrel <= BF16_STATE_REL
    assert yr <= Y_MAXNORM_REL and sr <= 5e-3 and zrel <= Z_REL
    # the state at the prefix lengths T'
    idx = torch.tensor(heads, device="cuda")
    for t1 in ends:
        pre = lambda t: t[:, idx, :t1].contiguous()
        Yp = torch.empty_like(pre(V))
        Sp = torch.empty((1, len(heads), cfg.d, cfg.dv), device="cuda")
        zp = torch.empty((1, len(heads), cfg.d), device="cuda")
        la.la_state_init(Sp, zp)
        la.la_prefill_chunked(pre(Q), pre(K), pre(V), pre(A), cfg.eps, cfg.chunk, Yp, Sp, zp)
        torch.cuda.synchronize()
        Sref, zref = states[t1]
        s_err, z_err = maxnorm_rel(to_f64(Sp[0]), Sref, 2), elem_rel(to_f64(zp[0]), zref)
        print("  state at T' = %6d: S max-norm rel %.3e  z rel %.3e" % (t1, s_err, z_err))
        assert s_err <= 5e-3 and z_err <= Z_REL


def test_decode_full_config_sampled(torch):
    """65,536 states seeded by 256 writes each (la_prefill_chunked from zero), then 1024
    decode steps; 2048 sampled states checked at every step and at the end."""
    cfg = wl.DECODE
    N = cfg.n_states
    ks, vs = wl.decode_seed_inputs(cfg, "cuda")
    S = torch.empty((N, 1, cfg.d, cfg.dv), device="cuda")
    z = torch.empty((N, 1, cfg.d), device="cuda")
    la.la_state_init(S, z)
    Yseed = torch.empty_like(vs)
    la.la_prefill_chunked(ks, ks, vs, None, cfg.eps, 64, Yseed, S, z)  # outputs discarded
    del Yseed
    S, z = S.view(N, cfg.d, cfg.dv), z.view(N, cfg.d)
    picks = wl.sampled_states(cfg, 2048)
    pick_t = torch.from_numpy(picks).cuda()
    S_seed = to_f64(S[pick_t])
    z_seed = to_f64(z[pick_t])
    # the seeding itself against the oracle (fp64 sum of the same 256 writes)
    _, Ss, zs, _ = oracle.recurrence_heads(to_f64(ks[pick_t, 0]), to_f64(ks[pick_t, 0]), to_f64(vs[pick_t, 0]),
                                           eps=cfg.eps, threads=THREADS)
    assert maxnorm_rel(S_seed, Ss, 2) <= 5e-3 and elem_rel(z_seed, zs) <= Z_REL
    del ks, vs
    y = torch.empty((N, cfg.dv), device="cuda", dtype=torch.bfloat16)
    qh, kh, vh, yh = [], [], [], []
    for step in range(cfg.steps):
        q, k, v = wl.decode_step_inputs(cfg, step, "cuda")
        la.la_decode_step(q, k, v, None, cfg.eps, y, S, z)
        qh.append(q[pick_t].cpu()), kh.append(k[pick_t].cpu()), vh.append(v[pick_t].cpu())
        yh.append(y[pick_t].cpu())
    torch.cuda.synchronize()
    st = lambda xs: np.stack([x.to(torch.float64).numpy() for x in xs], axis=1)
    # decode steps from the device's own seeded state (exact fp32 values)
    Yr, Sr, zr, _ = oracle.recurrence_heads(st(qh), st(kh), st(vh), eps=cfg.eps, S0=S_seed, z0=z_seed,
                                            threads=THREADS)
    Yg = st(yh)
    ya, yr = max_abs(Yg, Yr), maxnorm_rel(Yg, Yr, 2)
    sr, zrel = maxnorm_rel(to_f64(S[pick_t]), Sr, 2), elem_rel(to_f64(z[pick_t]), zr)
    _report(cfg.name + " (2048 sampled states)", ya, yr, sr, zrel)
    assert ya <= BF16_Y_ABS and sr <= BF16_STATE_REL and zrel <= BF16_STATE_REL
    assert sr <= 1e-4 and zrel <= 1e-4 and yr <= 1e-2


def test_numerics_protocol_long_heads(torch):
    """The numerics check of the page "Linear attention：把历史写进状态" (section "长历史下，状态的
    数值范围会增长": sweep the length, the input scale and the chunk, recording the largest
    error and the smallest denominator).  Heads 0, 11, 22 and 31 of the long gated workload,
    with Q, K and V scaled by 1, 4 and 16 (powers of two: exact in bf16), run at chunks 64
    and 128 against the FP64 oracle on the same values.  Printed per run: the error of y per
    window of positions [2^k, 2^(k+1)), the smallest denominator, and the final S and z."""
    cfg = wl.PREFILL_LONG
    Q, K, V, A = wl.prefill_inputs(cfg, "cuda")
    idx = torch.tensor([0, 11, 22, 31], device="cuda")
    Q4, K4, V4, A4 = (t[:, idx].contiguous() for t in (Q, K, V, A))
    del Q, K, V, A
    H = 4
    for scale in (1, 4, 16):
        Qs, Ks, Vs = (t * scale for t in (Q4, K4, V4))
        Yr, Sr, zr, den = oracle.recurrence_heads(to_f64(Qs), to_f64(Ks), to_f64(Vs), to_f64(A4), eps=cfg.eps,
                                                  threads=THREADS)
        for chunk in (64, 128):
            Y = torch.empty_like(Vs)
            S = torch.empty((1, H, cfg.d, cfg.dv), device="cuda")
            z = torch.empty((1, H, cfg.d), device="cuda")
            la.la_state_init(S, z)
            la.la_prefill_chunked(Qs, Ks, Vs, A4, cfg.eps, chunk, Y, S, z)
            torch.cuda.synchronize()
            Yg = to_f64(Y)
            ya, yr = max_abs(Yg, Yr), maxnorm_rel(Yg, Yr, 2)
            sr, zrel = maxnorm_rel(to_f64(S), Sr, 2), elem_rel(to_f64(z), zr)
            err = np.abs(Yg - Yr).max(axis=(0, 1, 3))
            wins = []
            for k in range(18):
                lo, hi = (1 << k) - 1, min((1 << (k + 1)) - 1, cfg.T)
                if lo >= cfg.T:
                    break
                wins.append("%.1e" % err[lo:hi].max())
            print("protocol scale x%-2d chunk %3d: y max abs %.2e  y max-norm rel %.2e  S rel %.2e  z rel %.2e"
                  "  min den %.3e  max |y| %.2e" % (scale, chunk, ya, yr, sr, zrel, den.min(), np.abs(Yr).max()),
                  flush=True)
            print("  max |dy| per window [2^k - 1, 2^(k+1) - 1), k = 0..17: " + " ".join(wins), flush=True)
            assert np.isfinite(Yg).all()
            assert yr <= Y_MAXNORM_REL and sr <= BF16_STATE_REL and zrel <= Z_REL, (scale, chunk, yr, sr, zrel)
