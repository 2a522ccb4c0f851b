"""Shared test helpers: error measures and the oracle run on device tensors.

Error measures (the pages define none):
* S, and Y against the fp32 bar: per-head max-norm relative error
  max|got - ref| / max|ref|, because entries of S and Y cross zero and an
  elementwise relative error is unbounded for any finite-precision result;
* z: elementwise relative error (z > 0 always);
* Y against the bf16 bar: elementwise max absolute error.
"""
from __future__ import annotations

import numpy as np

import oracle

# bars
F32_REL = 1e-4          # fp32 inputs: outputs and final S/z
BF16_Y_ABS = 2e-2       # bf16 inputs: outputs
BF16_STATE_REL = 1e-2   # bf16 inputs: final S/z
BF16_U = 2.0 ** -8      # unit roundoff of bf16 under round-to-nearest
# Internal bounds, tighter than the bars above.  z accumulates the write weights w phi(k)
# in fp32 before they are rounded to bf16 for S, so only fp32 accumulation separates it
# from the exact sum of positive terms.  The outputs' per-head max-norm relative error is
# flagged above 1e-2 (observed: a few 1e-3, from bf16 operands of relative error 2^-9).
Z_REL = 1e-5
Y_MAXNORM_REL = 1e-2


def to_f64(t) -> np.ndarray:
    """Exact upcast of a device or host tensor (bf16/f32/f64) to a float64 array."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def maxnorm_rel(got, ref, head_axes: int) -> float:
    """Largest per-head max|got-ref|/max|ref|; the last ``head_axes`` axes form one head."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lead = got.shape[: got.ndim - head_axes]
    g = got.reshape(int(np.prod(lead)) if lead else 1, -1)
    r = ref.reshape(g.shape)
    err = np.abs(g - r).max(axis=1)
    scale = np.abs(r).max(axis=1)
    scale = np.where(scale == 0, 1.0, scale)
    return float((err / scale).max())


def elem_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float((np.abs(got - ref) / np.abs(ref)).max())


def max_abs(got, ref) -> float:
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max())


def oracle_prefill(Q, K, V, alpha, eps, S0=None, z0=None, threads=8, phi_mode="elu1"):
    """Oracle on the exact values of device tensors Q, K, V [B,H,T,d] etc."""
    return oracle.recurrence_heads(to_f64(Q), to_f64(K), to_f64(V),
                                   None if alpha is None else to_f64(alpha), eps=eps,
                                   S0=None if S0 is None else to_f64(S0),
                                   z0=None if z0 is None else to_f64(z0), phi_mode=phi_mode, threads=threads)


def oracle_noncausal(Q, K, V, eps, S0=None, z0=None, threads=8, phi_mode="elu1"):
    """Non-causal oracle on the exact values of device tensors."""
    return oracle.noncausal_heads(to_f64(Q), to_f64(K), to_f64(V), eps=eps,
                                  S0=None if S0 is None else to_f64(S0),
                                  z0=None if z0 is None else to_f64(z0), phi_mode=phi_mode, threads=threads)


def assert_prefill_parity(Y, S, z, ref, bar: str, label: str = ""):
    """Compare device results with the oracle's (Y, S, z, den) under a named bar."""
    Yr, Sr, zr, _ = ref
    Yg, Sg, zg = to_f64(Y), to_f64(S), to_f64(z)
    assert np.isfinite(Yg).all() and np.isfinite(Sg).all() and np.isfinite(zg).all(), label
    ys = maxnorm_rel(Yg, Yr, 2)
    ss = maxnorm_rel(Sg, Sr, 2)
    zs = elem_rel(zg, zr)
    if bar == "f32":
        assert ys <= F32_REL and ss <= F32_REL and zs <= F32_REL, (label, ys, ss, zs)
    elif bar == "f64":
        assert ys <= 1e-11 and ss <= 1e-11 and zs <= 1e-11, (label, ys, ss, zs)
    elif bar == "bf16":
        ya = max_abs(Yg, Yr)
        assert ya <= BF16_Y_ABS and ss <= BF16_STATE_REL and zs <= BF16_STATE_REL, (label, ya, ss, zs)
    else:
        raise ValueError(bar)
    return {"y_maxnorm_rel": ys, "S_maxnorm_rel": ss, "z_rel": zs, "y_abs": max_abs(Yg, Yr)}
