"""Exact rational recurrence for the worked examples (TEST INFRASTRUCTURE ONLY).

The same recurrence as the FP64 oracle -- write first (S <- a*S + k~ v^T,
z <- a*z + k~), then read y = q~^T S / (q~^T z + eps) -- but in
``fractions.Fraction`` arithmetic, on feature-space inputs (the page
"Linear attention：把历史写进状态" states its examples directly in terms of
phi(k), phi(q) and v).  Used only to check the page's printed values and the
FP64 oracle on them; it rounds nothing, so any disagreement is the FP64 side's
rounding or a mistake.
"""
from __future__ import annotations

from fractions import Fraction


def _frac(x) -> Fraction:
    return x if isinstance(x, Fraction) else Fraction(x)


def recurrence_exact(qf, kf, v, alpha=None, eps=0):
    """qf, kf: T lists of r features; v: T lists of dv values; alpha: T gates or None.

    Returns ``(ys, Ss, zs, nums, dens)``: per token the output, the state after
    the write, the normaliser after the write, the numerator q~^T S and the
    denominator q~^T z (without eps).
    """
    T = len(qf)
    r = len(kf[0])
    dv = len(v[0])
    eps = _frac(eps)
    S = [[Fraction(0)] * dv for _ in range(r)]
    z = [Fraction(0)] * r
    ys, Ss, zs, nums, dens = [], [], [], [], []
    for t in range(T):
        a = Fraction(1) if alpha is None else _frac(alpha[t])
        k_t = [_frac(x) for x in kf[t]]
        q_t = [_frac(x) for x in qf[t]]
        v_t = [_frac(x) for x in v[t]]
        S = [[a * S[i][j] + k_t[i] * v_t[j] for j in range(dv)] for i in range(r)]
        z = [a * z[i] + k_t[i] for i in range(r)]
        num = [sum((q_t[i] * S[i][j] for i in range(r)), Fraction(0)) for j in range(dv)]
        den = sum((q_t[i] * z[i] for i in range(r)), Fraction(0))
        ys.append([n / (den + eps) for n in num])
        Ss.append([row[:] for row in S])
        zs.append(z[:])
        nums.append(num)
        dens.append(den)
    return ys, Ss, zs, nums, dens


def delta_exact(q, k, v, beta, S0):
    """The delta rule in rationals: per step p = S^T k, e = v - p, S <- S + beta k e^T,
    y = S^T q (read after the write).  q, k: T lists of r; v: T lists of dv; beta: T
    values; S0: r lists of dv.  Returns ``(ys, Ss, preds, errs)`` per step."""
    S = [[_frac(x) for x in row] for row in S0]
    r, dv = len(S), len(S[0])
    ys, Ss, preds, errs = [], [], [], []
    for t in range(len(k)):
        k_t = [_frac(x) for x in k[t]]
        q_t = [_frac(x) for x in q[t]]
        v_t = [_frac(x) for x in v[t]]
        b = _frac(beta[t])
        p = [sum((k_t[i] * S[i][j] for i in range(r)), Fraction(0)) for j in range(dv)]
        e = [v_t[j] - p[j] for j in range(dv)]
        S = [[S[i][j] + b * k_t[i] * e[j] for j in range(dv)] for i in range(r)]
        y = [sum((q_t[i] * S[i][j] for i in range(r)), Fraction(0)) for j in range(dv)]
        ys.append(y)
        Ss.append([row[:] for row in S])
        preds.append(p)
        errs.append(e)
    return ys, Ss, preds, errs


def relu1_exact(x) -> Fraction:
    """max(x, 0) + 1 in rationals (the positive feature map of the datawhalechina chapter
    "Linear Attention and Recurrent State", Step 4)."""
    x = _frac(x)
    return (x if x > 0 else Fraction(0)) + 1


def noncausal_exact(qf, kf, v, eps=0):
    """The non-causal form in rationals, from a zero state: S = sum of k~ v^T and
    z = sum of k~ over every token, then y_t = q~_t^T S / (q~_t^T z + eps) for every t.
    Returns ``(ys, S, z)``."""
    r, dv = len(kf[0]), len(v[0])
    eps = _frac(eps)
    S = [[sum((_frac(kf[t][i]) * _frac(v[t][j]) for t in range(len(kf))), Fraction(0)) for j in range(dv)]
         for i in range(r)]
    z = [sum((_frac(kf[t][i]) for t in range(len(kf))), Fraction(0)) for i in range(r)]
    ys = []
    for q_t in qf:
        q_t = [_frac(x) for x in q_t]
        den = sum((q_t[i] * z[i] for i in range(r)), Fraction(0))
        ys.append([sum((q_t[i] * S[i][j] for i in range(r)), Fraction(0)) / (den + eps) for j in range(dv)])
    return ys, S, z
