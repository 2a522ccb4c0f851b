"""Pins of the delta-rule oracle (``oracle.delta_steps``) to the page "Linear
attention：把历史写进状态", section "Delta rule：先读旧答案，再写误差" and exercise 3:
the printed worked values (exact rationals and FP64), the error recurrence
e' = (1 - beta ||k||^2) e derived under "key 的范数决定了纠错力度", convergence for
0 < beta ||k||^2 < 2, untouched orthogonal keys, and read-after-write.  A meta-test
plants plausible mistakes in a copy of the rule and checks each fails a pin."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.exact import delta_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _cases(name):
    fx = _load(name)
    return fx["cases"] if "cases" in fx else [{"inputs": fx["inputs"], "checks": fx["checks"]}]


def _F(x):
    return Fraction(x)


FIXTURES = ["p2_delta_two_key.json", "p2_delta_repeat.json", "p2_delta_exercise3.json"]


def _oracle_impl(q, k, v, beta, S0):
    return oracle.delta_steps(q, k, v, beta, S0)


def _check(impl, name):
    for case in _cases(name):
        inp = case["inputs"]
        q = [[float(_F(x)) for x in row] for row in inp["q"]]
        k = [[float(_F(x)) for x in row] for row in inp["k"]]
        v = [[float(_F(x)) for x in row] for row in inp["v"]]
        beta = [float(_F(x)) for x in inp["beta"]]
        S0 = [[float(_F(x)) for x in row] for row in inp["S0"]]
        T = len(k)
        # run step by step so every intermediate state is visible
        S = np.array(S0, dtype=np.float64)
        per = []
        for t in range(T):
            Y, S1, P = impl(np.array(q[t:t + 1]), np.array(k[t:t + 1]), np.array(v[t:t + 1]),
                            np.array(beta[t:t + 1]), S)
            per.append({"S": S1, "pred": P[0], "err": np.array(v[t]) - P[0], "y": Y[0]})
            S = S1
        for c in case["checks"]:
            got = np.asarray(per[c["t"] - 1][c["field"]], dtype=np.float64).ravel()
            want = np.array([float(_F(x)) for x in np.asarray(c["value"], dtype=object).ravel()])
            if not np.allclose(got, want, rtol=2e-15, atol=0.0):
                return False
    return True


@pytest.mark.parametrize("name", FIXTURES)
def test_delta_golden_exact_rational(name):
    for case in _cases(name):
        inp = case["inputs"]
        ys, Ss, preds, errs = delta_exact(inp["q"], inp["k"], inp["v"], inp["beta"], inp["S0"])
        fields = {"y": ys, "S": Ss, "pred": preds, "err": errs}
        for c in case["checks"]:
            got = fields[c["field"]][c["t"] - 1]
            want = c["value"]
            if c["field"] == "S":
                assert [[x for x in row] for row in got] == [[_F(x) for x in row] for row in want], (name, c)
            else:
                assert list(got) == [_F(x) for x in want], (name, c)


@pytest.mark.parametrize("name", FIXTURES)
def test_delta_golden_fp64_oracle(name):
    assert _check(_oracle_impl, name)


def _pin_error_recurrence(impl, rng):
    # after one write with key k, the error for the same (k, v) is (1 - beta ||k||^2) e
    for _ in range(20):
        r, dv = int(rng.integers(1, 9)), int(rng.integers(1, 5))
        k = rng.standard_normal(r) * rng.uniform(0.2, 2.0)
        v = rng.standard_normal(dv)
        S0 = rng.standard_normal((r, dv))
        beta = rng.uniform(0.05, 1.5)
        _, _, P = impl(np.stack([k, k]), np.stack([k, k]), np.stack([v, v]), np.array([beta, 0.0]), S0)
        e0, e1 = v - P[0], v - P[1]
        if not np.allclose(e1, (1.0 - beta * (k @ k)) * e0, rtol=1e-12, atol=1e-12):
            return False
    return True


def _pin_convergence(impl):
    k = np.array([[0.6, 0.8]])  # unit norm
    v = np.array([[3.0, -1.0]])
    S0 = np.zeros((2, 2))
    for beta, converges in ((0.5, True), (1.5, True), (2.5, False)):
        _, _, P = impl(np.repeat(k, 60, 0), np.repeat(k, 60, 0), np.repeat(v, 60, 0), np.full(60, beta), S0)
        err = np.abs(v[0] - P[-1]).max()
        if converges != (err < 1e-6):
            return False
    # ||k|| = 2, beta = 1: the error is multiplied by -3 (the page's overshoot case)
    k2 = np.array([[2.0]])
    _, _, P = impl(np.repeat(k2, 2, 0), np.repeat(k2, 2, 0), np.array([[5.0], [5.0]]), np.array([1.0, 0.0]),
                   np.array([[1.0]]))
    return np.isclose(5.0 - P[1, 0], -3.0 * (5.0 - P[0, 0]), rtol=1e-15)


def _pin_orthogonal_untouched(impl, rng):
    Qm, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    k1, k2 = Qm[:, 0], Qm[:, 1]
    S0 = rng.standard_normal((6, 3))
    v = rng.standard_normal(3)
    _, S1, _ = impl(k1[None], k1[None], v[None], np.array([0.7]), S0)
    return np.allclose(k2 @ S1, k2 @ S0, rtol=1e-13, atol=1e-13) and np.allclose(k1 @ S1, k1 @ S0 + 0.7 * (v - k1 @ S0),
                                                                                  rtol=1e-13, atol=1e-13)


def _pin_read_after_write(impl, rng):
    r, dv = 5, 4
    q, k = rng.standard_normal((1, r)), rng.standard_normal((1, r))
    v, S0 = rng.standard_normal((1, dv)), rng.standard_normal((r, dv))
    Y, S1, _ = impl(q, k, v, np.array([0.3]), S0)
    return np.allclose(Y[0], q[0] @ S1, rtol=1e-14, atol=1e-14) and not np.allclose(Y[0], q[0] @ S0)


def test_delta_error_recurrence():
    assert _pin_error_recurrence(_oracle_impl, np.random.default_rng(11))


def test_delta_convergence_and_overshoot():
    assert _pin_convergence(_oracle_impl)


def test_delta_orthogonal_key_untouched():
    assert _pin_orthogonal_untouched(_oracle_impl, np.random.default_rng(12))


def test_delta_read_after_write():
    assert _pin_read_after_write(_oracle_impl, np.random.default_rng(13))


def test_delta_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.delta_steps(np.zeros((2, 3)), np.zeros((2, 4)), np.zeros((2, 1)), np.zeros(2))
    with pytest.raises(ValueError):
        oracle.delta_steps(np.zeros((0, 3)), np.zeros((0, 3)), np.zeros((0, 1)), np.zeros(0))


# ---------------------------------------------------------------- planted mistakes
def _mutant(kind):
    def impl(q, k, v, beta, S0):
        q, k, v = np.asarray(q, float), np.asarray(k, float), np.asarray(v, float)
        S = np.array(S0, dtype=float, copy=True)
        T, dv = v.shape
        Y, P = np.empty((T, dv)), np.empty((T, dv))
        for t in range(T):
            b = float(beta[t])
            p = S.T @ k[t] if kind != "transposed_read" else (S @ k[t][:S.shape[1]] if S.shape[0] == S.shape[1] else S.T @ k[t] * 1.0001)
            P[t] = p
            e = v[t] - p if kind != "flipped_error" else p - v[t]
            if kind == "read_before_write":
                Y[t] = S.T @ q[t]
            if kind == "accumulating_write":
                S = S + b * np.outer(k[t], v[t])
            elif kind == "no_beta":
                S = S + np.outer(k[t], e)
            elif kind == "normalised_key":
                kn = k[t] / np.linalg.norm(k[t])
                S = S + b * np.outer(kn, v[t] - S.T @ kn)
            else:
                S = S + b * np.outer(k[t], e)
            if kind != "read_before_write":
                Y[t] = S.T @ q[t]
        return Y, S, P
    return impl


def _pins_pass(impl):
    try:
        return (all(_check(impl, n) for n in FIXTURES)
                and _pin_error_recurrence(impl, np.random.default_rng(11))
                and _pin_convergence(impl)
                and _pin_orthogonal_untouched(impl, np.random.default_rng(12))
                and _pin_read_after_write(impl, np.random.default_rng(13)))
    except (ValueError, IndexError):
        return False


DELTA_MUTANTS = ["flipped_error", "read_before_write", "accumulating_write", "no_beta", "normalised_key",
                 "transposed_read"]


def test_delta_pins_pass_for_correct_rule():
    assert _pins_pass(_mutant("none"))


@pytest.mark.parametrize("kind", DELTA_MUTANTS)
def test_delta_pins_catch_planted_mistake(kind):
    assert not _pins_pass(_mutant(kind)), kind
