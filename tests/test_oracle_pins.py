"""Pins for the FP64 oracle (CPU only).

Everything here ties the oracle to facts fixed outside the oracle itself:
the page's printed worked examples (``tests/golden/*.json``, each citing its
section of "Linear attention：把历史写进状态", hs-black.github.io), exact
rational arithmetic, closed forms, invariants and brute force.  The last test
plants plausible mistakes in a copy of the recurrence and checks that every
one of them fails at least one pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.exact import recurrence_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _F(x):
    return Fraction(x) if not isinstance(x, list) else [_F(e) for e in x]


def _preimage(f):
    """x with ELU(x)+1 == f: exactly for f in {0, 1, 2, 3, ...}, by log for 0 < f < 1."""
    f = float(f)
    if f == 0.0:
        return -math.inf
    if f >= 1.0:
        return f - 1.0
    return math.log(f)


def _close(got, exact, rel=2e-15):
    exact = float(exact)
    return abs(got - exact) <= rel * abs(exact) + 1e-300


TRAJECTORY_FIXTURES = ["p2_two_dim_state.json", "p2_accumulators_readout.json",
                       "p2_exercise1.json", "p2_gate_walkthrough.json", "p2_exercise2.json"]


def _inputs(fx):
    inp = fx["inputs"]
    qf, kf, v = (_F(inp[n]) for n in ("qf", "kf", "v"))
    alpha = None if inp["alpha"] is None else _F(inp["alpha"])
    return qf, kf, v, alpha


def _fp64_trajectory(impl, qf, kf, v, alpha, eps, phi_mode):
    """Run an implementation one prefix at a time so every intermediate S, z is visible."""
    T = len(qf)
    out = []
    for t in range(1, T + 1):
        if phi_mode == "identity":
            q = np.array([[float(x) for x in row] for row in qf[:t]])
            k = np.array([[float(x) for x in row] for row in kf[:t]])
        else:
            q = np.array([[_preimage(x) for x in row] for row in qf[:t]])
            k = np.array([[_preimage(x) for x in row] for row in kf[:t]])
        vv = np.array([[float(x) for x in row] for row in v[:t]])
        a = None if alpha is None else np.array([float(x) for x in alpha[:t]])
        Y, S, z, den = impl(q, k, vv, a, eps, phi_mode)
        num = Y[t - 1] * (den[t - 1] + eps)
        out.append({"y": Y[t - 1], "S": S, "z": z, "den": den[t - 1], "num": num})
    return out


def _oracle_impl(q, k, v, alpha, eps, phi_mode):
    return oracle.recurrence(q, k, v, alpha, eps=eps, phi_mode=phi_mode)


def _check_fixture(impl, name, phi_mode):
    fx = _load(name)
    qf, kf, v, alpha = _inputs(fx)
    traj = _fp64_trajectory(impl, qf, kf, v, alpha, 0.0, phi_mode)
    for c in fx["checks"]:
        got = traj[c["t"] - 1][c["field"]]
        want = c["value"]
        if c["field"] == "num":
            # num is reconstructed as y*(den+eps): allow the division's and product's rounding
            ok = all(_close(g, Fraction(w), rel=8e-16 * 4) for g, w in zip(np.ravel(got), want))
        elif isinstance(want, list):
            flat_w = [Fraction(w) for w in (np.ravel(np.array(want, dtype=object)))]
            ok = np.shape(got) == np.shape(np.array(want, dtype=object)) and all(
                _close(g, w) for g, w in zip(np.ravel(got), flat_w))
        else:
            ok = _close(float(got), Fraction(want))
        if not ok:
            return False
    return True


# ----------------------------------------------------------------- worked examples

@pytest.mark.parametrize("name", TRAJECTORY_FIXTURES)
def test_golden_exact_rational(name):
    """The page's printed values hold exactly for the rational recurrence."""
    fx = _load(name)
    qf, kf, v, alpha = _inputs(fx)
    ys, Ss, zs, nums, dens = recurrence_exact(qf, kf, v, alpha, eps=0)
    fields = {"y": ys, "S": Ss, "z": zs, "num": nums, "den": dens}
    for c in fx["checks"]:
        got = fields[c["field"]][c["t"] - 1]
        want = c["value"]
        if isinstance(want, list):
            assert got == _F([[Fraction(x) for x in r] if isinstance(r, list) else Fraction(r)
                              for r in want]), (name, c)
        else:
            assert got == Fraction(want), (name, c)


@pytest.mark.parametrize("name", TRAJECTORY_FIXTURES)
@pytest.mark.parametrize("phi_mode", ["identity", "elu1"])
def test_golden_fp64_oracle(name, phi_mode):
    """The C oracle reproduces the page's values to FP64 rounding, both on the
    features directly and through ELU+1 on exact preimages (-inf, 0, 1, 2)."""
    assert _check_fixture(_oracle_impl, name, phi_mode)


def test_quadratic_weights_two_dim():
    """Row t=2 of (Q~K~^T)*M is [2, 1]; the normalised weights are 2/3, 1/3."""
    fx = _load("p2_two_dim_state.json")
    qf, kf, v, _ = _inputs(fx)
    q = np.array([[float(x) for x in r] for r in qf])
    k = np.array([[float(x) for x in r] for r in kf])
    A = (q @ k.T) * oracle.gate_products(None, 2)
    quad = fx["quadratic"]
    assert list(A[1]) == [float(Fraction(x)) for x in quad["A_row"]]
    w = A[1] / A[1].sum()
    assert all(_close(g, Fraction(x)) for g, x in zip(w, quad["weights"]))
    Yq, _ = oracle.quadratic_masked(q, k, np.array([[2.0, 1.0], [4.0, 3.0]]), eps=0.0,
                                    phi_mode="identity")
    assert _close(Yq[1, 0], Fraction(8, 3)) and _close(Yq[1, 1], Fraction(5, 3))


def test_exercise2_coefficients_and_alpha1_irrelevant():
    """Exercise 2: the history coefficients at t=3 are [a2*a3, a3, 1]; alpha1 only
    multiplies the zero initial state."""
    fx = _load("p2_exercise2.json")
    alpha = [float(Fraction(a)) for a in fx["inputs"]["alpha"]]
    D = oracle.gate_products(alpha, 3)
    assert list(D[2]) == [float(Fraction(c)) for c in fx["coefficients"]["value"]]
    ones = np.ones((3, 1))
    v = np.array([[2.0], [4.0], [8.0]])
    for a1 in (1.0, 0.5, 0.0, 0.123):
        Y, S, z, _ = oracle.recurrence(ones, ones, v, [a1, 0.5, 0.25], eps=0.0, phi_mode="identity")
        assert _close(Y[2, 0], Fraction(74, 11))


def test_eps_convention():
    """eps is added to the denominator: y = 1 at eps=1e-6, 1.9802 at eps=1e-8; the
    max(den, eps) reading would give 2."""
    fx = _load("p2_eps.json")
    exact_case, approx_case, max_case = fx["cases"]
    # exact rational
    ys, *_ = recurrence_exact(_F(fx["inputs"]["qf"]), _F(fx["inputs"]["kf"]), _F(fx["inputs"]["v"]),
                              eps=Fraction(exact_case["eps"]))
    assert ys[0][0] == Fraction(exact_case["y"])
    # FP64 oracle, raw input ln(1e-6) through ELU+1
    x = math.log(1e-6)
    for case in (exact_case, approx_case):
        eps = float(Fraction(case["eps"]))
        Y, _, _, den = oracle.recurrence([[x]], [[0.0]], [[2.0]], eps=eps)
        assert abs(den[0] - 1e-6) < 1e-20
        if case["exact"]:
            assert abs(Y[0, 0] - float(Fraction(case["y"]))) < 1e-12
        else:
            assert round(Y[0, 0], case["page_digits"]) == float(case["y"])
    Y, _, _, den = oracle.recurrence([[x]], [[0.0]], [[2.0]], eps=1e-6)
    assert abs(Y[0, 0] - float(max_case["y_if_max"])) > 0.5


# ----------------------------------------------------------------- closed forms

def test_phi_closed_form():
    """ELU+1 with scale 1: x+1 above zero, exp(x) at or below; positive, continuous
    at 0, exactly 0 at -inf (the feature-map contract of the first page, ch. 45)."""
    cases = {-math.inf: 0.0, 0.0: 1.0, 1.0: 2.0, 2.0: 3.0, 0.5: 1.5, -1.0: math.exp(-1.0),
             -30.0: math.exp(-30.0), -2.0: math.exp(-2.0), 1e-300: 1.0}
    for x, want in cases.items():
        assert oracle.phi_scalar_c(x) == want
        assert float(oracle.phi(np.array([x]))[0]) == want
    assert (oracle.phi(np.array([-2.0, 0.0])) > 0).all()
    # through the recurrence: one token, phi(q)=1, v=1 -> den = phi(k)
    for x in (-1.0, 0.25, -7.5):
        _, _, z, den = oracle.recurrence([[0.0]], [[x]], [[1.0]], eps=0.0)
        assert den[0] == (x + 1.0 if x > 0 else math.exp(x)) and z[0] == den[0]


def test_repeated_key_invariant():
    """m copies of the same (k, v): y = m a v / (m a + eps), exactly v at eps = 0,
    gated or not (section "没有 z，输出会随重复次数增长")."""
    rng = np.random.default_rng(11)
    for gated in (False, True):
        for m in (1, 5, 37):
            r, dv = 4, 3
            k = np.tile(rng.normal(size=(1, r)), (m, 1))
            q = np.tile(rng.normal(size=(1, r)), (m, 1))
            v = np.tile(rng.normal(size=(1, dv)), (m, 1))
            alpha = rng.uniform(0.2, 1.0, size=m) if gated else None
            Y0, *_ = oracle.recurrence(q, k, v, alpha, eps=0.0)
            assert np.allclose(Y0, v, rtol=1e-14, atol=0)
            if not gated:
                eps = 1e-3
                Y, _, z, den = oracle.recurrence(q, k, v, None, eps=eps)
                a = float(oracle.phi(q[0]) @ oracle.phi(k[0]))
                t = np.arange(1, m + 1)[:, None]
                assert np.allclose(Y, v * (t * a) / (t * a + eps), rtol=1e-13, atol=0)


def _rand_case(rng, T, r, dv, gated, with_state):
    q = rng.normal(size=(T, r)) * 1.3
    k = rng.normal(size=(T, r)) * 1.3
    v = rng.normal(size=(T, dv))
    alpha = rng.uniform(0.0, 1.0, size=T) if gated else None
    if gated and T > 3:
        alpha[T // 3] = 0.0  # a full reset inside the sequence
        alpha[1] = 1.0
    S0 = rng.normal(size=(r, dv)) if with_state else None
    z0 = np.abs(rng.normal(size=r)) + 0.1 if with_state else None
    return q, k, v, alpha, S0, z0


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_recurrence_equals_quadratic_bruteforce(gated, with_state):
    """The recurrence equals the quadratic masked form (brute force, O(T^2) gate
    products) on random tiny inputs."""
    rng = np.random.default_rng(100 + 2 * gated + with_state)
    for T, r, dv in [(1, 1, 1), (2, 3, 2), (9, 4, 5), (33, 6, 3), (48, 8, 8)]:
        q, k, v, alpha, S0, z0 = _rand_case(rng, T, r, dv, gated, with_state)
        Y, S, z, den = oracle.recurrence(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
        Yq, denq = oracle.quadratic_masked(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
        assert np.allclose(Y, Yq, rtol=1e-12, atol=1e-13)
        assert np.allclose(den, denq, rtol=1e-12, atol=0)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 3, 7, 16, 64, 128])
def test_recurrence_equals_chunkwise(gated, chunk):
    """The chunk equations (with the gated extension) give the recurrence's result
    for every chunk size, including ragged last chunks."""
    rng = np.random.default_rng(200 + chunk + 1000 * gated)
    for T, r, dv in [(1, 2, 2), (10, 4, 3), (70, 5, 6), (130, 3, 4)]:
        q, k, v, alpha, S0, z0 = _rand_case(rng, T, r, dv, gated, True)
        Y, S, z, den = oracle.recurrence(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
        Yc, Sc, zc, denc = oracle.chunkwise(q, k, v, alpha, eps=1e-6, chunk=chunk, S0=S0, z0=z0)
        assert np.allclose(Y, Yc, rtol=1e-11, atol=1e-12)
        assert np.allclose(S, Sc, rtol=1e-11, atol=1e-12)
        assert np.allclose(z, zc, rtol=1e-12, atol=0)


@pytest.mark.parametrize("gated", [False, True])
def test_recurrence_equals_tree_scan_and_order_matters(gated):
    """Tree-ordered composition of (a, B) maps equals the sequential recurrence;
    composing in the swapped order does not (gated case)."""
    rng = np.random.default_rng(300 + gated)
    for T in (1, 2, 5, 16, 29):
        q, k, v, alpha, S0, z0 = _rand_case(rng, T, 3, 4, gated, True)
        Y, S, z, _ = oracle.recurrence(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
        Ys, Ss, zs, _ = oracle.scan_prefix(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
        assert np.allclose(Y, Ys, rtol=1e-11, atol=1e-12)
        assert np.allclose(S, Ss, rtol=1e-11, atol=1e-12)
        assert np.allclose(z, zs, rtol=1e-12, atol=0)
    if gated:
        q, k, v, alpha, S0, z0 = _rand_case(rng, 12, 3, 4, True, False)
        alpha = rng.uniform(0.1, 0.9, size=12)
        Ys, *_ = oracle.scan_prefix(q, k, v, alpha, eps=1e-6)
        Yw, *_ = oracle.scan_prefix(q, k, v, alpha, eps=1e-6, order="swapped")
        assert not np.allclose(Ys, Yw, rtol=1e-6)


# ----------------------------------------------------------------- invariants and contracts

def test_prefix_causality_bitwise():
    """Moving later tokens by finite amounts leaves earlier outputs bit-identical."""
    rng = np.random.default_rng(5)
    for gated in (False, True):
        q, k, v, alpha, S0, z0 = _rand_case(rng, 40, 6, 5, gated, True)
        Y, *_ = oracle.recurrence(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
        for t in (0, 17, 38):
            k2, v2, q2 = k.copy(), v.copy(), q.copy()
            k2[t + 1:] += 100.0
            v2[t + 1:] += 100.0
            q2[t + 1:] -= 3.0
            a2 = None if alpha is None else alpha.copy()
            if a2 is not None:
                a2[t + 1:] = 0.5
            Y2, *_ = oracle.recurrence(q2, k2, v2, a2, eps=1e-6, S0=S0, z0=z0)
            assert np.array_equal(Y[: t + 1], Y2[: t + 1])


def test_first_page_contracts():
    """The three-token fixture of ch. 45: output shape = V shape, S is [2, 1], z is
    [2], finite, z > 0; earlier outputs survive a +100 change of the last key and
    value."""
    fx = _load("p1_fixture.json")["inputs"]
    q, k, v = (np.array(fx[n]) for n in ("q", "k", "v"))
    Y, S, z, den = oracle.recurrence(q, k, v, eps=1e-6)
    assert Y.shape == v.shape and S.shape == (2, 1) and z.shape == (2,)
    assert np.isfinite(Y).all() and (z > 0).all() and (den > 0).all()
    k2, v2 = k.copy(), v.copy()
    k2[-1] += 100.0
    v2[-1] += 100.0
    Y2, *_ = oracle.recurrence(q, k2, v2, eps=1e-6)
    assert np.array_equal(Y[:-1], Y2[:-1])


def test_input_contract_rejections():
    """Q/K width mismatch and an empty sequence are rejected (ch. 45 input contract)."""
    with pytest.raises(ValueError):
        oracle.recurrence(np.ones((2, 2)), np.ones((2, 3)), np.ones((2, 1)))
    with pytest.raises(ValueError):
        oracle.recurrence(np.empty((0, 2)), np.empty((0, 2)), np.empty((0, 1)))
    with pytest.raises(ValueError):
        oracle.recurrence(np.ones((3, 2)), np.ones((3, 2)), np.ones((2, 1)))


def test_state_resume_is_exact():
    """Running T1 tokens, then T2 more from the returned state, is bit-identical to
    running T1+T2 at once (the state is the whole summary of the history)."""
    rng = np.random.default_rng(9)
    q, k, v, alpha, S0, z0 = _rand_case(rng, 50, 4, 3, True, True)
    Y, S, z, _ = oracle.recurrence(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
    Ya, Sa, za, _ = oracle.recurrence(q[:20], k[:20], v[:20], alpha[:20], eps=1e-6, S0=S0, z0=z0)
    Yb, Sb, zb, _ = oracle.recurrence(q[20:], k[20:], v[20:], alpha[20:], eps=1e-6, S0=Sa, z0=za)
    assert np.array_equal(Y, np.concatenate([Ya, Yb])) and np.array_equal(S, Sb) and np.array_equal(z, zb)


def test_zero_gate_resets_history():
    """alpha_t = 0 wipes everything before t: outputs from t on equal a fresh run from t."""
    rng = np.random.default_rng(13)
    q, k, v, _, S0, z0 = _rand_case(rng, 30, 4, 3, False, True)
    alpha = rng.uniform(0.3, 1.0, size=30)
    alpha[12] = 0.0
    Y, S, z, _ = oracle.recurrence(q, k, v, alpha, eps=1e-6, S0=S0, z0=z0)
    Yf, Sf, zf, _ = oracle.recurrence(q[12:], k[12:], v[12:], alpha[12:], eps=1e-6)
    assert np.array_equal(Y[12:], Yf) and np.array_equal(S, Sf) and np.array_equal(z, zf)


def test_heads_threaded_equals_serial():
    rng = np.random.default_rng(17)
    Q = rng.normal(size=(3, 2, 20, 4))
    K = rng.normal(size=(3, 2, 20, 4))
    V = rng.normal(size=(3, 2, 20, 5))
    A = rng.uniform(0.5, 1.0, size=(3, 2, 20))
    a = oracle.recurrence_heads(Q, K, V, A, threads=1)
    b = oracle.recurrence_heads(Q, K, V, A, threads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    Y1, *_ = oracle.recurrence(Q[2, 1], K[2, 1], V[2, 1], A[2, 1])
    assert np.array_equal(a[0][2, 1], Y1)


# ----------------------------------------------------------------- the pins catch mistakes

def _mutant(kind):
    """A copy of the recurrence with one planted mistake (never the oracle itself)."""

    def impl(q, k, v, alpha, eps, phi_mode):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        T, r = q.shape
        dv = v.shape[1]

        def fmap(x):
            if phi_mode == "identity":
                return x
            if kind == "relu_plus_one":
                return np.maximum(x, 0.0) + 1.0
            if kind == "elu_without_plus_one":
                return np.where(x > 0, x, np.exp(np.minimum(x, 0)) - 1.0)
            return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0)))

        qf, kf = fmap(q), fmap(k)
        S, z = np.zeros((r, dv)), np.zeros(r)
        Y, den = np.empty((T, dv)), np.empty(T)
        for t in range(T):
            a = 1.0 if alpha is None else float(alpha[t])
            if kind == "gate_index_shift":
                a = 1.0 if alpha is None else float(alpha[t - 1]) if t > 0 else 1.0
            S_old, z_old = S.copy(), z.copy()
            if kind == "gate_after_write":
                S = a * (S + np.outer(kf[t], v[t]))
                z = a * (z + kf[t])
            elif kind == "gate_not_on_z":
                S = a * S + np.outer(kf[t], v[t])
                z = z + kf[t]
            elif kind == "minus_write":
                S = a * S - np.outer(kf[t], v[t])
                z = a * z + kf[t]
            elif kind == "transposed_state":
                S = a * S + np.outer(v[t], kf[t]).reshape(r, dv) if r == dv else a * S + np.outer(kf[t], v[t])
                z = a * z + kf[t]
            else:
                S = a * S + np.outer(kf[t], v[t])
                z = a * z + kf[t]
            Sr, zr = (S_old, z_old) if kind == "read_before_write" else (S, z)
            d = qf[t] @ zr
            if kind == "no_normaliser":
                d = 1.0
            den[t] = d
            if kind == "eps_as_max":
                Y[t] = (qf[t] @ Sr) / max(d, eps)
            elif kind == "query_key_swapped":
                Y[t] = (kf[t] @ Sr) / (kf[t] @ zr + eps)
            else:
                Y[t] = (qf[t] @ Sr) / (d + eps)
        return Y, S, z, den

    return impl


def _pins_pass(impl):
    results = []
    for name in TRAJECTORY_FIXTURES:
        for mode in ("identity", "elu1"):
            try:
                with np.errstate(all="ignore"):
                    results.append(_check_fixture(impl, name, mode))
            except (ValueError, ZeroDivisionError):
                results.append(False)
    # eps pin
    x = math.log(1e-6)
    Y, *_ = impl(np.array([[x]]), np.array([[0.0]]), np.array([[2.0]]), None, 1e-6, "elu1")
    results.append(abs(Y[0, 0] - 1.0) < 1e-9)
    # feature-map pin through the recurrence at negative and positive inputs
    for xv in (-1.0, 0.25):
        _, _, z, den = impl(np.array([[0.0]]), np.array([[xv]]), np.array([[1.0]]), None, 0.0, "elu1")
        results.append(den[0] == (xv + 1.0 if xv > 0 else math.exp(xv)))
    return all(results)


MUTANTS = ["read_before_write", "transposed_state", "no_normaliser", "gate_after_write",
           "gate_not_on_z", "gate_index_shift", "eps_as_max", "relu_plus_one",
           "elu_without_plus_one", "minus_write", "query_key_swapped"]


def test_pins_pass_for_oracle():
    assert _pins_pass(_oracle_impl)
    assert _pins_pass(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    assert not _pins_pass(_mutant(kind)), kind
