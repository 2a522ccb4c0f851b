"""Pins of the oracle's feature-map variants and of its non-causal form.

Feature maps: max(x,0)+1 (the positive map of the datawhalechina chapter "Linear
Attention and Recurrent State", Step 4), max(x,0)+1e-5 and sigmoid(x)+1e-5 (the
switchable maps of the pluggable module on the page "线性注意力架构演进", ai-master.cc).
They are pinned to their closed forms at points where the value is known exactly, to
strict positivity (the chapter's feature-map contract), and to a hand-worked run of the
chapter's three-token fixture.

Non-causal form (same ai-master.cc page: K~^T V and the key sum are formed once and
every query reads them; eps added to the denominator as on the hs-black.github.io page):
pinned to the hs-black page's exercise 1 (every token then reads the final state the
page prints, y = [17/6, 11/6]), to the hand-worked relu+1 fixture, to brute-force
unmasked attention, to the causal recurrence on the last token, to invariance under
reordering of the keys and values, to additivity over a split sequence, and to the
epsilon example.  A meta-test plants plausible mistakes in copies and checks that
each one fails a pin."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MODES = ["elu1", "relu1", "relu_eps", "sigmoid_eps"]


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _fl(a):
    return np.array([[float(Fraction(x)) for x in row] for row in a]) if isinstance(a[0], list) else \
        np.array([float(Fraction(x)) for x in a])


# ---------------------------------------------------------------- feature maps
CLOSED_FORMS = {
    # x: value, with x chosen so that the value is exact or a known constant
    "relu1": [(-math.inf, 1.0), (-3.0, 1.0), (0.0, 1.0), (0.5, 1.5), (2.0, 3.0), (1e3, 1001.0)],
    "relu_eps": [(-math.inf, 1e-5), (-3.0, 1e-5), (0.0, 1e-5), (0.5, 0.5 + 1e-5), (2.0, 2.0 + 1e-5)],
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4, limits 0 and 1
    "sigmoid_eps": [(-math.inf, 1e-5), (0.0, 0.5 + 1e-5), (math.log(3.0), 0.75 + 1e-5),
                    (-math.log(3.0), 0.25 + 1e-5), (math.inf, 1.0 + 1e-5), (-800.0, 1e-5)],
    # ELU+1: exp(x) below zero, x + 1 above, 1 at zero
    "elu1": [(-math.inf, 0.0), (0.0, 1.0), (math.log(0.25), 0.25), (2.0, 3.0)],
}


def _pin_closed_forms(fmap):
    for mode, pts in CLOSED_FORMS.items():
        for x, want in pts:
            if not math.isclose(fmap(x, mode), want, rel_tol=4e-16, abs_tol=0.0):
                return False
    return True


def _pin_positive(fmap):
    xs = np.concatenate([-np.logspace(-3, 2.5, 40), [0.0], np.logspace(-3, 2.5, 40)])
    return all(fmap(float(x), m) > 0.0 for m in ("relu1", "relu_eps", "sigmoid_eps") for x in xs)


def _c_map(x, mode):
    return oracle.phi_scalar_c(x, mode)


def _np_map(x, mode):
    return float(oracle.features(np.array([x]), mode)[0])


@pytest.mark.parametrize("fmap", [_c_map, _np_map], ids=["c", "numpy"])
def test_feature_map_closed_forms(fmap):
    assert _pin_closed_forms(fmap)


@pytest.mark.parametrize("fmap", [_c_map, _np_map], ids=["c", "numpy"])
def test_feature_maps_strictly_positive(fmap):
    # the chapter's contract: the map of [-2, 0] is positive
    assert _pin_positive(fmap)
    assert all(fmap(x, m) > 0 for m in ("relu1", "relu_eps", "sigmoid_eps") for x in (-2.0, 0.0))


def test_unknown_mode_rejected():
    with pytest.raises(ValueError):
        oracle.features(np.zeros(2), "softplus")
    with pytest.raises(ValueError):
        oracle.recurrence(np.zeros((1, 2)), np.zeros((1, 2)), np.zeros((1, 1)), phi_mode="softplus")


def _pin_relu1_fixture_causal(recur):
    fx = _load("p1_relu1.json")
    inp = fx["inputs"]
    Y, S, z, _ = recur(np.array(inp["q"]), np.array(inp["k"]), np.array(inp["v"]), None, 0.0, None, None, "relu1")
    want = fx["causal"]
    return (np.allclose(Y, _fl(want["y"]), rtol=4e-16, atol=0) and np.array_equal(S, _fl(want["S"]))
            and np.array_equal(z, _fl(want["z"])))


def test_relu1_fixture_causal():
    assert _pin_relu1_fixture_causal(oracle.recurrence)


def test_relu1_fixture_contracts():
    # the chapter's own checks on its fixture: shapes, finiteness, positive normaliser,
    # earlier outputs unchanged when the last key and value move by +100
    inp = _load("p1_relu1.json")["inputs"]
    q, k, v = np.array(inp["q"]), np.array(inp["k"]), np.array(inp["v"])
    Y, S, z, _ = oracle.recurrence(q, k, v, None, 0.0, phi_mode="relu1")
    assert Y.shape == v.shape and S.shape == (2, 1) and z.shape == (2,)
    assert np.isfinite(Y).all() and (z > 0).all()
    k2, v2 = k.copy(), v.copy()
    k2[-1] += 100.0
    v2[-1] += 100.0
    Y2, _, _, _ = oracle.recurrence(q, k2, v2, None, 0.0, phi_mode="relu1")
    assert np.array_equal(Y[:-1], Y2[:-1])


@pytest.mark.parametrize("mode", MODES)
def test_matrix_forms_agree_for_every_map(mode):
    # the NumPy maps used by the matrix forms and the C map used by the recurrence agree
    rng = np.random.default_rng(21)
    q, k, v = rng.normal(size=(17, 6)) * 2, rng.normal(size=(17, 6)) * 2, rng.normal(size=(17, 3))
    Y, S, z, _ = oracle.recurrence(q, k, v, None, 1e-6, phi_mode=mode)
    Yq, _ = oracle.quadratic_masked(q, k, v, None, 1e-6, phi_mode=mode)
    Yc, Sc, zc, _ = oracle.chunkwise(q, k, v, None, 1e-6, chunk=5, phi_mode=mode)
    assert np.allclose(Y, Yq, rtol=1e-12, atol=1e-13)
    assert np.allclose(Y, Yc, rtol=1e-12, atol=1e-13)
    assert np.allclose(S, Sc, rtol=1e-13, atol=1e-13) and np.allclose(z, zc, rtol=1e-13)


# ---------------------------------------------------------------- non-causal form
def _oracle_nc(q, k, v, eps, S0, z0, mode):
    return oracle.noncausal(q, k, v, eps, S0, z0, mode)


def _pin_exercise1(nc):
    fx = _load("p2_exercise1.json")["inputs"]
    Y, S, z, _ = nc(np.array(fx["qf"], float), np.array(fx["kf"], float), np.array(fx["v"], float), 0.0, None, None,
                    "identity")
    return (np.allclose(Y, np.tile([17 / 6, 11 / 6], (3, 1)), rtol=4e-16, atol=0)
            and np.array_equal(S, [[5, 3], [7, 5]]) and np.array_equal(z, [2, 2]))


def _pin_relu1_fixture(nc):
    fx = _load("p1_relu1.json")
    inp = fx["inputs"]
    Y, S, z, _ = nc(np.array(inp["q"]), np.array(inp["k"]), np.array(inp["v"]), 0.0, None, None, "relu1")
    want = fx["noncausal"]
    return (np.allclose(Y, _fl(want["y"]), rtol=4e-16, atol=0) and np.array_equal(S, _fl(want["S"]))
            and np.array_equal(z, _fl(want["z"])))


def _pin_brute_force(nc, rng):
    for mode in MODES:
        T, r, dv = int(rng.integers(1, 12)), int(rng.integers(1, 7)), int(rng.integers(1, 5))
        q, k, v = rng.normal(size=(T, r)), rng.normal(size=(T, r)), rng.normal(size=(T, dv))
        S0, z0 = rng.normal(size=(r, dv)), rng.uniform(0.5, 2.0, size=r)
        Y, _, _, den = nc(q, k, v, 1e-6, S0, z0, mode)
        Yb, denb = oracle.quadratic_unmasked(q, k, v, 1e-6, S0, z0, mode)
        if not (np.allclose(Y, Yb, rtol=1e-12, atol=1e-12) and np.allclose(den, denb, rtol=1e-13)):
            return False
    return True


def _pin_last_token_is_causal(nc, rng):
    for mode in MODES:
        q, k, v = rng.normal(size=(9, 4)), rng.normal(size=(9, 4)), rng.normal(size=(9, 3))
        Y, S, z, _ = nc(q, k, v, 1e-6, None, None, mode)
        Yc, Sc, zc, _ = oracle.recurrence(q, k, v, None, 1e-6, phi_mode=mode)
        if not (np.allclose(Y[-1], Yc[-1], rtol=1e-13, atol=1e-14) and np.allclose(S, Sc, rtol=1e-14, atol=1e-14)
                and np.allclose(z, zc, rtol=1e-14)):
            return False
        # and, unlike the causal form, earlier tokens see the later ones
        if np.allclose(Y[0], Yc[0]):
            return False
    return True


def _pin_key_order_free(nc, rng):
    q, k, v = rng.normal(size=(11, 5)), rng.normal(size=(11, 5)), rng.normal(size=(11, 2))
    Y, S, z, _ = nc(q, k, v, 1e-6, None, None, "elu1")
    perm = rng.permutation(11)
    Yk, Sk, zk, _ = nc(q, k[perm], v[perm], 1e-6, None, None, "elu1")
    Yq, _, _, _ = nc(q[perm], k, v, 1e-6, None, None, "elu1")
    return (np.allclose(Y, Yk, rtol=1e-13, atol=1e-14) and np.allclose(S, Sk, rtol=1e-13, atol=1e-14)
            and np.allclose(Y[perm], Yq, rtol=1e-13, atol=1e-14))


def _pin_additive(nc, rng):
    # the state after [A; B] is the state after A continued with B, and with S0 = z0 = 0
    # the read uses only that state
    q, k, v = rng.normal(size=(10, 4)), rng.normal(size=(10, 4)), rng.normal(size=(10, 3))
    S0, z0 = rng.normal(size=(4, 3)), rng.uniform(0.5, 1.5, size=4)
    Y, S, z, _ = nc(q, k, v, 1e-6, S0, z0, "sigmoid_eps")
    _, Sa, za, _ = nc(q[:4], k[:4], v[:4], 1e-6, S0, z0, "sigmoid_eps")
    _, Sb, zb, _ = nc(q[4:], k[4:], v[4:], 1e-6, Sa, za, "sigmoid_eps")
    qf = oracle.features(q, "sigmoid_eps")
    Yr = (qf @ S) / ((qf @ z) + 1e-6)[:, None]
    return (np.allclose(S, Sb, rtol=1e-13, atol=1e-13) and np.allclose(z, zb, rtol=1e-14)
            and np.allclose(Y, Yr, rtol=1e-13, atol=1e-14))


def _pin_eps(nc):
    # the hs-black page's epsilon example: q~ = 1e-6, k~ = 1, v = 2 gives 1 at eps = 1e-6
    # and 1.980198... at eps = 1e-8 (max(den, eps) would give 2)
    q, k, v = np.array([[math.log(1e-6)]]), np.array([[0.0]]), np.array([[2.0]])
    y1 = nc(q, k, v, 1e-6, None, None, "elu1")[0][0, 0]
    y2 = nc(q, k, v, 1e-8, None, None, "elu1")[0][0, 0]
    return math.isclose(y1, 1.0, rel_tol=1e-12) and math.isclose(y2, 2e-6 / (1e-6 + 1e-8), rel_tol=1e-12)


def test_noncausal_exercise1_reads_final_state():
    assert _pin_exercise1(_oracle_nc)


def test_noncausal_relu1_fixture():
    assert _pin_relu1_fixture(_oracle_nc)


def test_noncausal_equals_unmasked_brute_force():
    assert _pin_brute_force(_oracle_nc, np.random.default_rng(22))


def test_noncausal_last_token_equals_causal():
    assert _pin_last_token_is_causal(_oracle_nc, np.random.default_rng(23))


def test_noncausal_key_order_free():
    assert _pin_key_order_free(_oracle_nc, np.random.default_rng(24))


def test_noncausal_additive_over_split():
    assert _pin_additive(_oracle_nc, np.random.default_rng(25))


def test_noncausal_eps_convention():
    assert _pin_eps(_oracle_nc)


def test_noncausal_convex_combination():
    # with eps = 0 every output is a convex combination of the values
    rng = np.random.default_rng(26)
    for mode in MODES:
        q, k, v = rng.normal(size=(30, 6)), rng.normal(size=(30, 6)), rng.normal(size=(30, 4))
        Y = oracle.noncausal(q, k, v, 0.0, phi_mode=mode)[0]
        assert (Y <= v.max(axis=0) + 1e-12).all() and (Y >= v.min(axis=0) - 1e-12).all()


def test_noncausal_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.noncausal(np.zeros((2, 3)), np.zeros((2, 4)), np.zeros((2, 1)))
    with pytest.raises(ValueError):
        oracle.noncausal(np.zeros((0, 3)), np.zeros((0, 3)), np.zeros((0, 1)))


# ---------------------------------------------------------------- planted mistakes
def _nc_mutant(kind):
    def impl(q, k, v, eps, S0, z0, mode):
        q, k, v = np.asarray(q, float), np.asarray(k, float), np.asarray(v, float)
        qf, kf = oracle.features(q, mode), oracle.features(k, mode)
        if kind == "raw_query":
            qf = q.copy()
        T, r = q.shape
        S = np.zeros((r, v.shape[1])) if S0 is None else np.array(S0, float)
        z = np.zeros(r) if z0 is None else np.array(z0, float)
        Y, den = np.empty((T, v.shape[1])), np.empty(T)
        if kind == "causal_read":
            for t in range(T):
                S = S + np.outer(kf[t], v[t])
                z = z + kf[t]
                den[t] = qf[t] @ z
                Y[t] = (qf[t] @ S) / (den[t] + eps)
            return Y, S, z, den
        if kind == "drops_start_state":
            S, z = np.zeros_like(S), np.zeros_like(z)
        if kind == "transposed_write":
            S = S + (kf.T @ v if r != v.shape[1] else (kf.T @ v).T)
        else:
            S = S + kf.T @ v
        z = z + kf.sum(axis=0)
        den = qf @ z
        if kind == "eps_as_max":
            Y = (qf @ S) / np.maximum(den, eps)[:, None]
        elif kind == "query_sum_eps":
            # eps inside the key sum: q~ . (sum k~ + eps 1)
            Y = (qf @ S) / (qf @ (z + eps))[:, None]
        else:
            Y = (qf @ S) / (den + eps)[:, None]
        return Y, S, z, den
    return impl


def _nc_pins_pass(impl):
    try:
        return (_pin_exercise1(impl) and _pin_relu1_fixture(impl)
                and _pin_brute_force(impl, np.random.default_rng(22))
                and _pin_last_token_is_causal(impl, np.random.default_rng(23))
                and _pin_key_order_free(impl, np.random.default_rng(24))
                and _pin_additive(impl, np.random.default_rng(25)) and _pin_eps(impl))
    except (ValueError, IndexError):
        return False


NC_MUTANTS = ["causal_read", "drops_start_state", "transposed_write", "eps_as_max", "query_sum_eps", "raw_query"]


def test_noncausal_reference_mutant_passes():
    assert _nc_pins_pass(_nc_mutant("none"))


@pytest.mark.parametrize("kind", NC_MUTANTS)
def test_noncausal_planted_mistake_fails_a_pin(kind):
    assert not _nc_pins_pass(_nc_mutant(kind))


def _map_mutant(kind):
    def fmap(x, mode):
        if mode == "relu1":
            return max(x, 0.0) + (0.0 if kind == "relu_without_one" else 1.0)
        if mode == "relu_eps":
            return max(x, 0.0) + (1.0 if kind == "relu_eps_as_one" else 1e-5)
        if mode == "sigmoid_eps":
            s = 1.0 / (1.0 + math.exp(x if kind == "sigmoid_flipped" else -x)) if abs(x) < 700 else (
                0.0 if (x < 0) != (kind == "sigmoid_flipped") else 1.0)
            return s + (0.0 if kind == "sigmoid_without_eps" else 1e-5)
        if mode == "elu1":
            if x > 0:
                return x + 1.0
            return (math.exp(x) + (1.0 if kind == "elu_plus_one_below" else 0.0)) if x > -math.inf else (
                1.0 if kind == "elu_plus_one_below" else 0.0)
        raise ValueError(mode)
    return fmap


MAP_MUTANTS = ["relu_without_one", "relu_eps_as_one", "sigmoid_flipped", "sigmoid_without_eps", "elu_plus_one_below"]


def test_map_reference_mutant_passes():
    assert _pin_closed_forms(_map_mutant("none")) and _pin_positive(_map_mutant("none"))


@pytest.mark.parametrize("kind", MAP_MUTANTS)
def test_map_planted_mistake_fails_a_pin(kind):
    f = _map_mutant(kind)
    assert not (_pin_closed_forms(f) and _pin_positive(f))


def test_relu1_fixture_is_what_its_script_writes():
    """p1_relu1.json is the output of tests/golden/make_p1_relu1.py (exact rationals, checked
    against the values worked out by hand inside the script)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_p1_relu1", os.path.join(GOLDEN, "make_p1_relu1.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _load("p1_relu1.json") == mod.build()
