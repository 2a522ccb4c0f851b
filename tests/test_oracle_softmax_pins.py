"""Pins of the softmax-attention decode oracle (``oracle.softmax_decode``), the
explicit-history comparator of the datawhalechina chapter "Linear Attention and
Recurrent State" (Step 5).  It computes the attention row of the hs-black.github.io
page, section "先看普通 attention 在读什么": y = sum_i softmax(q.k_i / sqrt(d))_i v_i.
The page prints no numbers for it, so it is pinned to what the definition fixes:
one token returns its value, equal keys average the values, two tokens whose scores
differ by ln 3 weigh 3/4 and 1/4 (with the default 1/sqrt(d) scale too), a constant
shift of every score and any reordering of the history change nothing, a duplicated
token counts twice, a very large scale selects the best-scoring value, and scores of
order 1e3 stay finite.  A meta-test plants plausible mistakes and checks each fails."""
import math

import numpy as np
import pytest

import oracle


def _oracle(q, K, V, scale):
    return oracle.softmax_decode(q, K, V, scale)[0]


def _pin_single_token(f, rng):
    for _ in range(5):
        r, dv = int(rng.integers(1, 9)), int(rng.integers(1, 5))
        v = rng.normal(size=(1, dv))
        y = f(rng.normal(size=r), rng.normal(size=(1, r)) * 5, v, float(rng.uniform(0.1, 3)))
        if not np.array_equal(y, v[0]):
            return False
    return True


def _pin_equal_keys(f, rng):
    k = rng.normal(size=6)
    K = np.tile(k, (9, 1))
    V = rng.normal(size=(9, 3))
    y = f(rng.normal(size=6), K, V, 0.7)
    return np.allclose(y, V.mean(axis=0), rtol=1e-14, atol=1e-15)


def _pin_two_tokens(f):
    # scores differ by ln 3: weights 3/4 and 1/4
    v = np.array([[4.0, -8.0], [8.0, 4.0]])
    want = 0.75 * v[0] + 0.25 * v[1]
    K = np.array([[math.log(3.0), 0.0], [0.0, 0.0]])
    ok = np.allclose(f(np.array([1.0, 0.0]), K, v, 1.0), want, rtol=1e-15, atol=1e-15)
    # the default scale 1/sqrt(d): d = 4, raw score difference 2 ln 3
    K4 = np.array([[2 * math.log(3.0), 0, 0, 0], [0.0, 0, 0, 0]])
    y4 = f(np.array([1.0, 0, 0, 0]), K4, v, None)
    return ok and np.allclose(y4, want, rtol=1e-15, atol=1e-15)


def _pin_shift_and_order(f, rng):
    q = np.array([1.0, 0.0, 0.0, 0.0])
    K = rng.normal(size=(12, 4))
    V = rng.normal(size=(12, 2))
    y = f(q, K, V, 0.9)
    Ks = K.copy()
    Ks[:, 0] += 3.0  # every score moves by 0.9 * 3
    perm = rng.permutation(12)
    return (np.allclose(f(q, Ks, V, 0.9), y, rtol=1e-13, atol=1e-14)
            and np.allclose(f(q, K[perm], V[perm], 0.9), y, rtol=1e-13, atol=1e-14))


def _pin_duplicate(f, rng):
    # a token present twice weighs as one token with its score raised by ln 2
    q = np.array([1.0, 0.5])
    K = rng.normal(size=(5, 2))
    V = rng.normal(size=(5, 3))
    Kd = np.vstack([K, K[2:3]])
    Vd = np.vstack([V, V[2:3]])
    Kb = K.copy()
    Kb[2, 0] += math.log(2.0)  # q . k gains ln 2 (q[0] = 1, scale 1)
    return np.allclose(f(q, Kd, Vd, 1.0), f(q, Kb, V, 1.0), rtol=1e-13, atol=1e-14)


def _pin_large_scale(f, rng):
    q = rng.normal(size=5)
    K = rng.normal(size=(7, 5))
    V = rng.normal(size=(7, 3))
    best = int(np.argmax(K @ q))
    return np.array_equal(f(q, K, V, 1e6), V[best])


def _pin_finite(f):
    q = np.array([30.0, 30.0])
    K = np.array([[30.0, 30.0], [29.0, 30.0], [-30.0, 0.0]])  # scores 1800, 1770, -900
    V = np.array([[1.0], [2.0], [3.0]])
    y = f(q, K, V, 1.0)
    w1 = 1.0 / (1.0 + math.exp(-30.0))
    return np.isfinite(y).all() and math.isclose(y[0], w1 * 1.0 + (1 - w1) * 2.0, rel_tol=1e-14)


PINS = [
    lambda f: _pin_single_token(f, np.random.default_rng(31)),
    lambda f: _pin_equal_keys(f, np.random.default_rng(32)),
    _pin_two_tokens,
    lambda f: _pin_shift_and_order(f, np.random.default_rng(33)),
    lambda f: _pin_duplicate(f, np.random.default_rng(34)),
    lambda f: _pin_large_scale(f, np.random.default_rng(35)),
    _pin_finite,
]


@pytest.mark.parametrize("i", range(len(PINS)))
def test_softmax_oracle_pin(i):
    assert PINS[i](_oracle)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(36)
    _, w = oracle.softmax_decode(rng.normal(size=16), rng.normal(size=(100, 16)), rng.normal(size=(100, 4)))
    assert math.isclose(w.sum(), 1.0, rel_tol=1e-14) and (w > 0).all()


def test_softmax_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.softmax_decode(np.zeros(3), np.zeros((2, 4)), np.zeros((2, 1)))
    with pytest.raises(ValueError):
        oracle.softmax_decode(np.zeros(3), np.zeros((0, 3)), np.zeros((0, 1)))


def _mutant(kind):
    def f(q, K, V, scale):
        q, K, V = np.asarray(q, float), np.asarray(K, float), np.asarray(V, float)
        sc = 1.0 / math.sqrt(K.shape[1]) if scale is None else scale
        if kind == "no_scale":
            sc = 1.0
        if kind == "scale_twice":
            sc = sc / math.sqrt(K.shape[1])
        if kind == "last_token_dropped" and K.shape[0] > 1:
            K, V = K[:-1], V[:-1]
        s = sc * (K @ q)
        if kind == "linear_weights":
            w = s - s.min() + 1.0
        elif kind == "no_max_shift":
            with np.errstate(over="ignore", invalid="ignore"):
                w = np.exp(s)
        else:
            w = np.exp(s - s.max())
        if kind == "unnormalised":
            return w @ V
        with np.errstate(invalid="ignore"):
            return (w @ V) / w.sum()
    return f


MUTANTS = ["no_scale", "scale_twice", "last_token_dropped", "linear_weights", "no_max_shift", "unnormalised"]


def test_reference_mutant_passes():
    assert all(p(_mutant("none")) for p in PINS)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_fails_a_pin(kind):
    assert not all(p(_mutant(kind)) for p in PINS)
