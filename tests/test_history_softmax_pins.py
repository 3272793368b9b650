"""Pins for the comparator oracle: the same affinity and aggregation as SA
with the softmax taken over the history axis (SequenceO1 close reading,
sections 2.1 and 3.1).  Each pin is a check over an implementation dict so
that planted mistakes can be shown to be caught."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import sa_oracle as O


def _rand(seed, n, k, d, tau=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    P = rng.standard_normal((k, d))
    WQ = rng.standard_normal((d, d)) / math.sqrt(d)
    WK = rng.standard_normal((d, d)) / math.sqrt(d)
    return X, P, WQ, WK, (1.0 / math.sqrt(d) if tau is None else tau)


REF = {"assignment": O.history_assignment, "sketch": O.history_sketch_user}


def pin_rows_sum_to_one(impl):
    X, P, WQ, WK, tau = _rand(1, 41, 6, 5)
    A = impl["assignment"](O.affinity(X, P, WQ, WK, tau))
    return A.shape == (6, 41) and np.allclose(A.sum(axis=1), 1.0, atol=1e-12, rtol=0)


def pin_single_row(impl):
    # n = 1: every prototype puts all its weight on the one row
    X, P, WQ, WK, tau = _rand(2, 1, 5, 4)
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), np.repeat(X, 5, axis=0), atol=1e-12)


def pin_wk_zero_mean_rows(impl):
    X, P, WQ, WK, tau = _rand(3, 29, 4, 6)
    Y = impl["sketch"](X, P, WQ, 0 * WK, tau)
    return np.allclose(Y, np.repeat(X.mean(axis=0, keepdims=True), 4, axis=0), atol=1e-12)


def pin_duplicating_rows_changes_nothing(impl):
    # softmax over the history: a doubled history halves every weight and doubles every term
    X, P, WQ, WK, tau = _rand(4, 17, 5, 4)
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), impl["sketch"](np.vstack([X, X]), P, WQ, WK, tau),
                       atol=1e-12)


def pin_scipy_softmax_history_axis(impl):
    X, P, WQ, WK, tau = _rand(5, 23, 7, 5)
    S = O.affinity(X, P, WQ, WK, tau)
    return np.allclose(impl["assignment"](S), scipy.special.softmax(S, axis=1), atol=1e-14)


def pin_row_permutation(impl):
    X, P, WQ, WK, tau = _rand(6, 31, 5, 6)
    perm = np.random.default_rng(7).permutation(31)
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), impl["sketch"](X[perm], P, WQ, WK, tau), atol=1e-12)


def pin_index_loops(impl):
    X, P, WQ, WK, tau = _rand(8, 4, 3, 3, tau=0.8)
    k, n, d = 3, 4, 3
    S = [[tau * sum(sum(P[j][a] * WQ[a][b] for a in range(d)) * sum(X[i][c] * WK[c][b] for c in range(d))
                    for b in range(d)) for i in range(n)] for j in range(k)]
    want = np.zeros((k, d))
    for j in range(k):
        tot = sum(math.exp(S[j][i]) for i in range(n))
        for i in range(n):
            for c in range(d):
                want[j][c] += math.exp(S[j][i]) / tot * X[i][c]
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), want, atol=1e-12)


def pin_empty_history(impl):
    _, P, WQ, WK, tau = _rand(9, 0, 3, 4)
    return np.array_equal(impl["sketch"](np.zeros((0, 4)), P, WQ, WK, tau), np.zeros((3, 4)))


PINS = [pin_rows_sum_to_one, pin_single_row, pin_wk_zero_mean_rows, pin_duplicating_rows_changes_nothing,
        pin_scipy_softmax_history_axis, pin_row_permutation, pin_index_loops, pin_empty_history]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_history_softmax_pin(pin):
    assert pin(REF)


def test_batch_matches_users():
    X, P, WQ, WK, tau = _rand(10, 50, 4, 5)
    offs = [0, 20, 20, 50]
    got = O.history_sketch_batch(X, offs, P, WQ, WK, tau)
    for u in range(3):
        assert np.allclose(got[u], O.history_sketch_user(X[offs[u]:offs[u + 1]], P, WQ, WK, tau), atol=0)


# ------------------------------------------------------ planted mistakes
def _sketch_with(asg):
    def sketch(X, P, WQ, WK, tau):
        X = np.asarray(X, dtype=np.float64)
        if X.shape[0] == 0:
            return np.zeros(np.asarray(P).shape)
        return asg(O.affinity(X, P, WQ, WK, tau)) @ X
    return sketch


def _mut(name):
    if name == "prototype_axis":          # the SA normalisation instead of the comparator's
        asg = O.assignment
    elif name == "no_normalisation":
        asg = lambda S: np.exp(S)
    elif name == "sum_not_weights":       # normalised by n instead of the exp sum
        asg = lambda S: np.exp(S) / S.shape[1]
    elif name == "prototypes_reversed":   # rows of the assignment attached to the wrong prototypes
        asg = lambda S: O.history_assignment(S[::-1])
    else:
        raise KeyError(name)
    return {"assignment": asg, "sketch": _sketch_with(asg)}


@pytest.mark.parametrize("name", ["prototype_axis", "no_normalisation", "sum_not_weights", "prototypes_reversed"])
def test_planted_mistake_is_caught(name):
    impl = _mut(name)
    assert not all(p(impl) for p in PINS), f"no pin catches {name}"
