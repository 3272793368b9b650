"""Pins for the CPU oracle: facts fixed by the page and by mathematics.

The page (SequenceO1 close reading, section 2.1) prints no worked numeric
example of SA, so the oracle is pinned to closed forms, invariants, a
library softmax and brute-force index sums instead.  Each pin is written as a
check function over a `sketch`/`assignment` pair so that the planted-mistake
test at the bottom can run every pin against deliberately wrong variants of
the oracle and show that each plausible mistake is caught.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

from oracle import sa_oracle as O


def _rand(seed, n, k, d, tau=None, w_std=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    P = rng.standard_normal((k, d))
    ws = (1.0 / math.sqrt(d)) if w_std is None else w_std
    WQ = rng.standard_normal((d, d)) * ws
    WK = rng.standard_normal((d, d)) * ws
    return X, P, WQ, WK, (1.0 / math.sqrt(d) if tau is None else tau)


# ---------------------------------------------------------------- pin checks
# Each returns True when the pin holds for the given implementation.

def pin_columns_sum_to_one(impl):
    X, P, WQ, WK, tau = _rand(1, 37, 5, 6)
    A = impl["assignment"](impl["affinity"](X, P, WQ, WK, tau))
    return A.shape == (5, 37) and np.allclose(A.sum(axis=0), 1.0, atol=1e-12, rtol=0)


def pin_mass_identity(impl):
    X, P, WQ, WK, tau = _rand(2, 50, 7, 4)
    Y = impl["sketch"](X, P, WQ, WK, tau)
    return np.allclose(Y.sum(axis=0), X.sum(axis=0), atol=1e-10, rtol=1e-12)


def pin_k_equals_one(impl):
    X, P, WQ, WK, tau = _rand(3, 23, 1, 5)
    Y = impl["sketch"](X, P, WQ, WK, tau)
    return Y.shape == (1, 5) and np.allclose(Y[0], X.sum(axis=0), atol=1e-12, rtol=1e-12)


def pin_wk_zero_uniform(impl):
    X, P, WQ, WK, tau = _rand(4, 19, 6, 5)
    Y = impl["sketch"](X, P, WQ, np.zeros_like(WK), tau)
    want = np.broadcast_to(X.sum(axis=0) / 6.0, (6, 5))
    return np.allclose(Y, want, atol=1e-12, rtol=1e-12)


def pin_row_permutation(impl):
    X, P, WQ, WK, tau = _rand(5, 31, 4, 6, tau=0.9)
    perm = np.random.default_rng(55).permutation(31)
    return np.allclose(impl["sketch"](X[perm], P, WQ, WK, tau), impl["sketch"](X, P, WQ, WK, tau),
                       atol=1e-12, rtol=1e-12)


def pin_prototype_permutation(impl):
    X, P, WQ, WK, tau = _rand(6, 29, 5, 4, tau=0.7)
    perm = np.random.default_rng(66).permutation(5)
    return np.allclose(impl["sketch"](X, P[perm], WQ, WK, tau), impl["sketch"](X, P, WQ, WK, tau)[perm],
                       atol=1e-12, rtol=1e-12)


def pin_additivity(impl):
    X, P, WQ, WK, tau = _rand(7, 40, 6, 5, tau=1.3)
    whole = impl["sketch"](X, P, WQ, WK, tau)
    parts = impl["sketch"](X[:13], P, WQ, WK, tau) + impl["sketch"](X[13:], P, WQ, WK, tau)
    return np.allclose(whole, parts, atol=1e-12, rtol=1e-12)


def pin_k_two_logistic(impl):
    """k = 2: the weight on prototype 0 is the logistic function of S_0i - S_1i."""
    X, P, WQ, WK, tau = _rand(8, 9, 2, 3, tau=1.7)
    n, d = X.shape
    # affinity by explicit index sums, independent of any matrix routine
    S = [[tau * sum(P[j, a] * WQ[a, b] * X[i, c] * WK[c, b]
                    for a in range(d) for b in range(d) for c in range(d))
          for i in range(n)] for j in range(2)]
    w0 = [1.0 / (1.0 + math.exp(-(S[0][i] - S[1][i]))) for i in range(n)]
    want = np.array([[sum(w0[i] * X[i, c] for i in range(n)) for c in range(d)],
                     [sum((1.0 - w0[i]) * X[i, c] for i in range(n)) for c in range(d)]])
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), want, atol=1e-12, rtol=1e-11)


def pin_single_row_rank_one(impl):
    """n = 1: the sketch is the outer product of the weights and the one row."""
    X, P, WQ, WK, tau = _rand(9, 1, 4, 5, tau=0.8)
    s = tau * (P @ WQ) @ (WK.T @ X[0])
    w = np.exp(s - s.max())
    w /= w.sum()
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), np.outer(w, X[0]), atol=1e-12, rtol=1e-12)


def pin_brute_force(impl):
    """Tiny cases against the definition written as explicit loops with math.exp."""
    for seed, (n, k, d) in enumerate([(1, 1, 1), (2, 3, 2), (3, 4, 3), (5, 2, 3), (4, 3, 2), (5, 4, 3)]):
        X, P, WQ, WK, tau = _rand(100 + seed, n, k, d, tau=0.9)
        S = [[tau * sum(P[j, a] * WQ[a, b] * X[i, c] * WK[c, b]
                        for a in range(d) for b in range(d) for c in range(d))
              for i in range(n)] for j in range(k)]
        want = np.zeros((k, d))
        for i in range(n):
            den = sum(math.exp(S[jj][i]) for jj in range(k))
            for j in range(k):
                a = math.exp(S[j][i]) / den
                for c in range(d):
                    want[j, c] += a * X[i, c]
        if not np.allclose(impl["sketch"](X, P, WQ, WK, tau), want, atol=1e-12, rtol=1e-11):
            return False
    return True


def pin_scipy_softmax(impl):
    X, P, WQ, WK, tau = _rand(10, 33, 8, 6, tau=2.0)
    S = impl["affinity"](X, P, WQ, WK, tau)
    return np.allclose(impl["assignment"](S), scipy.special.softmax(S, axis=0), atol=1e-13, rtol=1e-12)


def pin_hard_assignment(impl):
    """Large tau with well-separated scores: each row goes wholly to its argmax."""
    rng = np.random.default_rng(11)
    d, k, n = 4, 4, 60
    WQ = np.eye(d)
    WK = np.eye(d)
    P = np.eye(k, d) * 3.0
    X = rng.standard_normal((n, d))
    X[np.arange(n), rng.integers(0, d, n)] += 4.0          # one clearly dominant coordinate
    tau = 60.0
    hard = np.zeros((k, d))
    owner = np.argmax(X @ P.T, axis=1)
    for i in range(n):
        hard[owner[i]] += X[i]
    return np.allclose(impl["sketch"](X, P, WQ, WK, tau), hard, atol=1e-8, rtol=1e-8)


def pin_empty_history(impl):
    _, P, WQ, WK, tau = _rand(12, 1, 3, 4)
    Y = impl["sketch"](np.zeros((0, 4)), P, WQ, WK, tau)
    return Y.shape == (3, 4) and not Y.any()


PINS = [pin_columns_sum_to_one, pin_mass_identity, pin_k_equals_one, pin_wk_zero_uniform,
        pin_row_permutation, pin_prototype_permutation, pin_additivity, pin_k_two_logistic,
        pin_single_row_rank_one, pin_brute_force, pin_scipy_softmax, pin_hard_assignment,
        pin_empty_history]

ORACLE = {"sketch": O.sketch_user, "assignment": O.assignment, "affinity": O.affinity}


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    assert pin(ORACLE)


def test_fold_identity():
    """(P W_Q)(X W_K)^T equals (P W_Q W_K^T) X^T by associativity."""
    X, P, WQ, WK, tau = _rand(13, 64, 16, 32)
    lhs = O.affinity(X, P, WQ, WK, tau)
    rhs = tau * O.fold_reference(P, WQ, WK) @ X.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(lhs))


def test_fold_identity_by_loops():
    X, P, WQ, WK, tau = _rand(14, 2, 3, 3)
    F = O.fold_reference(P, WQ, WK)
    want = np.array([[sum(P[j, a] * WQ[a, b] * WK[c, b] for a in range(3) for b in range(3))
                      for c in range(3)] for j in range(3)])
    assert np.allclose(F, want, atol=1e-14, rtol=1e-13)


def test_identical_prototypes_give_identical_rows():
    X, P, WQ, WK, tau = _rand(15, 21, 5, 4)
    P[:] = P[0]
    Y = O.sketch_user(X, P, WQ, WK, tau)
    assert np.allclose(Y, np.broadcast_to(X.sum(axis=0) / 5.0, Y.shape), atol=1e-12)


def test_batch_equals_per_user_and_empty_users():
    rng = np.random.default_rng(16)
    lengths = [3, 0, 7, 1, 0]
    offs = np.concatenate([[0], np.cumsum(lengths)])
    X = rng.standard_normal((offs[-1], 4))
    _, P, WQ, WK, tau = _rand(17, 1, 3, 4)
    Y = O.sketch_batch(X, offs, P, WQ, WK, tau)
    for u in range(len(lengths)):
        assert np.array_equal(Y[u], O.sketch_user(X[offs[u]:offs[u + 1]], P, WQ, WK, tau))
    assert not Y[1].any() and not Y[4].any()
    sub = O.sketch_batch(X, offs, P, WQ, WK, tau, users=[2, 0])
    assert np.array_equal(sub[0], Y[2]) and np.array_equal(sub[1], Y[0])


def test_duplicated_row_counts_twice():
    """A row copied into the history contributes its assignment column again."""
    X, P, WQ, WK, tau = _rand(18, 12, 4, 5)
    Xd = np.concatenate([X, X[3:4]])
    extra = O.sketch_user(X[3:4], P, WQ, WK, tau)
    assert np.allclose(O.sketch_user(Xd, P, WQ, WK, tau), O.sketch_user(X, P, WQ, WK, tau) + extra,
                       atol=1e-12)


# ------------------------------------------------------ planted mistakes
# Wrong variants of the oracle, each a plausible slip; every one must fail
# at least one pin above.

def _mut_softmax_wrong_axis(S):
    S = np.asarray(S, dtype=np.float64)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    return E / E.sum(axis=1, keepdims=True)


def _mut_affinity_wk_transposed(X, P, WQ, WK, tau):
    return tau * (P @ WQ) @ (X @ WK.T).T


def _mut_affinity_no_tau(X, P, WQ, WK, tau):
    return (P @ WQ) @ (X @ WK).T


def _mut_affinity_wq_transposed(X, P, WQ, WK, tau):
    return tau * (P @ WQ.T) @ (X @ WK).T


def _sketch_from(aff, asg, value=None, mean=False, drop_max_row=False):
    def sketch(X, P, WQ, WK, tau):
        X = np.asarray(X, dtype=np.float64)
        if X.shape[0] == 0:
            return np.zeros(P.shape)
        A = asg(aff(X, P, WQ, WK, tau))
        V = X if value is None else X @ value(X.shape[1])
        Y = A @ V
        if mean:
            Y = Y / A.sum(axis=1, keepdims=True)
        return Y
    return sketch


def _mut_impl(name):
    aff, asg = O.affinity, O.assignment
    if name == "softmax over history axis":
        asg = _mut_softmax_wrong_axis
    elif name == "W_K transposed":
        aff = _mut_affinity_wk_transposed
    elif name == "W_Q transposed":
        aff = _mut_affinity_wq_transposed
    elif name == "tau dropped":
        aff = _mut_affinity_no_tau
    impl = {"affinity": aff, "assignment": asg}
    if name == "value projection added":
        impl["sketch"] = _sketch_from(aff, asg, value=lambda d: np.tril(np.ones((d, d))))
    elif name == "mean instead of sum":
        impl["sketch"] = _sketch_from(aff, asg, mean=True)
    else:
        impl["sketch"] = _sketch_from(aff, asg)
    return impl


MUTANTS = ["softmax over history axis", "W_K transposed", "W_Q transposed", "tau dropped",
           "value projection added", "mean instead of sum"]


@pytest.mark.parametrize("name", MUTANTS)
def test_planted_mistake_is_caught(name):
    impl = _mut_impl(name)
    failed = [p.__name__ for p in PINS if not p(impl)]
    assert failed, f"mutant {name!r} passed every pin"


def test_unmutated_rebuild_passes_all_pins():
    """The mutant scaffolding itself is sound: with no mistake it passes."""
    impl = {"affinity": O.affinity, "assignment": O.assignment,
            "sketch": _sketch_from(O.affinity, O.assignment)}
    assert all(p(impl) for p in PINS)
