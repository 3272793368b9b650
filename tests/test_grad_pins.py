"""Pins for the backward oracle (gradients of the sketch of SequenceO1 close
reading, section 2.1, by the chain rule).  Each pin checks an implementation
of the per-user gradient so that planted mistakes can be shown to be caught;
the main pin is central finite differences of the forward oracle."""
import math

import numpy as np
import pytest

from oracle import grad_oracle as GO
from oracle import sa_oracle as O


def _rand(seed, n, k, d, tau=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    P = rng.standard_normal((k, d))
    WQ = rng.standard_normal((d, d)) / math.sqrt(d)
    WK = rng.standard_normal((d, d)) / math.sqrt(d)
    G = rng.standard_normal((k, d))
    return X, P, WQ, WK, (0.9 if tau is None else tau), G


def _loss(X, P, WQ, WK, tau, G):
    return float((G * O.sketch_user(X, P, WQ, WK, tau)).sum())


def _fd(arg, X, P, WQ, WK, tau, G, h=1e-6):
    """Central differences of the forward oracle's loss w.r.t. one input."""
    args = {"dX": X, "dP": P, "dW_Q": WQ, "dW_K": WK}
    base = args[arg]
    out = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        plus, minus = base.copy(), base.copy()
        plus[idx] += h
        minus[idx] -= h
        a = dict(args, **{arg: plus})
        b = dict(args, **{arg: minus})
        out[idx] = (_loss(a["dX"], a["dP"], a["dW_Q"], a["dW_K"], tau, G) -
                    _loss(b["dX"], b["dP"], b["dW_Q"], b["dW_K"], tau, G)) / (2 * h)
    return out


def pin_finite_differences(impl):
    ok = True
    for seed, (n, k, d) in enumerate([(5, 3, 4), (7, 4, 3), (2, 5, 2)]):
        X, P, WQ, WK, tau, G = _rand(10 + seed, n, k, d)
        got = impl(X, P, WQ, WK, tau, G)
        for key in ("dX", "dP", "dW_Q", "dW_K"):
            want = _fd(key, X, P, WQ, WK, tau, G)
            ok &= got[key].shape == want.shape and np.allclose(got[key], want, rtol=1e-6, atol=1e-7)
    return ok


def pin_constant_upstream_rows(impl):
    # G_j = g for every j: L = g . sum_j X~_j = g . sum_i x_i (mass identity), so
    # dX_i = g and the weights get no gradient
    X, P, WQ, WK, tau, G = _rand(2, 9, 5, 4)
    G = np.repeat(G[:1], 5, axis=0)
    got = impl(X, P, WQ, WK, tau, G)
    return (np.allclose(got["dX"], np.repeat(G[:1], 9, axis=0), atol=1e-12) and
            all(np.allclose(got[key], 0, atol=1e-12) for key in ("dP", "dW_Q", "dW_K")))


def pin_single_prototype(impl):
    # k = 1: A = 1, X~ = sum_i x_i
    X, P, WQ, WK, tau, G = _rand(3, 6, 1, 5)
    got = impl(X, P, WQ, WK, tau, G)
    return (np.allclose(got["dX"], np.repeat(G, 6, axis=0), atol=1e-12) and
            all(np.allclose(got[key], 0, atol=1e-12) for key in ("dP", "dW_Q", "dW_K")))


def pin_wk_zero(impl):
    # W_K = 0: uniform assignment 1/k, dX_i = mean_j G_j (the key path carries
    # W_K), and P, W_Q see no gradient because K = X W_K = 0
    X, P, WQ, WK, tau, G = _rand(4, 8, 4, 3)
    got = impl(X, P, WQ, 0 * WK, tau, G)
    return (np.allclose(got["dX"], np.repeat(G.mean(axis=0, keepdims=True), 8, axis=0), atol=1e-12) and
            np.allclose(got["dP"], 0, atol=1e-12) and np.allclose(got["dW_Q"], 0, atol=1e-12))


def pin_empty_history(impl):
    X, P, WQ, WK, tau, G = _rand(5, 0, 3, 4)
    got = impl(X, P, WQ, WK, tau, G)
    return got["dX"].shape == (0, 4) and all(np.allclose(got[key], 0) for key in ("dP", "dW_Q", "dW_K"))


PINS = [pin_finite_differences, pin_constant_upstream_rows, pin_single_prototype, pin_wk_zero, pin_empty_history]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_grad_pin(pin):
    assert pin(GO.sketch_grad_user)


def test_batch_is_the_sum_over_users():
    rng = np.random.default_rng(6)
    k, d = 3, 4
    lengths = [4, 0, 7]
    offsets = np.concatenate([[0], np.cumsum(lengths)])
    X = rng.standard_normal((int(offsets[-1]), d))
    P = rng.standard_normal((k, d))
    WQ, WK = rng.standard_normal((d, d)) / 2, rng.standard_normal((d, d)) / 2
    G = rng.standard_normal((3, k, d))
    got = GO.sketch_grad_batch(X, offsets, P, WQ, WK, 0.7, G)
    for key in ("dP", "dW_Q", "dW_K"):
        want = sum(GO.sketch_grad_user(X[offsets[u]:offsets[u + 1]], P, WQ, WK, 0.7, G[u])[key] for u in range(3))
        assert np.allclose(got[key], want, atol=1e-12)
    for u in range(3):
        want = GO.sketch_grad_user(X[offsets[u]:offsets[u + 1]], P, WQ, WK, 0.7, G[u])["dX"]
        assert np.allclose(got["dX"][offsets[u]:offsets[u + 1]], want, atol=1e-12)


# ------------------------------------------------------- planted mistakes
def _mutant(kind):
    def impl(X, P, WQ, WK, tau, G):
        k, d = P.shape
        Q, K = P @ WQ, X @ WK
        A = O.assignment(O.affinity(X, P, WQ, WK, tau))
        dA = G @ X.T
        c = (A * dA).sum(axis=0, keepdims=True)
        if kind == "no_centring":
            c = 0 * c
        if kind == "centre_over_rows":
            c = (A * dA).sum(axis=1, keepdims=True)
        dS = A * (dA - c)
        if kind == "no_tau":
            tau = 1.0
        dK = tau * (dS.T @ Q)
        dQ = tau * (dS @ K)
        dX = A.T @ G + dK @ WK.T
        if kind == "no_aggregation_term":
            dX = dK @ WK.T
        if kind == "wk_untransposed":
            dX = A.T @ G + dK @ WK
        dP = dQ @ WQ.T
        if kind == "wq_untransposed":
            dP = dQ @ WQ
        return {"dX": dX, "dP": dP, "dW_Q": P.T @ dQ, "dW_K": X.T @ dK}
    return impl


@pytest.mark.parametrize("kind", ["no_centring", "centre_over_rows", "no_tau", "no_aggregation_term",
                                  "wk_untransposed", "wq_untransposed"])
def test_planted_mistake_is_caught(kind):
    impl = _mutant(kind)
    assert _mutant("none")(*_rand(1, 5, 3, 4))["dX"].shape == (5, 4)
    assert pin_finite_differences(_mutant("none"))
    assert not all(pin(impl) for pin in PINS), kind
