"""Pins for the stacked-refinement oracle (SequenceO1 close reading,
section 2.2): facts fixed by library routines, closed forms, invariants and
explicit index loops, each written as a check over an implementation dict
so that the planted-mistake test can show every plausible mistake is caught.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import refine_oracle as R
from oracle import sa_oracle as O


def _layer(rng, d, d_ff, w_std=None, ln_random=True):
    ws = (1.0 / math.sqrt(d)) if w_std is None else w_std
    g = (lambda: 1.0 + 0.2 * rng.standard_normal(d)) if ln_random else (lambda: np.ones(d))
    b = (lambda: 0.1 * rng.standard_normal(d)) if ln_random else (lambda: np.zeros(d))
    return R.LayerParams(
        W_Q=rng.standard_normal((d, d)) * ws, W_K=rng.standard_normal((d, d)) * ws,
        ln1_gain=g(), ln1_bias=b(),
        ffn_gate=rng.standard_normal((d, d_ff)) / math.sqrt(d), ffn_up=rng.standard_normal((d, d_ff)) / math.sqrt(d),
        ffn_down=rng.standard_normal((d_ff, d)) / math.sqrt(d_ff),
        ln2_gain=g(), ln2_bias=b())


def _case(seed, n, k, d, d_ff):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)), rng.standard_normal((k, d)), _layer(rng, d, d_ff), 1.0 / math.sqrt(d)


REF = {"layer_norm": R.layer_norm, "silu": R.silu, "ffn": R.swiglu_ffn, "layer": R.refine_layer, "stack": R.stack_user}


# ---------------------------------------------------------------- pin checks

def pin_layer_norm_torch(impl):
    rng = np.random.default_rng(11)
    Z = rng.standard_normal((9, 16)) * 3 + 1
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    ref = torch.nn.functional.layer_norm(torch.tensor(Z), (16,), torch.tensor(g), torch.tensor(b), eps=R.LN_EPS)
    return np.allclose(impl["layer_norm"](Z, g, b), ref.numpy(), atol=1e-12, rtol=0)


def pin_layer_norm_hand_row(impl):
    # (z - 2.5) / sqrt(1.25) for z = 1..4, eps = 0: +-1.5/1.1180339887 and +-0.5/1.1180339887
    out = impl["layer_norm"](np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), np.zeros(4), 0.0)
    return np.allclose(out, [[-1.3416407865, -0.4472135955, 0.4472135955, 1.3416407865]], atol=1e-9)


def pin_silu_logistic(impl):
    x = np.linspace(-12, 12, 97)
    return np.allclose(impl["silu"](x), x * scipy.special.expit(x), atol=1e-14, rtol=1e-13)


def pin_ffn_hand_value(impl):
    # d = d_ff = 1: silu(2 * 1) * (2 * 3) * 0.5 = 3 * 2 / (1 + e^-2) = 5.284782468
    out = impl["ffn"](np.array([[2.0]]), np.array([[1.0]]), np.array([[3.0]]), np.array([[0.5]]))
    return abs(out[0, 0] - 5.284782468) < 1e-8


def pin_ffn_zero_and_linear(impl):
    rng = np.random.default_rng(12)
    Z, Wg, Wu, Wd = (rng.standard_normal(s) for s in ((5, 4), (4, 6), (4, 6), (6, 4)))
    base = impl["ffn"](Z, Wg, Wu, Wd)
    return (np.allclose(impl["ffn"](Z, Wg, Wu, 0 * Wd), 0) and np.allclose(impl["ffn"](Z, 0 * Wg, Wu, Wd), 0)
            and np.allclose(impl["ffn"](Z, Wg, 0 * Wu, Wd), 0)
            and np.allclose(impl["ffn"](Z, Wg, Wu, 2 * Wd), 2 * base, atol=1e-12))


def pin_k_one_row_sum(impl):
    # k = 1: every weight is 1, the aggregate is the row sum of X
    X, P, p, tau = _case(13, 19, 1, 6, 5)
    Y = X.sum(axis=0, keepdims=True)
    xbar = R.layer_norm(P + Y, p.ln1_gain, p.ln1_bias)
    want = R.layer_norm(xbar + R.swiglu_ffn(xbar, p.ffn_gate, p.ffn_up, p.ffn_down), p.ln2_gain, p.ln2_bias)
    return np.allclose(impl["layer"](P, X, p, tau), want, atol=1e-10, rtol=1e-10)


def pin_wk_zero_row_mean(impl):
    # W_K = 0: S = 0, every weight is 1/k, each prototype receives mean-of-rows * n / k
    X, P, p, tau = _case(14, 23, 4, 5, 7)
    p.W_K = np.zeros_like(p.W_K)
    Y = np.repeat(X.sum(axis=0, keepdims=True) / 4.0, 4, axis=0)
    xbar = R.layer_norm(P + Y, p.ln1_gain, p.ln1_bias)
    want = R.layer_norm(xbar + R.swiglu_ffn(xbar, p.ffn_gate, p.ffn_up, p.ffn_down), p.ln2_gain, p.ln2_bias)
    return np.allclose(impl["layer"](P, X, p, tau), want, atol=1e-10, rtol=1e-10)


def pin_row_permutation(impl):
    X, P, p, tau = _case(15, 31, 5, 6, 8)
    perm = np.random.default_rng(16).permutation(31)
    return np.allclose(impl["layer"](P, X, p, tau), impl["layer"](P, X[perm], p, tau), atol=1e-11)


def pin_ffn_zero_eps_zero_normalised(impl):
    # W_down = 0, unit gains, zero biases, eps = 0: the output is LN(Q + Y) (LN is idempotent), whose rows
    # have mean 0 and population variance 1
    X, P, p, tau = _case(17, 12, 3, 8, 4)
    p.ffn_down = np.zeros_like(p.ffn_down)
    for a in ("ln1_gain", "ln2_gain"):
        setattr(p, a, np.ones(8))
    for a in ("ln1_bias", "ln2_bias"):
        setattr(p, a, np.zeros(8))
    out = impl["layer"](P, X, p, tau, eps=0.0)
    Y = O.sketch_user(X, P, p.W_Q, p.W_K, tau)
    return (np.allclose(out.mean(axis=1), 0, atol=1e-12) and np.allclose(out.var(axis=1), 1, atol=1e-12)
            and np.allclose(out, impl["layer_norm"](P + Y, np.ones(8), np.zeros(8), 0.0), atol=1e-12))


def _loops_layer(Q, X, p, tau, eps):
    """One layer by explicit index loops (pure Python)."""
    k, d = len(Q), len(Q[0])
    n, d_ff = len(X), len(p.ffn_gate[0])
    qw = [[sum(Q[j][a] * p.W_Q[a][b] for a in range(d)) for b in range(d)] for j in range(k)]
    xw = [[sum(X[i][c] * p.W_K[c][b] for c in range(d)) for b in range(d)] for i in range(n)]
    S = [[tau * sum(qw[j][b] * xw[i][b] for b in range(d)) for i in range(n)] for j in range(k)]
    Y = [[0.0] * d for _ in range(k)]
    for i in range(n):
        m = max(S[j][i] for j in range(k))
        e = [math.exp(S[j][i] - m) for j in range(k)]
        tot = sum(e)
        for j in range(k):
            for c in range(d):
                Y[j][c] += e[j] / tot * X[i][c]

    def ln(row, g, b):
        mu = sum(row) / d
        var = sum((v - mu) ** 2 for v in row) / d
        return [(row[c] - mu) / math.sqrt(var + eps) * g[c] + b[c] for c in range(d)]

    out = []
    for j in range(k):
        xb = ln([Q[j][c] + Y[j][c] for c in range(d)], p.ln1_gain, p.ln1_bias)
        h = []
        for f in range(d_ff):
            gt = sum(xb[c] * p.ffn_gate[c][f] for c in range(d))
            up = sum(xb[c] * p.ffn_up[c][f] for c in range(d))
            h.append(gt / (1.0 + math.exp(-gt)) * up)
        ff = [sum(h[f] * p.ffn_down[f][c] for f in range(d_ff)) for c in range(d)]
        out.append(ln([xb[c] + ff[c] for c in range(d)], p.ln2_gain, p.ln2_bias))
    return out


def pin_two_layers_by_loops(impl):
    rng = np.random.default_rng(18)
    X, P = rng.standard_normal((4, 3)), rng.standard_normal((2, 3))
    layers = [_layer(rng, 3, 2, w_std=0.9), _layer(rng, 3, 2, w_std=0.9)]
    tau = 0.7
    state = P.tolist()
    for p in layers:
        state = _loops_layer(state, X.tolist(), p, tau, R.LN_EPS)
    return np.allclose(impl["stack"](X, P, layers, tau), np.array(state), atol=1e-11, rtol=1e-11)


def pin_empty_history(impl):
    _, P, p, tau = _case(19, 0, 3, 4, 5)
    xbar = R.layer_norm(P, p.ln1_gain, p.ln1_bias)
    want = R.layer_norm(xbar + R.swiglu_ffn(xbar, p.ffn_gate, p.ffn_up, p.ffn_down), p.ln2_gain, p.ln2_bias)
    return np.allclose(impl["layer"](P, np.zeros((0, 4)), p, tau), want, atol=1e-12)


PINS = [pin_layer_norm_torch, pin_layer_norm_hand_row, pin_silu_logistic, pin_ffn_hand_value, pin_ffn_zero_and_linear,
        pin_k_one_row_sum, pin_wk_zero_row_mean, pin_row_permutation, pin_ffn_zero_eps_zero_normalised,
        pin_two_layers_by_loops, pin_empty_history]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_refine_pin(pin):
    assert pin(REF)


def test_stack_batch_matches_users():
    rng = np.random.default_rng(20)
    X = rng.standard_normal((40, 6))
    P = rng.standard_normal((3, 6))
    layers = [_layer(rng, 6, 4), _layer(rng, 6, 4)]
    offs = [0, 10, 10, 40]
    got = R.stack_batch(X, offs, P, layers, 0.4)
    for u in range(3):
        assert np.allclose(got[u], R.stack_user(X[offs[u]:offs[u + 1]], P, layers, 0.4), atol=0)


# ------------------------------------------------------ planted mistakes

def _ln_axis0(Z, gain, bias, eps=R.LN_EPS):
    Z = np.asarray(Z, dtype=np.float64)
    mu = Z.mean(axis=0, keepdims=True)
    var = ((Z - mu) ** 2).mean(axis=0, keepdims=True)
    return (Z - mu) / np.sqrt(var + eps) * gain + bias


def _ln_rms(Z, gain, bias, eps=R.LN_EPS):
    Z = np.asarray(Z, dtype=np.float64)
    return Z / np.sqrt((Z ** 2).mean(axis=-1, keepdims=True) + eps) * gain + bias


def _ln_unbiased(Z, gain, bias, eps=R.LN_EPS):
    Z = np.asarray(Z, dtype=np.float64)
    mu = Z.mean(axis=-1, keepdims=True)
    var = ((Z - mu) ** 2).sum(axis=-1, keepdims=True) / (Z.shape[-1] - 1)
    return (Z - mu) / np.sqrt(var + eps) * gain + bias


def _layer_with(ln=R.layer_norm, ffn=R.swiglu_ffn, residual1=True, residual2=True):
    def layer(Q, X, p, tau, eps=R.LN_EPS):
        Q = np.asarray(Q, dtype=np.float64)
        X = np.asarray(X, dtype=np.float64)
        Y = np.zeros_like(Q) if X.shape[0] == 0 else O.assignment(O.affinity(X, Q, p.W_Q, p.W_K, tau)) @ X
        xbar = ln((Q if residual1 else 0) + Y, p.ln1_gain, p.ln1_bias, eps)
        return ln((xbar if residual2 else 0) + ffn(xbar, p.ffn_gate, p.ffn_up, p.ffn_down), p.ln2_gain, p.ln2_bias, eps)
    return layer


def _ffn_gate_up_swapped(Z, Wg, Wu, Wd):
    return R.swiglu_ffn(Z, Wu, Wg, Wd)


def _ffn_sigmoid(Z, Wg, Wu, Wd):
    Z = np.asarray(Z, dtype=np.float64)
    return (scipy.special.expit(Z @ Wg) * (Z @ Wu)) @ Wd


def _silu_wrong(x):
    return scipy.special.expit(np.asarray(x, dtype=np.float64))


def _stack_query_from_p(X, P, layers, tau, eps=R.LN_EPS):
    # layer l >= 2 queries with P instead of the previous state (keeps the residual of the state)
    state = np.asarray(P, dtype=np.float64)
    for p in layers:
        Y = O.assignment(O.affinity(X, P, p.W_Q, p.W_K, tau)) @ np.asarray(X, dtype=np.float64)
        xbar = R.layer_norm(state + Y, p.ln1_gain, p.ln1_bias, eps)
        state = R.layer_norm(xbar + R.swiglu_ffn(xbar, p.ffn_gate, p.ffn_up, p.ffn_down), p.ln2_gain, p.ln2_bias, eps)
    return state


def _mut(name):
    impl = dict(REF)
    if name == "ln_over_prototypes":
        impl["layer_norm"] = _ln_axis0
        impl["layer"] = _layer_with(ln=_ln_axis0)
    elif name == "ln_without_centering":
        impl["layer_norm"] = _ln_rms
        impl["layer"] = _layer_with(ln=_ln_rms)
    elif name == "ln_unbiased_variance":
        impl["layer_norm"] = _ln_unbiased
        impl["layer"] = _layer_with(ln=_ln_unbiased)
    elif name == "silu_is_sigmoid":
        impl["silu"] = _silu_wrong
        impl["ffn"] = _ffn_sigmoid
        impl["layer"] = _layer_with(ffn=_ffn_sigmoid)
    elif name == "gate_up_swapped":
        impl["ffn"] = _ffn_gate_up_swapped
        impl["layer"] = _layer_with(ffn=_ffn_gate_up_swapped)
    elif name == "no_first_residual":
        impl["layer"] = _layer_with(residual1=False)
    elif name == "no_ffn_residual":
        impl["layer"] = _layer_with(residual2=False)
    elif name == "later_layers_query_with_p":
        impl["stack"] = _stack_query_from_p
    else:
        raise KeyError(name)
    if impl["layer"] is not REF["layer"] and impl["stack"] is REF["stack"]:
        layer = impl["layer"]

        def stack(X, P, layers, tau, eps=R.LN_EPS):
            s = np.asarray(P, dtype=np.float64)
            for p in layers:
                s = layer(s, X, p, tau, eps)
            return s
        impl["stack"] = stack
    return impl


MUTATIONS = ["ln_over_prototypes", "ln_without_centering", "ln_unbiased_variance", "silu_is_sigmoid",
             "gate_up_swapped", "no_first_residual", "no_ffn_residual", "later_layers_query_with_p"]


@pytest.mark.parametrize("name", MUTATIONS)
def test_planted_mistake_is_caught(name):
    impl = _mut(name)
    assert not all(p(impl) for p in PINS), f"no pin catches {name}"
