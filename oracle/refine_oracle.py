"""Plain fp64 CPU oracle for stacked refinement of SA sketches.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with
it.

What it computes follows the SequenceO1 close-reading page ("SequenceO1:
End-to-End Ultra-Long (100K) Sequence Modeling in Recommendation with
Low-Rank Caching"), section 2.2 "Stacked Refinement and action-side fusion":
after one assignment and aggregation the prototypes carry user information,
so they query the same raw history again.  The page keeps the symbols of the
lost state-update equations: the layer index l, the start state
X~(0) = P(0), the layer's assignment A(l), an intermediate state formed by
adding the history aggregate and normalising, layer normalisation (LN) and
a feed-forward network (FFN); every layer reads the original X, and the
final configuration uses two layers.

Readings taken where the page leaves the update open:

* layer l uses its own projections W_Q(l), W_K(l) and the previous state
  as the query: S(l) = tau * (X~(l-1) W_Q(l))(X W_K(l))^T, assignment over
  the prototype axis exactly as in section 2.1, aggregate Y = A(l) X;
* post-norm residual blocks: Xbar = LN(X~(l-1) + Y), then
  X~(l) = LN(Xbar + FFN(Xbar)), each LN with its own gain and bias over the
  width d and epsilon 1e-5 inside the square root;
* the FFN is the SwiGLU form the page gives for the action fusion:
  FFN(z) = (silu(z W_gate) * (z W_up)) W_down, silu(x) = x / (1 + e^-x), no
  biases.

Every step is computed in float64 from the exact inputs, with numpy's
matrix product as the library primitive and no fusion or reordering.

Pins (tests under "not gpu"): the layer norm against torch's layer_norm in
float64 and a hand-computed row; silu against scipy's logistic function;
k = 1 (the aggregate is the plain row sum) and W_K = 0 (the aggregate is
the row mean in every prototype) closed forms; invariance under permuting
history rows; explicit index loops on tiny inputs; planted mistakes.  No
function here is left unpinned.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence

import numpy as np

from .sa_oracle import affinity, assignment

__all__ = ["LayerParams", "layer_norm", "silu", "swiglu_ffn", "refine_layer", "stack_user", "stack_batch"]

LN_EPS = 1e-5


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


@dataclass
class LayerParams:
    """Parameters of one refinement layer (any array-likes; read as float64)."""
    W_Q: np.ndarray        # d x d
    W_K: np.ndarray        # d x d
    ln1_gain: np.ndarray   # d
    ln1_bias: np.ndarray   # d
    ffn_gate: np.ndarray   # d x d_ff
    ffn_up: np.ndarray     # d x d_ff
    ffn_down: np.ndarray   # d_ff x d
    ln2_gain: np.ndarray   # d
    ln2_bias: np.ndarray   # d


def layer_norm(Z, gain, bias, eps: float = LN_EPS) -> np.ndarray:
    """Normalise each row of Z over its d entries: (z - mean) / sqrt(var + eps)
    * gain + bias, with the population variance (divide by d)."""
    Z = _f64(Z)
    mu = Z.mean(axis=-1, keepdims=True)
    var = ((Z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (Z - mu) / np.sqrt(var + eps) * _f64(gain) + _f64(bias)


def silu(x) -> np.ndarray:
    """x * logistic(x) = x / (1 + e^-x)."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def swiglu_ffn(Z, W_gate, W_up, W_down) -> np.ndarray:
    """(silu(Z W_gate) * (Z W_up)) W_down: the gated feed-forward form the
    page gives for the action fusion (section 2.2), without biases."""
    Z = _f64(Z)
    return (silu(Z @ _f64(W_gate)) * (Z @ _f64(W_up))) @ _f64(W_down)


def refine_layer(Q, X, p: LayerParams, tau: float, eps: float = LN_EPS) -> np.ndarray:
    """One refinement layer for one user: the k x d state Q (X~(l-1))
    queries the user's raw history X (n x d) with the SA assignment of
    section 2.1, the aggregate is added to Q and normalised, then a
    residual FFN block and a second normalisation give X~(l)."""
    Q = _f64(Q)
    X = _f64(X)
    if X.shape[0] == 0:
        Y = np.zeros_like(Q)      # empty history: empty sum
    else:
        A = assignment(affinity(X, Q, p.W_Q, p.W_K, tau))   # k x n, columns sum to one
        Y = A @ X
    Xbar = layer_norm(Q + Y, p.ln1_gain, p.ln1_bias, eps)
    return layer_norm(Xbar + swiglu_ffn(Xbar, p.ffn_gate, p.ffn_up, p.ffn_down), p.ln2_gain, p.ln2_bias, eps)


def stack_user(X, P, layers: Sequence[LayerParams], tau: float, eps: float = LN_EPS) -> np.ndarray:
    """X~(L) for one user: X~(0) = P, then each layer in order, every one
    reading the original history X."""
    state = _f64(P)
    for p in layers:
        state = refine_layer(state, X, p, tau, eps)
    return state


def stack_batch(X, offsets, P, layers: Sequence[LayerParams], tau: float,
                users: Optional[Iterable[int]] = None, eps: float = LN_EPS) -> np.ndarray:
    """stack_user over a packed batch (user u owns rows offsets[u]:offsets[u+1]);
    float64 [U, k, d], or [len(users), k, d] for a chosen subset."""
    offsets = np.asarray(offsets, dtype=np.int64)
    U = offsets.shape[0] - 1
    sel: List[int] = list(range(U)) if users is None else [int(u) for u in users]
    P = _f64(P)
    out = np.zeros((len(sel),) + P.shape, dtype=np.float64)
    for slot, u in enumerate(sel):
        out[slot] = stack_user(X[int(offsets[u]):int(offsets[u + 1])], P, layers, tau, eps)
    return out
