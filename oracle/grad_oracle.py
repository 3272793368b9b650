"""Plain fp64 CPU oracle for the backward pass of Sketch Attention compression.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the HIP
library shares no code with it.

The SequenceO1 close-reading page trains the compression end to end through
the fused kernel (section 2.2 on the stacked refinement, section 2.4 on the
fused FlashSA pass), so the training miss path needs the gradients of the
sketch.  The page prints no backward equations; they follow from the forward
definition of section 2.1 by the chain rule.  For one user, with Q = P W_Q,
K = X W_K, S = tau Q K^T (k x n), A = softmax of S over the prototype axis
and X~ = A X, take a scalar loss L with upstream gradient G = dL/dX~ (k x d):

    dA = G X^T                                      (k x n)
    dS = A * (dA - 1 c^T),  c_i = sum_j A_ji dA_ji   (softmax over j, per column i)
    dX = A^T G + tau dS^T Q W_K^T                   (n x d: aggregation + key path)
    dQ = tau dS K,  dP = dQ W_Q^T,  dW_Q = P^T dQ,  dW_K = tau X^T dS^T Q

The weights are shared by all users, so a batch's weight gradients are the
sums over its users; each user's rows get their own dX.  Everything is
computed literally in float64 from the exact inputs, with numpy's matrix
product as the only library primitive.

Pins (tests under "not gpu"): central finite differences of the forward
oracle for every input; a gradient G whose rows are all equal gives dX_i = g
and zero weight gradients (the mass identity makes L independent of the
weights); k = 1; W_K = 0 (uniform assignment, dX_i = mean_j G_j, dP = dW_Q =
0); a batch equals the sum over its users; planted mistakes are caught.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .sa_oracle import affinity, assignment

__all__ = ["sketch_grad_user", "sketch_grad_batch"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def sketch_grad_user(X, P, W_Q, W_K, tau: float, G) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(G * X~) for one user: dict with dX (n x d), dP
    (k x d), dW_Q and dW_K (d x d), float64.  An empty history contributes
    nothing (its sketch is the constant zero)."""
    X, P, W_Q, W_K, G = _f64(X), _f64(P), _f64(W_Q), _f64(W_K), _f64(G)
    k, d = P.shape
    n = X.shape[0]
    if n == 0:
        z = np.zeros((d, d))
        return {"dX": np.zeros((0, d)), "dP": np.zeros((k, d)), "dW_Q": z, "dW_K": z.copy()}
    Q = P @ W_Q
    K = X @ W_K
    A = assignment(affinity(X, P, W_Q, W_K, tau))   # k x n, columns sum to one
    dA = G @ X.T                                     # dL/dA
    c = (A * dA).sum(axis=0, keepdims=True)          # per behaviour: sum_j A_ji dA_ji
    dS = A * (dA - c)                                # back through the softmax over j
    dK = float(tau) * (dS.T @ Q)                     # n x d
    dQ = float(tau) * (dS @ K)                       # k x d
    return {
        "dX": A.T @ G + dK @ W_K.T,
        "dP": dQ @ W_Q.T,
        "dW_Q": P.T @ dQ,
        "dW_K": X.T @ dK,
    }


def sketch_grad_batch(X, offsets, P, W_Q, W_K, tau: float, G, users: Optional[list] = None) -> Dict[str, np.ndarray]:
    """Gradients over a packed batch (user u owns rows offsets[u]:offsets[u+1],
    G is [U, k, d]): dX [N, d] (rows of users not in `users` left zero), and
    the weight gradients summed over the users."""
    offsets = np.asarray(offsets, dtype=np.int64)
    U = offsets.shape[0] - 1
    P = _f64(P)
    k, d = P.shape
    sel = range(U) if users is None else users
    out = {"dX": np.zeros((int(offsets[-1]), d)), "dP": np.zeros((k, d)), "dW_Q": np.zeros((d, d)),
           "dW_K": np.zeros((d, d))}
    for u in sel:
        a, b = int(offsets[u]), int(offsets[u + 1])
        g = sketch_grad_user(X[a:b], P, W_Q, W_K, tau, G[u])
        out["dX"][a:b] = g["dX"]
        for key in ("dP", "dW_Q", "dW_K"):
            out[key] += g[key]
    return out
