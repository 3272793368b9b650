"""Plain fp64 CPU oracle for Sketch Attention (SA) compression.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with
it.

What it computes follows the SequenceO1 close-reading page
("SequenceO1: End-to-End Ultra-Long (100K) Sequence Modeling in
Recommendation with Low-Rank Caching"), section 2.1 "Sketch Attention":

* a user's history X (n x d) and the k shared prototypes P (k x d);
* an affinity S (k x n) between every prototype j and every behaviour i,
  built from two projections W_Q, W_K (d x d): S = tau * (P W_Q)(X W_K)^T
  (i indexes behaviours, j prototypes).  The placement of tau and the
  row-vector convention (x @ W) are the readings this oracle takes;
* an assignment A (k x n) obtained by normalising S over the prototype
  index: the page states that the denominator sums over j, so every
  behaviour's weights over the k prototypes add up to one;
* the sketch X~ = A X (k x d): the raw X is aggregated, with no value
  projection (the page warns not to add one), as a weighted sum (not a mean).

Every step is computed literally in float64 from the exact input values
(bfloat16 and float32 inputs are exactly representable in float64): W_Q and
W_K are applied as written, the affinity and assignment matrices are formed
in full, and no blocking, folding or reordering is done beyond what the
definition states.  numpy's matrix product serves as the library primitive
for each product.

Pins (tests under "not gpu"): columns of A sum to one; the mass identity
sum_j X~_j = sum_i X_i; k = 1 gives sum_i X_i; W_K = 0 gives (1/k) sum_i X_i
in every row; invariance under permuting history rows; additivity over any
split of a user's rows; k = 2 reduces to the logistic function; n = 1 gives
a rank-one sketch; brute-force index sums on tiny inputs; the hard-assignment
limit; scipy's softmax on the prototype axis; planted mistakes are caught.
The comparator (softmax over the history axis, section 3.1) is pinned in
its own tests: rows of its assignment sum to one, n = 1 and W_K = 0 closed
forms, invariance under duplicating every row, scipy's softmax on the
history axis, index loops, planted mistakes.  No function here is left
unpinned.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

__all__ = ["affinity", "assignment", "sketch_user", "sketch_batch", "fold_reference", "history_assignment",
           "history_sketch_user", "history_sketch_batch"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def affinity(X, P, W_Q, W_K, tau: float) -> np.ndarray:
    """S = tau * (P W_Q)(X W_K)^T, shape (k, n).

    Section 2.1: S is the prototype-behaviour affinity, W_Q and W_K the two
    d x d projections; tau multiplies the affinity before normalisation.
    """
    Q = _f64(P) @ _f64(W_Q)          # queries from the prototypes   (k x d)
    K = _f64(X) @ _f64(W_K)          # keys from the history rows    (n x d)
    return float(tau) * (Q @ K.T)    # (k x n)


def assignment(S) -> np.ndarray:
    """A = softmax of S over the prototype axis (axis 0), shape (k, n).

    Section 2.1: the denominator sums over the prototype index j, so each
    behaviour i distributes a unit of mass over the k prototypes.  The
    column maximum is subtracted first only to keep exp() in range; the
    softmax is unchanged by it.
    """
    S = _f64(S)
    m = S.max(axis=0, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=0, keepdims=True)


def sketch_user(X, P, W_Q, W_K, tau: float) -> np.ndarray:
    """X~ = A X for one user, shape (k, d), float64.

    Section 2.1: the sketch aggregates the raw history with the assignment
    weights; no value projection is applied.  An empty history gives the
    empty sum, a zero sketch.
    """
    X = _f64(X)
    P = _f64(P)
    k, d = P.shape
    if X.shape[0] == 0:
        return np.zeros((k, d), dtype=np.float64)
    A = assignment(affinity(X, P, W_Q, W_K, tau))
    return A @ X


def sketch_batch(X, offsets, P, W_Q, W_K, tau: float,
                 users: Optional[Iterable[int]] = None) -> np.ndarray:
    """Sketches of a packed batch: user u owns rows offsets[u]:offsets[u+1].

    Section 2.4 asks the fused kernel to handle batches of unequal-length
    histories; users are independent, so each is computed on its own.
    Returns float64 [U, k, d] (or [len(users), k, d] for a chosen subset).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    U = offsets.shape[0] - 1
    sel = list(range(U)) if users is None else [int(u) for u in users]
    P = _f64(P)
    out = np.zeros((len(sel), P.shape[0], P.shape[1]), dtype=np.float64)
    for slot, u in enumerate(sel):
        out[slot] = sketch_user(X[int(offsets[u]):int(offsets[u + 1])], P, W_Q, W_K, tau)
    return out


def fold_reference(P, W_Q, W_K) -> np.ndarray:
    """P W_Q W_K^T in float64, shape (k, d).

    By associativity (P W_Q)(X W_K)^T = (P W_Q W_K^T) X^T, so this k x d
    matrix carries all of the affinity's dependence on the weights.  The
    page cites the same reordering idea for single-query cross-attention,
    which avoids forming the history's key projection (section 1).
    """
    return (_f64(P) @ _f64(W_Q)) @ _f64(W_K).T


# ------------------------------------------------------------------ comparator
def history_assignment(S) -> np.ndarray:
    """softmax of S over the history axis (axis 1), shape (k, n).

    Section 2.1 of the close reading contrasts SA with the usual latent
    cross-attention, which normalises over history positions so that each
    prototype selects content from the history; section 3.1 (Figure 3,
    Table 1) compares the two with only the softmax axis changed.  Each row
    of this assignment sums to one over the n behaviours."""
    S = _f64(S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


def history_sketch_user(X, P, W_Q, W_K, tau: float) -> np.ndarray:
    """The comparator's k x d summary for one user: history_assignment(S) X,
    the same affinity and the same aggregation of the raw X as sketch_user;
    an empty history gives zeros."""
    X = _f64(X)
    P = _f64(P)
    if X.shape[0] == 0:
        return np.zeros(P.shape, dtype=np.float64)
    return history_assignment(affinity(X, P, W_Q, W_K, tau)) @ X


def history_sketch_batch(X, offsets, P, W_Q, W_K, tau: float, users: Optional[Iterable[int]] = None) -> np.ndarray:
    """history_sketch_user over a packed batch, float64 [U, k, d] (or a chosen subset)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    U = offsets.shape[0] - 1
    sel = list(range(U)) if users is None else [int(u) for u in users]
    P = _f64(P)
    out = np.zeros((len(sel), P.shape[0], P.shape[1]), dtype=np.float64)
    for slot, u in enumerate(sel):
        out[slot] = history_sketch_user(X[int(offsets[u]):int(offsets[u + 1])], P, W_Q, W_K, tau)
    return out
