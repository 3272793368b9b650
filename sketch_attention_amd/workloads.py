"""Seeded synthetic inputs for Sketch Attention compression.

This module only draws random numbers and lays them out; it performs none of
the method's arithmetic.  Both the GPU path (through the tests and the
benchmark) and the CPU oracle receive the arrays built here, so the two sides
always see the same input bits.

Problem statement followed (SequenceO1 close-reading page, section 2.1): one
user's history is a matrix X with n rows (behaviours, n up to 100K) and d
columns; k learned prototypes P (k x d) are shared by all users; two
projections W_Q and W_K are d x d; tau scales the affinity.  A batch of users
is packed row-wise into one matrix with an int64 offsets array of length U+1
(user u owns rows offsets[u] .. offsets[u+1]-1); the page's fused kernel must
accept such unequal-length batches (section 2.4).

The pages publish no dataset for this path (their data is proprietary), so
the named workloads below are synthetic stand-ins with the paper's
shapes: SA width d = 128 and about a thousand prototypes (section 3.2), and
histories up to 100K behaviours (section 2.1).

All values are generated in float32 with numpy's PCG64 and, for bfloat16
workloads, rounded once to bfloat16 (round to nearest, ties to even).  The
arrays returned are float32 arrays whose values are exactly representable in
the workload's dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Union

import numpy as np

__all__ = [
    "Workload",
    "round_to_bf16",
    "make_workload",
    "named_workload",
    "NAMED_WORKLOADS",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 value (ties to even).

    Returns a float32 array whose low 16 mantissa bits are zero.  Inputs are
    finite synthetic data; NaN/Inf handling is not needed here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One batch of users plus the shared weights.

    X        float32 [N, d]   packed histories (N = offsets[-1])
    offsets  int64   [U+1]    row offsets, offsets[0] = 0, non-decreasing
    P        float32 [k, d]   prototypes
    W_Q, W_K float32 [d, d]   projections (row-vector convention: x @ W)
    tau      float            affinity scale
    dtype    "bf16" or "f32"  the dtype the values are representable in
    """

    name: str
    X: np.ndarray
    offsets: np.ndarray
    P: np.ndarray
    W_Q: np.ndarray
    W_K: np.ndarray
    tau: float
    dtype: str
    recipe: str = ""

    @property
    def d(self) -> int:
        return int(self.P.shape[1])

    @property
    def k(self) -> int:
        return int(self.P.shape[0])

    @property
    def num_users(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def total_rows(self) -> int:
        return int(self.offsets[-1])

    def user_rows(self, u: int) -> np.ndarray:
        return self.X[int(self.offsets[u]):int(self.offsets[u + 1])]


def _finish(arr: np.ndarray, dtype: str) -> np.ndarray:
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return round_to_bf16(arr) if dtype == "bf16" else arr


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def make_workload(
    *,
    lengths: Sequence[int],
    d: int,
    k: int,
    dtype: str = "bf16",
    seed: int = 0,
    tau: Optional[float] = None,
    x_kind: str = "normal",
    x_scale: float = 1.0,
    clusters: int = 64,
    cluster_sigma: float = 0.3,
    dup_fraction: float = 0.0,
    p_kind: str = "normal",
    w_std: Optional[float] = None,
    name: str = "custom",
) -> Workload:
    """Build a seeded workload.

    lengths      per-user history lengths n_u (zeros allowed)
    x_kind       "normal": X ~ N(0, x_scale^2);
                 "clusters": per user, `clusters` centres ~ N(0, I_d), each row
                 is a uniformly chosen centre plus cluster_sigma * N(0, I_d)
    dup_fraction within each user exactly floor(f * n_u) row positions i >= 1
                 (uniform, without replacement) become bitwise copies of a
                 uniformly chosen earlier row of the same user, applied in
                 increasing i
    p_kind       "normal": P ~ N(0, 1); "unit": each P row normalised to unit
                 Euclidean length
    w_std        standard deviation of W_Q, W_K entries (default 1/sqrt(d))
    tau          affinity scale (default 1/sqrt(d))
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    lengths = [int(n) for n in lengths]
    if any(n < 0 for n in lengths):
        raise ValueError("history lengths must be non-negative")
    rng = np.random.Generator(np.random.PCG64(seed))
    if tau is None:
        tau = 1.0 / math.sqrt(d)
    if w_std is None:
        w_std = 1.0 / math.sqrt(d)

    P = _normal(rng, (k, d))
    if p_kind == "unit":
        norms = np.sqrt((P.astype(np.float64) ** 2).sum(axis=1, keepdims=True))
        P = (P / norms).astype(np.float32)
    elif p_kind != "normal":
        raise ValueError(f"unknown p_kind {p_kind!r}")
    W_Q = _normal(rng, (d, d), w_std)
    W_K = _normal(rng, (d, d), w_std)

    offsets = np.zeros(len(lengths) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    N = int(offsets[-1])
    X = np.empty((N, d), dtype=np.float32)
    for u, n in enumerate(lengths):
        if n == 0:
            continue
        r0 = int(offsets[u])
        if x_kind == "normal":
            block = _normal(rng, (n, d), x_scale)
        elif x_kind == "clusters":
            centres = _normal(rng, (clusters, d))
            idx = rng.integers(0, clusters, size=n)
            block = centres[idx] + _normal(rng, (n, d), cluster_sigma)
            if x_scale != 1.0:
                block *= np.float32(x_scale)
        else:
            raise ValueError(f"unknown x_kind {x_kind!r}")
        block = _finish(block, dtype)
        ndup = int(math.floor(dup_fraction * n)) if n > 1 else 0
        if ndup > 0:
            positions = np.sort(rng.choice(np.arange(1, n), size=ndup, replace=False))
            sources = rng.integers(0, positions)  # source < position, uniform
            root = np.arange(n)
            for pos, src in zip(positions.tolist(), sources.tolist()):
                root[pos] = root[src]
            block = block[root]
        X[r0:r0 + n] = block

    return Workload(
        name=name,
        X=X,
        offsets=offsets,
        P=_finish(P, dtype),
        W_Q=_finish(W_Q, dtype),
        W_K=_finish(W_K, dtype),
        tau=float(tau),
        dtype=dtype,
    )


def _ragged_lengths(seed: int, users: int, lo: int, hi: int) -> list:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=users).tolist()


# The workloads: tiny fp32 check, recent-branch scale, full long history
# (the headline shape n=100K, k=256, d=128), many prototypes, ragged batch,
# and the page's final configuration (k = 1024 at d = 128).
NAMED_WORKLOADS = {
    "tiny": dict(
        recipe="1 user, n=1024, d=64, k=16, fp32; X,P ~ N(0,1); W ~ N(0,1/d); tau=1/sqrt(d)",
        args=dict(lengths=[1024], d=64, k=16, dtype="f32", seed=1001),
    ),
    "recent": dict(
        recipe="8 users x n=10000, d=128, k=64, bf16; X,P ~ N(0,1); W ~ N(0,1/d); tau=1/sqrt(d)",
        args=dict(lengths=[10000] * 8, d=128, k=64, dtype="bf16", seed=1002),
    ),
    "long": dict(
        recipe=("4 users x n=100000, d=128, k=256, bf16; X = per-user mixture of 64 "
                "N(0,I) centres + 0.3 N(0,I); P ~ N(0,1); W ~ N(0,1/d); tau=1/sqrt(d)"),
        args=dict(lengths=[100000] * 4, d=128, k=256, dtype="bf16", seed=1003,
                  x_kind="clusters", clusters=64, cluster_sigma=0.3),
    ),
    "many_proto": dict(
        recipe=("32 users x n=100000, d=64, k=1024, bf16; X ~ N(0,1); P rows unit-norm; "
                "W ~ N(0,1/d); tau=1/sqrt(d)"),
        args=dict(lengths=[100000] * 32, d=64, k=1024, dtype="bf16", seed=1004, p_kind="unit"),
    ),
    "ragged": dict(
        recipe=("64 users, n_u ~ U{1000..100000}, d=128, k=128, bf16; X,P ~ N(0,1); "
                "20% of rows exact copies of earlier rows; W ~ N(0,1/d); tau=1/sqrt(d)"),
        args=dict(d=128, k=128, dtype="bf16", seed=1005, dup_fraction=0.2),
        lengths=lambda: _ragged_lengths(2005, 64, 1000, 100000),
    ),
    # the final configuration of the SequenceO1 page (about a thousand
    # prototypes at width 128, section 3.2), on the long workload's histories
    "final": dict(
        recipe=("4 users x n=100000, d=128, k=1024, bf16; X = per-user mixture of 64 "
                "N(0,I) centres + 0.3 N(0,I); P ~ N(0,1); W ~ N(0,1/d); tau=1/sqrt(d)"),
        args=dict(lengths=[100000] * 4, d=128, k=1024, dtype="bf16", seed=1006,
                  x_kind="clusters", clusters=64, cluster_sigma=0.3),
    ),
}


def named_workload(name: str, users: Optional[int] = None,
                   lengths: Optional[Union[int, Sequence[int]]] = None) -> Workload:
    """Build one of the named workloads.

    `users` keeps the per-user shape and changes the number of users (the
    first `users` lengths of the recipe, cycled if more are asked for).
    `lengths` overrides the per-user lengths altogether.
    """
    spec = NAMED_WORKLOADS[name]
    args = dict(spec["args"])
    if "lengths" in spec:
        args["lengths"] = spec["lengths"]()
    if lengths is not None:
        args["lengths"] = [int(lengths)] * (users or 1) if isinstance(lengths, int) else list(lengths)
    elif users is not None:
        base = list(args["lengths"])
        args["lengths"] = [base[i % len(base)] for i in range(users)]
    wl = make_workload(name=name, **args)
    wl.recipe = spec["recipe"]
    return wl


def make_stack_layers(*, d: int, d_ff: int, layers: int, dtype: str = "bf16", seed: int = 0,
                      w_std: Optional[float] = None) -> list:
    """Seeded weights of a refinement stack: one dict per layer with W_Q, W_K
    ~ N(0, w_std^2) (default 1/d variance; rounded to the dtype), layer-norm
    gains 1 + 0.1 N(0, 1) and biases 0.1 N(0, 1), FFN gate/up ~ N(0, 1/d) and
    down ~ N(0, 1/d_ff), all float32 numpy arrays.  Random numbers only: no
    arithmetic of the method."""
    rng = np.random.default_rng(np.random.PCG64(seed + 7919))
    ws = (1.0 / np.sqrt(d)) if w_std is None else w_std
    out = []
    for _ in range(layers):
        out.append({
            "W_Q": _finish(_normal(rng, (d, d), ws), dtype),
            "W_K": _finish(_normal(rng, (d, d), ws), dtype),
            "ln1_gain": 1.0 + _normal(rng, (d,), 0.1),
            "ln1_bias": _normal(rng, (d,), 0.1),
            "ffn_gate": _normal(rng, (d, d_ff), 1.0 / np.sqrt(d)),
            "ffn_up": _normal(rng, (d, d_ff), 1.0 / np.sqrt(d)),
            "ffn_down": _normal(rng, (d_ff, d), 1.0 / np.sqrt(d_ff)),
            "ln2_gain": 1.0 + _normal(rng, (d,), 0.1),
            "ln2_bias": _normal(rng, (d,), 0.1),
        })
    return out


def make_upstream_grad(users: int, k: int, d: int, seed: int = 0, scale: float = 1.0) -> np.ndarray:
    """Seeded upstream gradient dL/dX~ for the backward pass: float32 [users, k, d], N(0, scale^2)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    return (rng.standard_normal((users, k, d)) * scale).astype(np.float32)


def make_action_inputs(rows: int, d: int, d_a: int, d_ff: int, n_actions: int, seed: int = 0) -> dict:
    """Seeded inputs of the action fusion: item embeddings E [rows, d] ~ N(0, 1),
    action ids [rows] uniform over n_actions (int32), an action table
    [n_actions, d_a] ~ N(0, 1), W_gate and W_up [d + d_a, d_ff] ~ N(0, 1/(d + d_a)),
    W_down [d_ff, d] ~ N(0, 1/d_ff); floating arrays rounded to bf16, float32."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    k_in = d + d_a
    return {
        "E": round_to_bf16(_normal(rng, (rows, d))),
        "actions": rng.integers(0, n_actions, size=rows).astype(np.int32),
        "table": round_to_bf16(_normal(rng, (n_actions, d_a))),
        "W_gate": round_to_bf16(_normal(rng, (k_in, d_ff), 1.0 / math.sqrt(k_in))),
        "W_up": round_to_bf16(_normal(rng, (k_in, d_ff), 1.0 / math.sqrt(k_in))),
        "W_down": round_to_bf16(_normal(rng, (d_ff, d), 1.0 / math.sqrt(d_ff))),
    }
