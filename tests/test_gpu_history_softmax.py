"""Parity of the comparator (softmax over the history axis, SequenceO1 close
reading section 3.1) through the C ABI with the fp64 CPU oracle: normwise
error per user within 2e-2 (bfloat16 inputs).  Covers every plan the
comparator runs on (32, 64 and 128 prototypes per wave, the folded matrix in
registers and in LDS, padded prototypes, and at d = 128 beyond 512 prototypes
independent blocks of 512, each its own work groups), several users per work group,
tiles cut by piece ends, maxima that jump between tiles, and the invariance
the comparator has and Sketch Attention has not: duplicating every row of a
history changes nothing.  The float32 comparator (lockstep pass, four waves
of 16, 32 or 64 prototypes, independent blocks beyond that) is held to 1e-4
on the same kinds of cases."""
import numpy as np
import pytest
import torch

from oracle import sa_oracle as O
from sketch_attention_amd import SketchAttention
from sketch_attention_amd import workloads as W
from sa_testlib import TOL, normwise_err, to_device

pytestmark = pytest.mark.gpu


def _run(wl, X=None, offsets=None):
    Xd, P, WQ, WK = to_device(wl)
    with SketchAttention(P, WQ, WK, wl.tau, norm="history") as sa:
        out = sa.compress(Xd if X is None else X, wl.offsets if offsets is None else offsets)
        torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(wl, got, users=None):
    want = O.history_sketch_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, users=users)
    sel = got if users is None else got[list(users)]
    err = max(normwise_err(g, w) for g, w in zip(sel, want))
    print(f"[history] {wl.name} err={err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[wl.dtype], err


CASES = [
    (128, 256, [1, 64, 65, 3000, 0, 129]),      # 32 prototypes per wave, matrix in registers
    (128, 64, [7, 500, 2]),                     # padded prototypes (k_pad 256)
    (128, 300, [33, 1500]),                     # 64 per wave, matrix in LDS
    (128, 512, [1, 777]),
    (64, 100, [5, 2000, 31]),
    (64, 400, [300, 64]),                       # d = 64, 64 per wave, matrix in registers
    (64, 700, [1, 900]),                        # d = 64, 128 per wave, matrix in LDS
    (64, 16, [40, 3]),
    (128, 600, [3, 1200, 0, 65]),               # d = 128 beyond 512: two independent blocks of 512 prototypes
    (128, 1000, [900, 1]),
    (128, 1024, [2048, 31]),
    (64, 1024, [333, 1000]),
]


@pytest.mark.parametrize("d,k,lengths", CASES, ids=lambda v: str(v))
def test_history_softmax_parity(d, k, lengths):
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="bf16", seed=13 * k + d, name=f"hist-{d}-{k}")
    _check(wl, _run(wl))


def test_history_softmax_many_users_and_empties():
    lengths = list(np.random.default_rng(8).integers(0, 120, size=300))
    wl = W.make_workload(lengths=lengths, d=128, k=128, dtype="bf16", seed=21, name="hist-many")
    got = _run(wl)
    for u, n in enumerate(lengths):
        if n == 0:
            assert not got[u].any()
    _check(wl, got)


def test_history_softmax_jumping_maxima():
    # a few rows deep into each history are scaled by 4 (exact in bfloat16), so many prototypes'
    # running maxima jump by more than the lazy threshold in a later tile and the accumulators are
    # rescaled there; scores stay within about 20 units of log2, where the folded matrix's rounding
    # keeps the weights within tolerance
    wl = W.make_workload(lengths=[4000, 700], d=128, k=256, dtype="bf16", seed=5, name="hist-jump")
    for r in (2500, 2501, 3999, 4000 + 650):
        wl.X[r] *= 4.0
    _check(wl, _run(wl))


def test_history_softmax_duplicated_rows_change_nothing():
    wl = W.make_workload(lengths=[900], d=128, k=256, dtype="bf16", seed=6, name="hist-dup")
    X = to_device(wl)[0]
    once = _run(wl)
    twice = _run(wl, X=torch.cat([X, X]).contiguous(), offsets=[0, 1800])
    err = normwise_err(twice[0], once[0].astype(np.float64))
    print(f"[history] duplicated rows: {err:.3e}", flush=True)
    assert err <= 1e-2


def test_history_softmax_long_workload_sampled_user():
    wl = W.named_workload("long")
    got = _run(wl)
    _check(wl, got, users=[1])


F32_CASES = [
    (64, 16, [40, 3, 0, 1]),                    # 16 prototypes per wave
    (64, 33, [1, 95, 33]),                      # padded to 64
    (128, 100, [7, 500, 2]),                    # 32 per wave, padded to 128
    (128, 128, [1, 64, 65, 1500, 0, 129]),
    (64, 256, [300, 64, 31]),                   # d = 64, 64 per wave
    (64, 700, [1, 900]),                        # d = 64, blocks of 256 (the last one padded)
    (128, 300, [33, 1200]),                     # d = 128, blocks of 128
    (128, 1024, [700, 31, 0]),
]


@pytest.mark.parametrize("d,k,lengths", F32_CASES, ids=lambda v: str(v))
def test_history_softmax_f32_parity(d, k, lengths):
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="f32", seed=7 * k + d, name=f"hist-f32-{d}-{k}")
    got = _run(wl)
    for u, n in enumerate(lengths):
        if n == 0:
            assert not got[u].any()
    _check(wl, got)


def test_history_softmax_f32_jumping_maxima():
    # rows scaled by 8 deep into the histories: maxima jump past the lazy threshold in later tiles
    wl = W.make_workload(lengths=[3000, 500], d=128, k=128, dtype="f32", seed=9, name="hist-f32-jump")
    for r in (1700, 1701, 2999, 3000 + 450):
        wl.X[r] *= 8.0
    _check(wl, _run(wl))


def test_history_softmax_f32_many_users():
    lengths = list(np.random.default_rng(4).integers(0, 90, size=280))  # two launches of users
    wl = W.make_workload(lengths=lengths, d=64, k=64, dtype="f32", seed=22, name="hist-f32-many")
    _check(wl, _run(wl))
