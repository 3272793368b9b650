"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Normwise error per user, max |G - O| / max |O|, must stay within 2e-2 for
bfloat16 inputs with float32 accumulation and 1e-4 for the float32 path, both
on the sketch and on the row-centred sketch.  The five full-size workloads are
checked on every user against the oracle and through the mass
identity (the prototype rows of a sketch add up to the sum of the history
rows, because each behaviour's weights over the prototypes add up to one).
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import sa_oracle as O
from sketch_attention_amd import SketchAttention, binding as B
from sketch_attention_amd import workloads as W
from sa_testlib import TOL, centred_within, normwise_err, run_gpu, to_device, worst_errors

pytestmark = pytest.mark.gpu


def _oracle(wl, users=None):
    """The oracle's sketches of the selected users (all by default), several users at a time on host
    threads (numpy releases the interpreter lock in its array loops and BLAS)."""
    ulist = list(range(wl.num_users)) if users is None else list(users)
    if len(ulist) < 4:
        return O.sketch_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, users=ulist)
    with ThreadPoolExecutor(max_workers=4) as ex:
        parts = list(ex.map(lambda u: O.sketch_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, users=[u]),
                            ulist))
    return np.concatenate(parts, axis=0)


def _assert_parity(wl, got, users=None, tol=None):
    want = _oracle(wl, users)
    sel = got if users is None else got[list(users)]
    e, c = worst_errors(sel, want)
    tol = TOL[wl.dtype] if tol is None else tol
    print(f"[parity] {wl.name} users={'all' if users is None else list(users)} err={e:.3e} centred={c:.3e}", flush=True)
    assert e <= tol, (e, c)
    if c > tol:
        # only ill-conditioned centred sketches reach this: apply the weight-rounding allowance
        ulist = list(range(wl.num_users)) if users is None else list(users)
        for g, w, u in zip(sel, want, ulist):
            Xu = wl.user_rows(u).astype(np.float64)
            if Xu.shape[0] == 0:
                continue
            A = O.assignment(O.affinity(Xu, wl.P, wl.W_Q, wl.W_K, wl.tau))
            assert centred_within(g, w, A @ np.abs(Xu), tol, wl.dtype), (u, e, c)
    return e, c


def _assert_mass_identity(wl, got, tol=None):
    """sum_j X~_j = sum_i X_i for every user, normwise against the row sum."""
    tol = TOL[wl.dtype] if tol is None else tol
    worst = 0.0
    for u in range(wl.num_users):
        rows = wl.user_rows(u).astype(np.float64)
        if rows.shape[0] == 0:  # no behaviours: the sketch is all zeros
            assert not np.any(got[u]), u
            continue
        want = rows.sum(axis=0)
        have = got[u].astype(np.float64).sum(axis=0)
        scale = max(float(np.abs(want).max()), float(np.abs(rows).max()) * math.sqrt(max(rows.shape[0], 1)), 1e-30)
        worst = max(worst, float(np.abs(have - want).max()) / scale)
    print(f"[mass] {wl.name} worst={worst:.3e}", flush=True)
    assert worst <= tol


# ------------------------------------------------------- named workloads
def test_tiny_f32_full():
    wl = W.named_workload("tiny")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_recent_full():
    wl = W.named_workload("recent")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_long_full():
    wl = W.named_workload("long")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_many_proto_full():
    # every one of the 32 users element by element (the fp64 oracle takes ~2 s per
    # 100 000-row user at k = 1024, four users at a time)
    wl = W.named_workload("many_proto")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_ragged_full():
    # every one of the 64 users element by element, shortest and longest included
    wl = W.named_workload("ragged")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


# ------------------------------------------------------ shape sweeps
# Small sizes that still span several tiles and leave ragged tails; every
# plan of the fused kernel is exercised (k decides the plan).
SWEEP = [
    # (dtype, d, k, lengths)
    ("f32", 64, 1, [1, 37, 200]),
    ("f32", 64, 16, [1, 2, 3, 5, 17, 31, 32, 33, 127, 128, 129, 1000]),
    ("f32", 128, 33, [1, 64, 65, 300]),
    ("f32", 128, 64, [129, 257, 7]),
    ("f32", 64, 100, [2, 500, 33]),
    ("f32", 128, 256, [3, 300, 64]),
    ("bf16", 128, 1, [5, 129, 1000]),
    ("bf16", 64, 2, [1, 2, 3, 4, 5]),
    ("bf16", 128, 3, [17, 1000]),
    ("bf16", 64, 16, [1, 31, 32, 33, 1000]),
    ("bf16", 128, 33, [1, 127, 128, 129, 2000]),
    ("bf16", 128, 64, [2, 513, 1500]),
    ("bf16", 64, 65, [33, 999]),
    ("bf16", 128, 128, [1, 64, 4097]),
    ("bf16", 128, 200, [31, 1000, 3]),
    ("bf16", 64, 256, [32, 33, 2500]),
    ("bf16", 128, 300, [1, 1200]),
    ("bf16", 128, 512, [65, 1500]),
    ("bf16", 64, 700, [1, 800]),
    ("bf16", 64, 1024, [5, 3000]),
    ("bf16", 64, 50, [1, 300, 4099]),
    ("bf16", 64, 400, [70, 2600]),
]


@pytest.mark.parametrize("dtype,d,k,lengths", SWEEP, ids=lambda v: str(v))
def test_sweep(dtype, d, k, lengths):
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype=dtype, seed=7 * k + d, name=f"sweep-{dtype}-{d}-{k}")
    got = run_gpu(wl)
    _assert_parity(wl, got)


def test_empty_users_and_all_empty():
    wl = W.make_workload(lengths=[0, 5, 0, 0, 100, 0], d=128, k=64, dtype="bf16", seed=3, name="empties")
    got = run_gpu(wl)
    assert not got[0].any() and not got[2].any() and not got[3].any() and not got[5].any()
    _assert_parity(wl, got)
    wl0 = W.make_workload(lengths=[0, 0, 0], d=64, k=16, dtype="f32", seed=4, name="all-empty")
    X = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    got0 = run_gpu(wl0, X=X)
    assert got0.shape == (3, 16, 64) and not got0.any()


def test_zero_users_is_noop():
    wl = W.make_workload(lengths=[10], d=64, k=16, dtype="f32", seed=5)
    X, P, WQ, WK = to_device(wl)
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        buf = torch.full((1, 16, 64), 7.0, device="cuda")
        B.sa_compress_batch(sa.handle, X[:0], [0], buf[:0])  # [0, k, d] view of a sentinel buffer
        torch.cuda.synchronize()
    assert torch.all(buf == 7.0)


def test_more_users_than_one_launch():
    rng = np.random.default_rng(9)
    lengths = rng.integers(0, 40, size=600).tolist()
    wl = W.make_workload(lengths=lengths, d=64, k=48, dtype="bf16", seed=10, name="many-users")
    got = run_gpu(wl)
    _assert_parity(wl, got)


# ------------------------------------------------------- invariants on GPU
def test_deterministic_bitwise():
    wl = W.named_workload("recent", users=3)
    a = run_gpu(wl)
    b = run_gpu(wl)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_bound_call_matches_direct_call():
    """sa_compress_batch_bound (arguments checked once, the C call re-issued):
    the same bits as sa_compress_batch, and the offsets are the bound call's own
    copy (changing the caller's array afterwards changes nothing)."""
    wl = W.make_workload(lengths=[700, 0, 1500, 33], d=128, k=256, dtype="bf16", seed=71, name="bound")
    X, P, WQ, WK = to_device(wl)
    offs = np.array(wl.offsets, dtype=np.int64)
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        a = sa.compress(X, offs).clone()
        out = torch.empty_like(a)
        run = B.sa_compress_batch_bound(sa.handle, X, offs, out)
        offs[1:] = 0  # the caller's array is not read again
        for _ in range(3):
            out.zero_()
            run()
            torch.cuda.synchronize()
            assert torch.equal(out, a)


def test_additivity_across_users():
    """One user of n rows equals the sum of the same rows split into two users."""
    base = W.make_workload(lengths=[3001], d=128, k=128, dtype="bf16", seed=11, name="add")
    split = W.Workload(name="add-split", X=base.X, offsets=np.array([0, 1234, 3001], np.int64), P=base.P,
                       W_Q=base.W_Q, W_K=base.W_K, tau=base.tau, dtype="bf16")
    whole = run_gpu(base)[0].astype(np.float64)
    parts = run_gpu(split).astype(np.float64)
    assert normwise_err(parts[0] + parts[1], whole) <= 1e-5


def test_row_permutation_invariance():
    wl = W.make_workload(lengths=[5000], d=64, k=256, dtype="bf16", seed=12, name="perm")
    perm = np.random.default_rng(1).permutation(5000)
    wp = W.Workload(name="perm2", X=wl.X[perm], offsets=wl.offsets, P=wl.P, W_Q=wl.W_Q, W_K=wl.W_K, tau=wl.tau,
                    dtype="bf16")
    assert normwise_err(run_gpu(wp)[0], run_gpu(wl)[0].astype(np.float64)) <= 1e-4


def test_k1_is_row_sum():
    wl = W.make_workload(lengths=[777, 64], d=128, k=1, dtype="bf16", seed=13, name="k1")
    got = run_gpu(wl)
    for u in range(2):
        want = wl.user_rows(u).astype(np.float64).sum(axis=0)
        assert np.abs(got[u, 0] - want).max() <= 1e-4 * max(1.0, np.abs(want).max())


def test_wk_zero_gives_uniform_rows():
    wl = W.make_workload(lengths=[2000], d=64, k=300, dtype="bf16", seed=14, name="wk0")
    wl.W_K = np.zeros_like(wl.W_K)
    got = run_gpu(wl)[0]
    want = wl.X.astype(np.float64).sum(axis=0) / 300.0
    # every weight is bf16(1/300): the one rounding of the weights bounds the error
    assert np.abs(got - want[None, :]).max() <= 2.0 ** -8 * np.abs(want).max()


def test_large_tau_hard_assignment():
    """Scores far outside exp's range: the softmax must stay finite and exact."""
    wl = W.make_workload(lengths=[4000, 33], d=128, k=64, dtype="f32", seed=15, tau=40.0, name="hard-f32")
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)


@pytest.mark.parametrize("d,k,lengths", [
    (64, 257, [1, 300, 0, 65]),
    (128, 300, [700, 31, 33]),
    (64, 512, [129, 1000]),
    (128, 700, [40, 0, 999]),
    (128, 1000, [513, 64]),
    (64, 1024, [2, 777]),
])
def test_f32_beyond_256_two_phase(d, k, lengths):
    """float32 beyond 256 prototypes: the four-wave plan in two phases over
    blocks of 256 (per-block log-sum-exp, merge, aggregation with 2^(s' - L));
    parity at the float32 tolerance, padded and full blocks, ragged users."""
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="f32", seed=3 * k + d, name=f"f32-{d}-{k}")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_f32_two_phase_hard_assignment():
    """Scores far outside exp's range in both phases of the float32 two-phase
    pass: the statistics phase takes its exact path, the aggregation needs none."""
    wl = W.make_workload(lengths=[3000, 17], d=128, k=600, dtype="f32", seed=16, tau=40.0, name="hard-f32-600")
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)


def _hard_bf16_workload(lengths, d, k, tau, seed, spike_rows=None):
    """bf16-exact weights (P = 8 I, W_Q = W_K = I) and rows with one dominant
    coordinate: scores reach several hundred (far past exp2's range), yet the
    assignment is a clean argmax, so rounding cannot change the answer."""
    rng = np.random.default_rng(seed)
    n = int(sum(lengths))
    X = rng.standard_normal((n, d)).astype(np.float32)
    rows = np.arange(n) if spike_rows is None else spike_rows
    X[rows, rng.integers(0, min(d, k), rows.shape[0])] += 6.0
    X = W.round_to_bf16(X)
    P = np.zeros((k, d), np.float32)
    P[np.arange(min(k, d)), np.arange(min(k, d))] = 8.0
    eye = np.eye(d, dtype=np.float32)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return W.Workload(name="hard-bf16", X=X, offsets=offs, P=P, W_Q=eye, W_K=eye.copy(), tau=tau, dtype="bf16")


@pytest.mark.parametrize("d,k,plan", [(64, 64, "rows"), (64, 128, "mixed"), (64, 256, "prototypes"),
                                      (64, 700, "one score buffer, padded"), (64, 1024, "one score buffer"),
                                      (128, 300, "one score buffer, d=128")])
def test_exact_path_bf16(d, k, plan):
    """Every tile overflows the unshifted softmax and takes the exact path."""
    wl = _hard_bf16_workload([3000, 77, 1], d=d, k=k, tau=4.0, seed=19 + k)
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)


def test_exact_path_in_some_tiles_only():
    """Only a few rows have huge scores: their tiles go exact, the rest stay fast."""
    rng = np.random.default_rng(20)
    spikes = np.sort(rng.choice(5000, size=7, replace=False))
    wl = _hard_bf16_workload([5000], d=64, k=128, tau=4.0, seed=21, spike_rows=spikes)
    wl.X = W.round_to_bf16(wl.X * np.float32(0.05))     # ordinary rows: small scores
    wl.X[spikes] = W.round_to_bf16(wl.X[spikes] * np.float32(20.0))
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)


def test_moderately_large_tau_bf16():
    wl = W.make_workload(lengths=[3000], d=64, k=256, dtype="bf16", seed=18, tau=1.0, name="tau1-bf16")
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)


def test_fold_matches_definition():
    for dtype, d, k in (("bf16", 128, 256), ("f32", 64, 16), ("bf16", 64, 1024)):
        wl = W.make_workload(lengths=[1], d=d, k=k, dtype=dtype, seed=16)
        X, P, WQ, WK = to_device(wl)
        with SketchAttention(P, WQ, WK, wl.tau) as sa:
            M = sa.folded().cpu().numpy().astype(np.float64)
        want = wl.tau * math.log2(math.e) * O.fold_reference(wl.P, wl.W_Q, wl.W_K)
        tol = 2.0 ** -8 if dtype == "bf16" else 1e-5
        assert np.abs(M - want).max() <= tol * np.abs(want).max(), dtype


def test_kernel_timing_api():
    wl = W.named_workload("recent", users=2)
    X, P, WQ, WK = to_device(wl)
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        B.sa_set_kernel_timing(sa.handle, True)
        for _ in range(3):
            sa.compress(X, wl.offsets)
        f, r, n = B.sa_read_kernel_timing(sa.handle)
        assert n == 3 and f > 0 and r > 0
        f2, r2, n2 = B.sa_read_kernel_timing(sa.handle)
        assert n2 == 0 and f2 == 0
        plan = sa.plan(wl.total_rows)
        assert plan["k_padded"] >= 64 and plan["groups"] >= 1


def test_device_side_argument_errors():
    wl = W.make_workload(lengths=[10], d=64, k=16, dtype="bf16", seed=17)
    X, P, WQ, WK = to_device(wl)
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        out = torch.zeros((1, 16, 64), device="cuda")
        with pytest.raises(ValueError):
            B.sa_compress_batch(sa.handle, X, [0, 11], out)
        lib = B.library()
        offs = np.array([0, 4], np.int64)
        st = lib.sa_compress_batch(sa.handle, ctypes_ptr(X, 2), B._i64_ptr(offs), 1, ctypes_ptr(out), None)
        assert st == B.SA_ERR_INVALID_ARG      # misaligned X
        st = lib.sa_compress_batch(sa.handle, ctypes_ptr(X), B._i64_ptr(offs), 1, ctypes_ptr(out, 4), None)
        assert st == B.SA_ERR_INVALID_ARG      # misaligned out
        bad = np.array([0, 6, 4], np.int64)
        st = lib.sa_compress_batch(sa.handle, ctypes_ptr(X), B._i64_ptr(bad), 2, ctypes_ptr(out), None)
        assert st == B.SA_ERR_INVALID_ARG      # decreasing offsets
        torch.cuda.synchronize()
        assert torch.all(out == 0)


def ctypes_ptr(t, byte_offset=0):
    import ctypes
    return ctypes.c_void_p(t.data_ptr() + byte_offset)
