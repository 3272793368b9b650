"""Parity of the backward pass (sa_grad_compute through the C ABI) with the
fp64 gradient oracle, normwise as for the forward: dX per user (max |G - O|
over the user's rows / max |O| over them), the weight gradients (sums over
the batch's users) over the whole tensor; <= 2e-2 (bfloat16 operands,
float32 accumulation; the upstream gradient is rounded to bfloat16 on the
device).
Cases: every wave count of the statistics pass (k <= 64, <= 128, <= 256),
two to four blocks of 256 prototypes walked in two phases (k up to 1024),
both widths, padded prototype counts, ragged and empty users, users shorter
than a tile, peaked assignments, more users than one launch carries, an empty
batch, repeated calls on one handle, and the full long workload."""
import numpy as np
import pytest
import torch

from oracle import grad_oracle as GO
from sketch_attention_amd import SketchAttentionGrad
from sketch_attention_amd import workloads as W
from sa_testlib import TOL, to_device

pytestmark = pytest.mark.gpu


def _nerr(got, want):
    den = float(np.max(np.abs(want))) if want.size else 0.0
    num = float(np.max(np.abs(got.astype(np.float64) - want))) if want.size else 0.0
    return num / den if den > 0 else num


def _run(wl, G, handle=None):
    X, P, WQ, WK = to_device(wl)
    Gd = torch.from_numpy(G).cuda()
    own = handle is None
    h = SketchAttentionGrad(P, WQ, WK, wl.tau) if own else handle
    try:
        out = h.backward(X, wl.offsets, Gd)
        torch.cuda.synchronize()
    finally:
        if own:
            h.close()
    return [t.float().cpu().numpy() for t in out]


def _dx_err(wl, got, want, users=None):
    """Worst per-user normwise error of dX (users without rows skipped)."""
    worst = 0.0
    for u in (range(wl.num_users) if users is None else users):
        a, b = int(wl.offsets[u]), int(wl.offsets[u + 1])
        if b > a:
            worst = max(worst, _nerr(got[a:b], want[a:b]))
    return worst


def _check(wl, G, got, tol=None, users=None):
    tol = TOL["bf16"] if tol is None else tol
    want = GO.sketch_grad_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, G, users=users)
    errs = {"dX": _dx_err(wl, got[0], want["dX"], users)}
    for name, g in zip(("dP", "dW_Q", "dW_K"), got[1:]):
        errs[name] = _nerr(g, want[name])
    print(f"[grad] {wl.name} {errs}", flush=True)
    for name, e in errs.items():
        assert e <= tol, (name, e)
    return errs


CASES = [
    # name, d, k, lengths, extra
    ("k256_d128", 128, 256, [700, 0, 1, 77, 1500, 31, 32, 33], {}),
    ("k128_d128", 128, 128, [900, 45, 0, 2000], {}),
    ("k64_d128", 128, 64, [513, 1, 1024], {}),
    ("k200_d128_pad", 128, 200, [640, 7, 1280], {}),
    ("k33_d128_pad", 128, 33, [300, 301], {}),
    ("k1_d128", 128, 1, [129, 5], {}),
    ("k256_d64", 64, 256, [1100, 0, 64, 900], {}),
    ("k100_d64_pad", 64, 100, [777, 333], {}),
    ("k256_hot", 128, 256, [1200, 800], dict(x_scale=6.0)),
    ("k256_clusters_dup", 128, 256, [2048, 600], dict(x_kind="clusters", dup_fraction=0.3)),
    ("k300_d128_pad", 128, 300, [900, 3, 0, 1500], {}),
    ("k512_d128", 128, 512, [1100, 640], {}),
    ("k1000_d128_pad", 128, 1000, [700, 1, 1300], {}),
    ("k1024_d128", 128, 1024, [1500, 33], {}),
    ("k1024_d64", 64, 1024, [600, 0, 900], {}),
    ("k1000_clusters", 128, 1000, [1600, 500], dict(x_kind="clusters")),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grad_parity(case):
    name, d, k, lengths, extra = case
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="bf16", seed=31, name=name, **extra)
    G = W.make_upstream_grad(len(lengths), k, d, seed=5)
    _check(wl, G, _run(wl, G))


@pytest.mark.parametrize("k", [256, 1000])
def test_grad_spike_rows_take_the_shifted_path(k):
    """Rows scaled by 100 give scores of several hundred (log2 units): their
    unshifted sums overflow in the waves holding the top prototypes and
    underflow in the others, so the statistics pass redoes them with row
    maxima.  The spike rows are those whose two best prototypes are at least
    1.7 log2 units apart before scaling (>= 170 after, per the oracle's
    scores), so every other weight of such a row is below 2^-150 in float64
    and float32 alike.  Their assignment is then well conditioned: the bf16
    rounding of the folded matrix moves a score of ~600 by ~1 log2 unit,
    which cannot lift a runner-up out of that range, while a wrong maximum,
    sum or log-sum-exp in the shifted path puts mass on it and shows in dX and
    in the weight gradients, which weigh each spike row by |x|^2 ~ 10^4.  All
    four gradients are compared at the usual tolerance."""
    from oracle import sa_oracle as SO

    wl = W.make_workload(lengths=[3000, 500, 64], d=128, k=k, dtype="bf16", seed=13, name=f"spikes{k}")
    s = np.sort(SO.affinity(wl.X, wl.P, wl.W_Q, wl.W_K, wl.tau), axis=0) / np.log(2.0)
    gap = s[-1] - s[-2]
    rows = []
    for u in range(wl.num_users):
        a, b = int(wl.offsets[u]), int(wl.offsets[u + 1])
        rows += [int(r) for r in np.nonzero(gap[a:b] >= 1.7)[0][:4] + a]
    assert len(rows) >= 8, rows
    for r in rows:
        wl.X[r] = W.round_to_bf16(wl.X[r] * 100.0)
    top = (np.sort(SO.affinity(wl.X[rows], wl.P, wl.W_Q, wl.W_K, wl.tau), axis=0) / np.log(2.0))[-1]
    assert np.all(top > 300.0), top  # far outside the unshifted range [2^-100, 2^100]
    G = W.make_upstream_grad(3, k, 128, seed=17)
    _check(wl, G, _run(wl, G))


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("k256_d128", "k200_d128_pad", "k100_d64_pad",
                                                                 "k256_hot", "k1000_d128_pad", "k1024_d64")],
                         ids=lambda c: c[0])
def test_grad_forced_shift_path(case, monkeypatch):
    """Every row block through the statistics pass's shifted path (its fallback
    for extreme scores), at normal scale, all four gradients at tolerance."""
    monkeypatch.setenv("SA_GRAD_FORCE_SHIFT", "1")
    name, d, k, lengths, extra = case
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="bf16", seed=31, name=name + "_shift", **extra)
    G = W.make_upstream_grad(len(lengths), k, d, seed=5)
    _check(wl, G, _run(wl, G))


def test_grad_many_users_two_launches():
    rng = np.random.default_rng(3)
    lengths = [int(x) for x in rng.integers(0, 60, size=300)]
    wl = W.make_workload(lengths=lengths, d=128, k=96, dtype="bf16", seed=4, name="many_users")
    G = W.make_upstream_grad(300, 96, 128, seed=8)
    _check(wl, G, _run(wl, G))


def test_grad_empty_batches():
    for lengths in ([], [0, 0, 0]):
        wl = W.make_workload(lengths=lengths, d=128, k=64, dtype="bf16", seed=2, name="empty")
        G = W.make_upstream_grad(len(lengths), 64, 128, seed=1)
        gX, gP, gQ, gK = _run(wl, G)
        assert gX.shape == (0, 128)
        for t in (gP, gQ, gK):
            assert np.all(t == 0)


def test_grad_repeated_calls_one_handle():
    big = W.make_workload(lengths=[3000, 500], d=128, k=256, dtype="bf16", seed=9, name="big")
    small = W.make_workload(lengths=[40, 0, 90], d=128, k=256, dtype="bf16", seed=9, name="small")
    small_same = W.make_workload(lengths=[40, 0, 90], d=128, k=256, dtype="bf16", seed=9, name="small")
    assert np.array_equal(small.P, big.P)
    X, P, WQ, WK = to_device(big)
    with SketchAttentionGrad(P, WQ, WK, big.tau) as h:
        for wl in (small, big, small_same):
            G = W.make_upstream_grad(wl.num_users, 256, 128, seed=11)
            _check(wl, G, _run(wl, G, handle=h))


def test_grad_long_full():
    wl = W.named_workload("long")
    G = W.make_upstream_grad(wl.num_users, wl.P.shape[0], wl.P.shape[1], seed=0)
    _check(wl, G, _run(wl, G))


def test_grad_many_proto_full_sampled():
    """The many-prototype workload at full size (32 users x 100K rows, d = 64,
    k = 1024: four blocks of 256 prototypes in two phases).  dX of two users
    against the oracle on those users; the weight gradients, sums over all
    3.2M rows, through additivity over users (the batch's gradients equal the
    sum of those of its two halves, each run on its own), which holds at any
    size."""
    wl = W.named_workload("many_proto")
    k, d = wl.P.shape
    G = W.make_upstream_grad(wl.num_users, k, d, seed=3)
    X, P, WQ, WK = to_device(wl)
    Gd = torch.from_numpy(G).cuda()
    users = [0, wl.num_users - 1]
    half = wl.num_users // 2
    off = np.asarray(wl.offsets, dtype=np.int64)
    with SketchAttentionGrad(P, WQ, WK, wl.tau) as h:
        full = [t.float().cpu().numpy() for t in h.backward(X, off, Gd)]
        lo = [t.float().cpu().numpy() for t in h.backward(X[: off[half]], off[: half + 1], Gd[:half])]
        hi = [t.float().cpu().numpy() for t in h.backward(X[off[half]:], off[half:] - off[half], Gd[half:])]
        torch.cuda.synchronize()
    want = GO.sketch_grad_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, G, users=users)
    e_dx = _dx_err(wl, full[0], want["dX"], users)
    e_add = [_nerr(f, a + b) for f, a, b in zip(full[1:], lo[1:], hi[1:])]
    e_dx_half = _nerr(full[0], np.concatenate([lo[0], hi[0]]))
    print(f"[grad] many_proto dX(sampled)={e_dx:.3e} additivity={e_add} dX halves={e_dx_half:.3e}", flush=True)
    assert e_dx <= TOL["bf16"]
    assert e_dx_half == 0.0  # a user's rows see the same kernels either way
    for e in e_add:
        assert e <= 1e-5, e_add  # float32 sums in another order


def test_grad_is_bitwise_deterministic():
    """Fixed-order reductions: two calls on the same inputs give identical bits."""
    wl = W.make_workload(lengths=[5000, 1, 2500], d=128, k=200, dtype="bf16", seed=44, name="det")
    G = W.make_upstream_grad(3, 200, 128, seed=45)
    X, P, WQ, WK = to_device(wl)
    Gd = torch.from_numpy(G).cuda()
    with SketchAttentionGrad(P, WQ, WK, wl.tau) as h:
        a = [t.clone() for t in h.backward(X, wl.offsets, Gd)]
        b = h.backward(X, wl.offsets, Gd)
        torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


F32_CASES = [
    # name, d, k, lengths: float32 inputs and gradients, per-user passes of at most 65536 rows
    ("f32_k16_d64", 64, 16, [1000, 0, 3]),
    ("f32_k1_d128", 128, 1, [129, 5]),
    ("f32_k100_d128_pad", 128, 100, [700, 0, 1, 1500]),
    ("f32_k256_d64", 64, 256, [300, 64]),
    ("f32_k1024_d128", 128, 1024, [600, 33]),
    ("f32_k300_two_passes", 128, 300, [70000, 10]),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_grad_f32_parity(case):
    """All four gradients within 1e-4 normwise (dX per user) of the fp64 oracle."""
    name, d, k, lengths = case
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="f32", seed=41, name=name)
    G = W.make_upstream_grad(len(lengths), k, d, seed=9)
    _check(wl, G, _run(wl, G), tol=TOL["f32"])


def test_grad_f32_empty_batch_and_repeat():
    wl = W.make_workload(lengths=[0, 0], d=64, k=32, dtype="f32", seed=2, name="f32_empty")
    G = W.make_upstream_grad(2, 32, 64, seed=1)
    got = _run(wl, G)
    for t in got[1:]:
        assert not np.any(t)
    wl2 = W.make_workload(lengths=[400, 90], d=64, k=32, dtype="f32", seed=3, name="f32_after_empty")
    X, P, WQ, WK = to_device(wl2)
    with SketchAttentionGrad(P, WQ, WK, wl2.tau) as h:
        for _ in range(2):  # the same handle twice: the workspace is reused
            out = [t.float().cpu().numpy() for t in h.backward(X, wl2.offsets, torch.from_numpy(G).cuda())]
            torch.cuda.synchronize()
            _check(wl2, G, out, tol=TOL["f32"])
