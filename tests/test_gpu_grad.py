"""Parity of the backward pass (sa_grad_compute through the C ABI) with the
fp64 gradient oracle.  Each gradient is compared normwise over the whole
tensor, max |G - O| / max |O| <= 2e-2 (bfloat16 operands, float32
accumulation; the upstream gradient is rounded to bfloat16 on the device).
Cases: every wave count of the statistics pass (k <= 64, <= 128, <= 256),
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


def _check(wl, G, got, tol=None, users=None):
    tol = TOL["bf16"] if tol is None else tol
    want = GO.sketch_grad_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, G, users=users)
    errs = {}
    for name, g in zip(("dX", "dP", "dW_Q", "dW_K"), got):
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
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grad_parity(case):
    name, d, k, lengths, extra = case
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype="bf16", seed=31, name=name, **extra)
    G = W.make_upstream_grad(len(lengths), k, d, seed=5)
    _check(wl, G, _run(wl, G))


def test_grad_spike_rows_take_the_shifted_path():
    """Rows scaled by 100 give scores of several hundred (log2 units): their
    unshifted sums overflow in the waves holding the top prototypes and
    underflow in the others, so the statistics pass redoes them with row
    maxima.  dX is compared at the usual tolerance (the spike rows' top two
    scores are >= 10 log2 units apart, so their assignment is well
    conditioned).  The weight gradients are not: dQ' weighs each spike row by
    |x|^2 = 10^4 times a runner-up weight <= 2^-10 whose relative error from
    the bf16 rounding of a score of ~400 (about 1 log2 unit) is O(1); they are
    only required to be finite here, and the shifted path's weight gradients
    are checked at normal scale by the forced-shift test below."""
    wl = W.make_workload(lengths=[3000, 500, 64], d=128, k=256, dtype="bf16", seed=13, name="spikes")
    # rows whose two best prototypes are >= 10 log2 units apart (checked against the oracle's scores)
    for r in (0, 1, 100, 102, 2999, 3000, 3002, 3499, 3500, 3563):
        wl.X[r] = W.round_to_bf16(wl.X[r] * 100.0)
    G = W.make_upstream_grad(3, 256, 128, seed=17)
    got = _run(wl, G)
    want = GO.sketch_grad_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau, G)
    e = _nerr(got[0], want["dX"])
    print(f"[grad] spikes dX {e:.3e}", flush=True)
    assert e <= TOL["bf16"], e
    for t in got[1:]:
        assert np.all(np.isfinite(t))


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("k256_d128", "k200_d128_pad", "k100_d64_pad",
                                                                 "k256_hot")], ids=lambda c: c[0])
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
