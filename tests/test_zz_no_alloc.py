"""sa_compress_batch_noalloc (the entry point that allocates nothing, its
partials in the library's fixed per-GPU array) against sa_compress_batch and
the oracle, through the C ABI: two calls in a row on one handle, the second
with a smaller batch, for a shape whose launch split is the same as the
allocating call's (bitwise equal) and one whose split differs (within the
parity tolerance).  Named to be collected last."""
import numpy as np
import pytest
import torch

from oracle import sa_oracle as SO
from sketch_attention_amd import SketchAttention, binding as B
from sketch_attention_amd import workloads as W
from sa_testlib import TOL, normwise_err, to_device

pytestmark = pytest.mark.gpu


def _both(sa, X, offsets, users, k, d):
    a = torch.full((users, k, d), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full((users, k, d), float("nan"), dtype=torch.float32, device="cuda")
    B.sa_compress_batch(sa.handle, X, offsets, a)
    B.sa_compress_batch_noalloc(sa.handle, X, offsets, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


@pytest.mark.parametrize("d,k,big,small,bitwise", [
    (128, 256, [30000, 0, 12345, 777], [5000, 64], True),       # same split as the allocating call
    (64, 1024, [9000, 1, 20000], [3000, 0, 17], False),         # 256 KB slots: fewer groups per launch
    (128, 1000, [9000, 0, 12000], [500, 3], True),              # two-phase pass: statistics in the array too
])
def test_noalloc_matches_the_allocating_call(d, k, big, small, bitwise):
    wl_big = W.make_workload(lengths=big, d=d, k=k, dtype="bf16", seed=71, name="noalloc-big")
    wl_small = W.make_workload(lengths=small, d=d, k=k, dtype="bf16", seed=71, name="noalloc-small")
    assert np.array_equal(wl_big.P, wl_small.P)
    Xb, P, WQ, WK = to_device(wl_big)
    Xs = to_device(wl_small)[0]
    with SketchAttention(P, WQ, WK, wl_big.tau) as sa:
        for wl, X in ((wl_big, Xb), (wl_small, Xs)):   # second call smaller than the first
            ref, got = _both(sa, X, wl.offsets, wl.num_users, k, d)
            assert np.all(np.isfinite(got))
            if bitwise:
                assert np.array_equal(ref, got)
            want = SO.sketch_batch(wl.X, wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau)
            for u in range(wl.num_users):
                assert normwise_err(got[u], want[u]) <= TOL["bf16"], u
                assert normwise_err(got[u], ref[u]) <= TOL["bf16"], u


def test_noalloc_many_users_and_empty():
    lengths = [int(x) for x in np.random.default_rng(5).integers(0, 300, size=600)]
    wl = W.make_workload(lengths=lengths, d=128, k=64, dtype="bf16", seed=72, name="noalloc-many")
    X, P, WQ, WK = to_device(wl)
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        ref, got = _both(sa, X, wl.offsets, wl.num_users, 64, 128)
        assert np.array_equal(ref, got)
        empty = W.make_workload(lengths=[0, 0], d=128, k=64, dtype="bf16", seed=72, name="noalloc-empty")
        ref, got = _both(sa, to_device(empty)[0], empty.offsets, 2, 64, 128)
        assert np.all(got == 0) and np.all(ref == 0)
