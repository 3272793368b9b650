"""sa_reserve on the GPU: a frozen handle gives, within its bounds, bitwise the
results of an unfrozen one, runs larger batches in launches sized to its
workspace, and a HIP graph captured from it still replays the same result
after a larger eager call (the workspace the graph uses never moves)."""
import numpy as np
import pytest
import torch

from sketch_attention_amd import SketchAttention
from sketch_attention_amd import workloads as W
from sa_testlib import normwise_err, to_device

pytestmark = pytest.mark.gpu


def _weights(wl):
    return to_device(wl)[1:]


def _ref(X, offsets, weights, tau):
    with SketchAttention(*weights, tau) as sa:
        out = sa.compress(X, offsets).clone()
        torch.cuda.synchronize()
    return out


def test_frozen_handle_matches_and_runs_larger_batches():
    small = W.make_workload(lengths=[1000, 0, 2000, 1500], d=128, k=256, dtype="bf16", seed=61, name="reserve-small")
    big = W.make_workload(lengths=[9000, 7, 12000, 3000, 500, 8000], d=128, k=256, dtype="bf16", seed=62,
                          name="reserve-big")
    weights = _weights(big)  # one set of weights for both batches
    X, Xb = to_device(small)[0], to_device(big)[0]
    want_small = _ref(X, small.offsets, weights, big.tau)
    want_big = _ref(Xb, big.offsets, weights, big.tau)
    with SketchAttention(*weights, big.tau) as sa:
        sa.reserve(int(small.offsets[-1]), small.num_users, freeze=True)
        got = sa.compress(X, small.offsets)
        torch.cuda.synchronize()
        assert torch.equal(got, want_small)          # within the bounds: the same launches, bitwise
        got_big = sa.compress(Xb, big.offsets)       # beyond them: launches sized to the frozen workspace
        torch.cuda.synchronize()
        for g, w in zip(got_big.cpu().numpy(), want_big.cpu().numpy()):
            assert normwise_err(g, w.astype(np.float64)) <= 1e-5
        sa.reserve(0, 0, freeze=False)                # growth on demand again
        assert torch.equal(sa.compress(Xb, big.offsets), want_big)
        torch.cuda.synchronize()


def test_graph_captured_on_a_frozen_handle_survives_a_larger_eager_call():
    small = W.make_workload(lengths=[3000, 1200], d=128, k=256, dtype="bf16", seed=63, name="reserve-graph")
    big = W.make_workload(lengths=[20000, 15000, 9000], d=128, k=256, dtype="bf16", seed=64, name="reserve-graph-big")
    X, P, WQ, WK = to_device(small)
    Xb = to_device(big)[0]
    with SketchAttention(P, WQ, WK, small.tau) as sa:
        sa.reserve(int(small.offsets[-1]), small.num_users, freeze=True)
        out = torch.empty((small.num_users, 256, 128), dtype=torch.float32, device="cuda")
        eager = sa.compress(X, small.offsets).clone()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sa.compress(X, small.offsets, out=out)   # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sa.compress(X, small.offsets, out=out)
        for rep in range(3):
            out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), rep
            sa.compress(Xb, big.offsets)              # eager, larger than the bounds
            torch.cuda.synchronize()
