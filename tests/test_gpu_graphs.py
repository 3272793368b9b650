"""The C-ABI calls recorded in a HIP graph (torch.cuda.graph stream capture) and replayed.  Once an eager
call has sized a handle's buffers, a call allocates nothing, synchronises nothing and records kernel nodes
only, so it can be captured.  Every replay is checked bit for bit against an eager call on the same inputs,
with other inputs copied into the captured buffers between replays and eager work on the same handle in
between.  The float32 comparator, backward and action fusion are captured the same way."""
import numpy as np
import pytest
import torch

from sketch_attention_amd import ActionFusion, SketchAttention, SketchAttentionGrad, SketchStack
from sketch_attention_amd import workloads as W
from sa_testlib import to_device

pytestmark = pytest.mark.gpu

LENGTHS = [1500, 0, 2600, 7, 300]


def _pair(d, k, dtype="bf16"):
    a = W.make_workload(lengths=LENGTHS, d=d, k=k, dtype=dtype, seed=51, name="graph-a")
    b = W.make_workload(lengths=LENGTHS, d=d, k=k, dtype=dtype, seed=52, name="graph-b")
    return a, b


def _replay_and_check(g, feed, outs, refs, eager_between):
    """Three replays on inputs a, b, a (fed by `feed`), each compared with its eager reference."""
    for i, which in enumerate((0, 1, 0)):
        feed(which)
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs[which]):
            assert torch.equal(o, r), (i, which)
        eager_between()
        torch.cuda.synchronize()


def test_compress_replays():
    a, b = _pair(128, 256)
    Xa, P, WQ, WK = to_device(a)
    Xb = to_device(b)[0]
    with SketchAttention(P, WQ, WK, a.tau) as sa:
        refs = [[sa.compress(Xa, a.offsets).clone()], [sa.compress(Xb, a.offsets).clone()]]
        X = Xa.clone()
        out = torch.empty_like(refs[0][0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sa.compress(X, a.offsets, out=out)
        _replay_and_check(g, lambda w: X.copy_((Xa, Xb)[w]), [out], refs, lambda: sa.compress(Xb, a.offsets))


def test_stack_replays():
    a, b = _pair(128, 256)
    Xa, P, _, _ = to_device(a)
    Xb = to_device(b)[0]
    layers = []
    for lay in W.make_stack_layers(d=128, d_ff=256, layers=2, dtype="bf16", seed=53):
        layers.append({n: torch.from_numpy(np.ascontiguousarray(v)).to(
            "cuda", dtype=torch.bfloat16 if n in ("W_Q", "W_K") else torch.float32) for n, v in lay.items()})
    with SketchStack(P, layers, a.tau) as st:
        refs = [[st.compress(Xa, a.offsets).clone()], [st.compress(Xb, a.offsets).clone()]]
        X = Xa.clone()
        out = torch.empty_like(refs[0][0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.compress(X, a.offsets, out=out)
        _replay_and_check(g, lambda w: X.copy_((Xa, Xb)[w]), [out], refs, lambda: st.compress(Xb, a.offsets))


def test_action_fusion_replays():
    ia = W.make_action_inputs(5000, 128, 64, 256, 8, seed=54)
    ib = W.make_action_inputs(5000, 128, 64, 256, 8, seed=55)
    dev = lambda v, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(v)).to("cuda", dtype=dt)
    Ea, Eb = dev(ia["E"]), dev(ib["E"])
    Aa, Ab = dev(ia["actions"], torch.int32), dev(ib["actions"], torch.int32)
    with ActionFusion(dev(ia["table"]), dev(ia["W_gate"]), dev(ia["W_up"]), dev(ia["W_down"]), 8) as af:
        refs = [[af.fuse(Ea, Aa).clone()], [af.fuse(Eb, Ab).clone()]]
        E, A = Ea.clone(), Aa.clone()
        out = torch.empty_like(Ea)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            af.fuse(E, A, out=out)

        def feed(w):
            E.copy_((Ea, Eb)[w])
            A.copy_((Aa, Ab)[w])

        _replay_and_check(g, feed, [out], refs, lambda: af.fuse(Eb, Ab))


@pytest.mark.parametrize("lengths", [LENGTHS, [0, 0, 0]], ids=["rows", "empty_batch"])
def test_backward_replays(lengths):
    """The empty batch takes the path that zeroes the weight gradients (a kernel, not a memset node)."""
    a = W.make_workload(lengths=lengths, d=128, k=256, dtype="bf16", seed=56, name="graph-grad-a")
    b = W.make_workload(lengths=lengths, d=128, k=256, dtype="bf16", seed=57, name="graph-grad-b")
    Xa, P, WQ, WK = to_device(a)
    Xb = to_device(b)[0]
    Ga = torch.from_numpy(W.make_upstream_grad(len(lengths), 256, 128, seed=58)).cuda()
    Gb = torch.from_numpy(W.make_upstream_grad(len(lengths), 256, 128, seed=59)).cuda()
    with SketchAttentionGrad(P, WQ, WK, a.tau) as h:
        refs = [[t.clone() for t in h.backward(Xa, a.offsets, Ga)], [t.clone() for t in h.backward(Xb, a.offsets, Gb)]]
        X, G = Xa.clone(), Ga.clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            outs = h.backward(X, a.offsets, G)

        def feed(w):
            X.copy_((Xa, Xb)[w])
            G.copy_((Ga, Gb)[w])

        _replay_and_check(g, feed, list(outs), refs, lambda: h.backward(Xb, a.offsets, Gb))


def test_f32_comparator_replays():
    a = W.make_workload(lengths=LENGTHS, d=128, k=300, dtype="f32", seed=61, name="graph-f32-hist-a")
    b = W.make_workload(lengths=LENGTHS, d=128, k=300, dtype="f32", seed=62, name="graph-f32-hist-b")
    Xa, P, WQ, WK = to_device(a)
    Xb = to_device(b)[0]
    with SketchAttention(P, WQ, WK, a.tau, norm="history") as sa:
        refs = [[sa.compress(Xa, a.offsets).clone()], [sa.compress(Xb, a.offsets).clone()]]
        X = Xa.clone()
        out = torch.empty_like(refs[0][0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sa.compress(X, a.offsets, out=out)
        _replay_and_check(g, lambda w: X.copy_((Xa, Xb)[w]), [out], refs, lambda: sa.compress(Xb, a.offsets))


def test_f32_backward_replays():
    """The float32 backward's passes (products, softmax rows, transposes, the zero fill of its sum) record
    kernel nodes only once the handle's workspace has grown."""
    a = W.make_workload(lengths=LENGTHS, d=64, k=100, dtype="f32", seed=63, name="graph-f32-grad-a")
    b = W.make_workload(lengths=LENGTHS, d=64, k=100, dtype="f32", seed=64, name="graph-f32-grad-b")
    Xa, P, WQ, WK = to_device(a)
    Xb = to_device(b)[0]
    Ga = torch.from_numpy(W.make_upstream_grad(len(LENGTHS), 100, 64, seed=65)).cuda()
    Gb = torch.from_numpy(W.make_upstream_grad(len(LENGTHS), 100, 64, seed=66)).cuda()
    with SketchAttentionGrad(P, WQ, WK, a.tau) as h:
        refs = [[t.clone() for t in h.backward(Xa, a.offsets, Ga)], [t.clone() for t in h.backward(Xb, a.offsets, Gb)]]
        X, G = Xa.clone(), Ga.clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            outs = h.backward(X, a.offsets, G)

        def feed(w):
            X.copy_((Xa, Xb)[w])
            G.copy_((Ga, Gb)[w])

        _replay_and_check(g, feed, list(outs), refs, lambda: h.backward(Xb, a.offsets, Gb))


def test_f32_action_fusion_replays():
    ia = W.make_action_inputs(3000, 64, 8, 96, 5, seed=67)
    ib = W.make_action_inputs(3000, 64, 8, 96, 5, seed=68)
    dev = lambda v, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(v)).to("cuda", dtype=dt)
    Ea, Eb = dev(ia["E"]), dev(ib["E"])
    Aa, Ab = dev(ia["actions"], torch.int32), dev(ib["actions"], torch.int32)
    with ActionFusion(dev(ia["table"]), dev(ia["W_gate"]), dev(ia["W_up"]), dev(ia["W_down"]), 5) as af:
        refs = [[af.fuse(Ea, Aa).clone()], [af.fuse(Eb, Ab).clone()]]
        E, A = Ea.clone(), Aa.clone()
        out = torch.empty_like(Ea)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            af.fuse(E, A, out=out)

        def feed(w):
            E.copy_((Ea, Eb)[w])
            A.copy_((Aa, Ab)[w])

        _replay_and_check(g, feed, [out], refs, lambda: af.fuse(Eb, Ab))
