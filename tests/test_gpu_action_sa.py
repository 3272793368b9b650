"""The action fusion as the prologue of the compression pass
(sa_action_compress_batch through the C ABI): the rows x_i = e_i +
SwiGLU-FFN([e_i; a_i]) (SequenceO1 close reading, section 2.2) are formed
inside the sketch kernel and never written.

Two bars:
  * bit for bit the result of the two-pass path (sa_action_fuse, then
    sa_compress_batch on the same handle: same work split, same instructions
    in the same order), on ragged batches, padded prototypes (k < 256), both
    K paddings of the FFN (d_a = 64 and 128), odd and even FFN chunk counts,
    a batch of more users than one launch takes, rows whose totals leave the
    unshifted softmax's range (the exact pass), and the full bench shape;
  * per user normwise within 2e-2 of the fp64 oracle sketch of the fp64
    oracle's rows (rounded to bf16 like the device rows), as for the
    two-pass path in test_gpu_action.py.
"""
import numpy as np
import pytest
import torch

from oracle import action_oracle as AO
from oracle import sa_oracle as O
from sketch_attention_amd import ActionFusion, SketchAttention
from sketch_attention_amd import workloads as W
from sketch_attention_amd.binding import SAError, SA_ERR_UNSUPPORTED, sa_read_kernel_timing, sa_set_kernel_timing
from sa_testlib import TOL

pytestmark = pytest.mark.gpu


def _dev(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dtype)


def _both(inp, n_act, wl):
    """(fused, two-pass) sketches of the action rows of inp under wl's weights, and the device rows."""
    d_a = inp["table"].shape[1]
    with ActionFusion(_dev(inp["table"]) if d_a else None, _dev(inp["W_gate"]), _dev(inp["W_up"]),
                      _dev(inp["W_down"]), n_act) as af, \
            SketchAttention(_dev(wl.P), _dev(wl.W_Q), _dev(wl.W_K), wl.tau) as sa:
        E, acts = _dev(inp["E"]), _dev(inp["actions"], torch.int32)
        U, k, d = wl.offsets.size - 1, wl.P.shape[0], wl.P.shape[1]
        fused = torch.full((U, k, d), float("nan"), device="cuda")
        af.compress(sa, E, acts, wl.offsets, out=fused)
        X = af.fuse(E, acts)
        two = sa.compress(X, wl.offsets)
        torch.cuda.synchronize()
    return fused.cpu().numpy(), two.cpu().numpy(), X.float().cpu().numpy()


def _oracle_check(name, inp, wl, got):
    x_or = AO.action_fuse(inp["E"], inp["actions"], inp["table"], inp["W_gate"], inp["W_up"], inp["W_down"])
    want = O.sketch_batch(W.round_to_bf16(x_or.astype(np.float32)), wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau)
    worst = 0.0
    for g, w in zip(got, want):
        den = max(float(np.abs(w).max()), 1e-30)
        worst = max(worst, float(np.abs(g - w).max()) / den)
    print(f"[action-sa] {name} worst per-user normwise err vs oracle {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"], worst


CASES = [
    # name, lengths, k, d_a, d_ff, n_actions
    ("ragged_k256_da64_ff256", [700, 0, 1300], 256, 64, 256, 8),
    ("padded_k200_da128_ff96", [513, 1, 64, 0, 1000], 200, 128, 96, 5),
    ("k129_da0_ff128", [2000], 129, 0, 128, 1),
    ("odd_tiles_k256_da32_ff64", [65, 63, 127, 129, 3], 256, 32, 64, 1000),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_two_pass_and_oracle(case):
    name, lengths, k, d_a, d_ff, n_act = case
    rows = int(sum(lengths))
    inp = W.make_action_inputs(rows, 128, d_a, d_ff, n_act, seed=rows + k)
    wl = W.make_workload(lengths=lengths, d=128, k=k, dtype="bf16", seed=k + d_ff, name=name)
    fused, two, _ = _both(inp, n_act, wl)
    assert np.isfinite(fused).all()
    assert np.array_equal(fused, two), float(np.abs(fused - two).max())
    _oracle_check(name, inp, wl, fused)


def test_fused_more_users_than_one_launch():
    """300 users (two launches of the batch loop), a third of them empty."""
    rng = np.random.default_rng(5)
    lengths = [int(v) if i % 3 else 0 for i, v in enumerate(rng.integers(1, 90, size=300))]
    inp = W.make_action_inputs(int(sum(lengths)), 128, 64, 128, 8, seed=31)
    wl = W.make_workload(lengths=lengths, d=128, k=256, dtype="bf16", seed=32, name="many-users")
    fused, two, _ = _both(inp, 8, wl)
    assert np.array_equal(fused, two)
    assert np.all(fused[[i for i, n in enumerate(lengths) if n == 0]] == 0.0)


def test_fused_exact_pass():
    """Scores of several hundred (P = 8 I, W_Q = W_K = I, tau = 4, one dominant coordinate per row of E that
    the small FFN update keeps): every tile takes the exact pass.  Bitwise against the two-pass path, and
    against the oracle sketch of the rows the device formed."""
    lengths, k, d = [3000, 77, 1], 256, 128
    rows = sum(lengths)
    inp = W.make_action_inputs(rows, d, 64, 128, 8, seed=41)
    rng = np.random.default_rng(42)
    E = inp["E"].copy()
    E[np.arange(rows), rng.integers(0, d, rows)] += 6.0
    inp["E"] = W.round_to_bf16(E)
    P = np.zeros((k, d), np.float32)
    P[np.arange(d), np.arange(d)] = 8.0
    eye = np.eye(d, dtype=np.float32)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    wl = W.Workload(name="hard-actions", X=None, offsets=offs, P=P, W_Q=eye, W_K=eye.copy(), tau=4.0, dtype="bf16")
    fused, two, X = _both(inp, 8, wl)
    assert np.isfinite(fused).all()
    assert np.array_equal(fused, two)
    want = O.sketch_batch(X, offs, P, eye, eye, 4.0)
    for g, w in zip(fused, want):
        assert float(np.abs(g - w).max()) <= TOL["bf16"] * max(float(np.abs(w).max()), 1e-30)


def test_fused_full_bench_shape():
    """4 users x 100 000 rows, k = 256, d_a = 64, d_ff = 256 (the shape bench.py --actions times): bitwise
    against the two-pass path for every user, and the first user against the oracle."""
    lengths = [100_000] * 4
    rows = sum(lengths)
    inp = W.make_action_inputs(rows, 128, 64, 256, 8, seed=7)
    wl = W.make_workload(lengths=lengths, d=128, k=256, dtype="bf16", seed=8, name="bench-actions")
    fused, two, _ = _both(inp, 8, wl)
    assert np.array_equal(fused, two)
    n0 = lengths[0]
    sub = {key: (v[:n0] if key in ("E", "actions") else v) for key, v in inp.items()}
    wl0 = W.Workload(name="bench-user0", X=None, offsets=np.array([0, n0], np.int64), P=wl.P, W_Q=wl.W_Q,
                     W_K=wl.W_K, tau=wl.tau, dtype="bf16")
    _oracle_check("bench_user0", sub, wl0, fused[:1])


def test_fused_unsupported_plans_enqueue_nothing():
    inp = W.make_action_inputs(100, 128, 64, 128, 8, seed=1)
    out = torch.full((1, 64, 128), 7.0, device="cuda")
    wl = W.make_workload(lengths=[100], d=128, k=64, dtype="bf16", seed=2, name="k64")
    with ActionFusion(_dev(inp["table"]), _dev(inp["W_gate"]), _dev(inp["W_up"]), _dev(inp["W_down"]), 8) as af, \
            SketchAttention(_dev(wl.P), _dev(wl.W_Q), _dev(wl.W_K), wl.tau) as sa:
        with pytest.raises(SAError) as e:
            af.compress(sa, _dev(inp["E"]), _dev(inp["actions"], torch.int32), wl.offsets, out=out)
        assert e.value.status == SA_ERR_UNSUPPORTED
        torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_fused_kernel_timing_on_the_sketch_handle():
    lengths = [5000, 3000]
    inp = W.make_action_inputs(sum(lengths), 128, 64, 256, 8, seed=11)
    wl = W.make_workload(lengths=lengths, d=128, k=256, dtype="bf16", seed=12, name="timed")
    with ActionFusion(_dev(inp["table"]), _dev(inp["W_gate"]), _dev(inp["W_up"]), _dev(inp["W_down"]), 8) as af, \
            SketchAttention(_dev(wl.P), _dev(wl.W_Q), _dev(wl.W_K), wl.tau) as sa:
        E, acts = _dev(inp["E"]), _dev(inp["actions"], torch.int32)
        sa_set_kernel_timing(sa.handle, True)
        for _ in range(3):
            af.compress(sa, E, acts, wl.offsets)
        fused_ms, reduce_ms, launches = sa_read_kernel_timing(sa.handle)
    assert launches == 3 and fused_ms > 0.0 and reduce_ms > 0.0
