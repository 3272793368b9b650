"""Parity of the stacked refinement (section 2.2) through the C ABI with the
fp64 CPU oracle: normwise error per user of X~(L), max |G - O| / max |O|,
within 2e-2 for bfloat16 inputs and 1e-4 for float32.  The cases cover every
kernel family the per-user folded matrices pass through: the streamed pass
with the matrix in registers and in LDS, the lockstep pass (bf16 with the
matrix in LDS, float32 in registers), several users per work group, and more
users than one launch carries."""
import numpy as np
import pytest
import torch

from oracle import refine_oracle as R
from sketch_attention_amd import SketchStack
from sketch_attention_amd import workloads as W
from sa_testlib import TOL, normwise_err, to_device

pytestmark = pytest.mark.gpu


def _layers_torch(layers, dtype, device="cuda"):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = []
    for lay in layers:
        t = {}
        for name, a in lay.items():
            want = dt if name in ("W_Q", "W_K") else torch.float32
            t[name] = torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=want)
        out.append(t)
    return out


def _oracle(wl, layers, users=None):
    params = [R.LayerParams(**{k: np.asarray(v, dtype=np.float64) for k, v in lay.items()}) for lay in layers]
    return R.stack_batch(wl.X, wl.offsets, wl.P, params, wl.tau, users=users)


def _run(wl, layers):
    X, P, _, _ = to_device(wl)
    with SketchStack(P, _layers_torch(layers, wl.dtype), wl.tau) as st:
        out = st.compress(X, wl.offsets)
        torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(wl, layers, users=None):
    got = _run(wl, layers)
    want = _oracle(wl, layers, users)
    sel = got if users is None else got[list(users)]
    err = max(normwise_err(g, w) for g, w in zip(sel, want))
    print(f"[stack] {wl.name} layers={len(layers)} err={err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[wl.dtype], err
    return got


CASES = [
    # dtype, d, k, d_ff, layers, lengths
    ("bf16", 128, 64, 256, 2, [1, 200, 3000, 0, 77]),        # streamed, matrix in registers, 4-wave groups
    ("bf16", 128, 256, 512, 2, [1500, 10, 4097]),            # streamed, eight waves (the long workload's plan)
    ("bf16", 128, 300, 256, 3, [50, 2000]),                  # streamed, matrix in LDS
    ("bf16", 128, 1000, 256, 2, [1200, 0, 3000, 1]),         # two-phase pass (the page's final configuration)
    ("bf16", 64, 700, 128, 2, [300, 2, 1000]),               # streamed, matrix in LDS, d = 64
    ("bf16", 64, 16, 128, 2, [5, 100, 0]),                   # lockstep, matrix in LDS
    ("f32", 64, 16, 64, 2, [1, 100, 33]),                    # lockstep float32, matrix in registers
    ("f32", 128, 100, 128, 1, [7, 300]),                     # one layer
    ("f32", 128, 600, 128, 2, [400, 0, 97]),                 # float32 two-phase pass, per-user matrices
]


@pytest.mark.parametrize("dtype,d,k,d_ff,nl,lengths", CASES, ids=lambda v: str(v))
def test_stack_parity(dtype, d, k, d_ff, nl, lengths):
    wl = W.make_workload(lengths=lengths, d=d, k=k, dtype=dtype, seed=31 * k + d, name=f"stack-{dtype}-{d}-{k}")
    layers = W.make_stack_layers(d=d, d_ff=d_ff, layers=nl, dtype=dtype, seed=k + nl)
    _check(wl, layers)


def test_stack_many_short_users_share_groups():
    # 300 users of 1..150 rows: several users per work group (the per-user matrix changes inside a
    # group's tile list) and two launches (at most 256 users per launch)
    lengths = list(np.random.default_rng(5).integers(1, 151, size=300))
    wl = W.make_workload(lengths=lengths, d=64, k=64, dtype="bf16", seed=9, name="stack-many-users")
    layers = W.make_stack_layers(d=64, d_ff=128, layers=2, dtype="bf16", seed=4)
    _check(wl, layers, users=None)


def test_stack_long_workload_sampled_user():
    # the long workload's shape (4 users x 100000 rows, d = 128, k = 256), two layers of width 512;
    # the oracle checks user 2 (a user in the middle of the batch)
    wl = W.named_workload("long")
    layers = W.make_stack_layers(d=128, d_ff=512, layers=2, dtype="bf16", seed=17)
    _check(wl, layers, users=[2])


def test_stack_repeat_calls_and_growth():
    # a smaller batch after a larger one reuses the buffers; results match a fresh handle
    wl_a = W.make_workload(lengths=[400, 900, 50], d=128, k=64, dtype="bf16", seed=1, name="a")
    wl_b = W.make_workload(lengths=[300], d=128, k=64, dtype="bf16", seed=2, name="b")
    layers = W.make_stack_layers(d=128, d_ff=128, layers=2, dtype="bf16", seed=3)
    Xa, P, _, _ = to_device(wl_a)
    Xb, _, _, _ = to_device(wl_b)
    lt = _layers_torch(layers, "bf16")
    with SketchStack(P, lt, wl_a.tau) as st:
        st.compress(Xa, wl_a.offsets)
        again_b = st.compress(Xb, wl_b.offsets)
        torch.cuda.synchronize()
    with SketchStack(P, lt, wl_a.tau) as st:
        fresh_b = st.compress(Xb, wl_b.offsets)
        torch.cuda.synchronize()
    assert torch.equal(again_b, fresh_b)
