"""Parity of the action-fusion pass (sa_action_fuse through the C ABI) with
the fp64 oracle x = e + SwiGLU-FFN([e; table[action]]) (SequenceO1 close
reading, section 2.2).  The FFN part is compared normwise,
max |(X - E) - (x - e)| <= 2e-2 max |x - e| + 2^-8 max |x| (bf16 operands,
float32 accumulation, and the one rounding of x to bf16 on output).  Cases:
every K padding (d + d_a up to 64, 128, 192, 256), both widths, one and two
FFN chunks per step, a single action type, many action types, row counts
around the 256-row tile and the work-group split, clamped action ids, and
the action-fused rows feeding the compression."""
import numpy as np
import pytest
import torch

from oracle import action_oracle as AO
from oracle import sa_oracle as O
from sketch_attention_amd import ActionFusion, SketchAttention
from sketch_attention_amd import workloads as W
from sa_testlib import TOL

pytestmark = pytest.mark.gpu


def _dev(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dtype)


def _run(inp, n_actions, actions=None):
    acts = inp["actions"] if actions is None else actions
    d_a = inp["table"].shape[1]
    with ActionFusion(_dev(inp["table"]) if d_a else None, _dev(inp["W_gate"]), _dev(inp["W_up"]),
                      _dev(inp["W_down"]), n_actions) as af:
        X = af.fuse(_dev(inp["E"]), _dev(acts, torch.int32))
        torch.cuda.synchronize()
    return X.float().cpu().numpy()


def _check(name, inp, got, actions=None):
    acts = inp["actions"] if actions is None else actions
    want = AO.action_fuse(inp["E"], acts, inp["table"], inp["W_gate"], inp["W_up"], inp["W_down"])
    f_want = want - inp["E"]
    f_got = got.astype(np.float64) - inp["E"]
    err = float(np.abs(f_got - f_want).max())
    bound = TOL["bf16"] * float(np.abs(f_want).max()) + 2.0 ** -8 * float(np.abs(want).max())
    print(f"[action] {name} err={err:.3e} bound={bound:.3e} rel={err / max(float(np.abs(f_want).max()), 1e-30):.3e}",
          flush=True)
    assert err <= bound, (err, bound)


CASES = [
    # name, rows, d, d_a, d_ff, n_actions
    ("d128_da64_ff256", 3000, 128, 64, 256, 8),
    ("d128_da0_ff128", 777, 128, 0, 128, 1),
    ("d128_da128_ff96", 513, 128, 128, 96, 5),     # K 256: one chunk per step, d_ff a multiple of 32
    ("d128_da32_ff512", 257, 128, 32, 512, 1000),  # K 192
    ("d64_da64_ff256", 1000, 64, 64, 256, 16),     # K 128
    ("d64_da0_ff64", 255, 64, 0, 64, 3),           # K 64
    ("d64_da192_ff128", 300, 64, 192, 128, 7),     # K 256
    ("one_row", 1, 128, 64, 128, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_action_parity(case):
    name, rows, d, d_a, d_ff, n_act = case
    inp = W.make_action_inputs(rows, d, d_a, d_ff, n_act, seed=rows)
    _check(name, inp, _run(inp, n_act))


def test_action_ids_out_of_range_are_clamped():
    inp = W.make_action_inputs(600, 128, 64, 128, 6, seed=3)
    acts = inp["actions"].copy()
    acts[::7] = -3
    acts[3::11] = 6 + 40
    got = _run(inp, 6, actions=acts)
    _check("clamped", inp, got, actions=np.clip(acts, 0, 5))


def test_action_rows_feed_the_compression():
    """x from the fused pass, then the sketch of section 2.1 on it: compared
    with the oracle sketch of the oracle's x (bf16-rounded like the device rows)."""
    lengths = [700, 0, 1300]
    rows = sum(lengths)
    inp = W.make_action_inputs(rows, 128, 64, 256, 8, seed=21)
    wl = W.make_workload(lengths=lengths, d=128, k=256, dtype="bf16", seed=22, name="actions")
    x_dev = _run(inp, 8)
    x_or = AO.action_fuse(inp["E"], inp["actions"], inp["table"], inp["W_gate"], inp["W_up"], inp["W_down"])
    with SketchAttention(_dev(wl.P), _dev(wl.W_Q), _dev(wl.W_K), wl.tau) as sa:
        got = sa.compress(_dev(x_dev), wl.offsets).cpu().numpy()
    want = O.sketch_batch(W.round_to_bf16(x_or.astype(np.float32)), wl.offsets, wl.P, wl.W_Q, wl.W_K, wl.tau)
    for g, w in zip(got, want):
        den = max(float(np.abs(w).max()), 1e-30)
        assert float(np.abs(g - w).max()) / den <= TOL["bf16"]


def test_action_fusion_is_bitwise_deterministic():
    inp = W.make_action_inputs(2000, 128, 64, 256, 8, seed=9)
    with ActionFusion(_dev(inp["table"]), _dev(inp["W_gate"]), _dev(inp["W_up"]), _dev(inp["W_down"]), 8) as af:
        E, acts = _dev(inp["E"]), _dev(inp["actions"], torch.int32)
        a = af.fuse(E, acts).clone()
        b = af.fuse(E, acts)
        torch.cuda.synchronize()
    assert torch.equal(a, b)


FULL_CASES = [
    # name, rows, d, d_a, d_ff, n_actions: row counts large enough that every work group walks several
    # 256-row tiles (the action ids and E rows of the next tile are loaded while the current one runs)
    ("bench_shape_400k", 400_000, 128, 64, 256, 8),   # the shape bench.py --actions times
    ("ragged_300007", 300_007, 128, 64, 256, 8),
    ("d128_da128_ff96_100003", 100_003, 128, 128, 96, 5),  # K 256: one chunk per step, no E prefetch
    ("d64_da64_ff128_70001", 70_001, 64, 64, 128, 16),
]


@pytest.mark.parametrize("case", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_action_full_size(case):
    """Every row of a full-size pass against the oracle (computed in blocks of rows), with the normwise
    bound of the small cases; the device output starts as NaN so that a row the pass never wrote fails."""
    name, rows, d, d_a, d_ff, n_act = case
    inp = W.make_action_inputs(rows, d, d_a, d_ff, n_act, seed=rows % 1000)
    with ActionFusion(_dev(inp["table"]), _dev(inp["W_gate"]), _dev(inp["W_up"]), _dev(inp["W_down"]),
                      n_act) as af:
        X = torch.full((rows, d), float("nan"), device="cuda", dtype=torch.bfloat16)
        af.fuse(_dev(inp["E"]), _dev(inp["actions"], torch.int32), out=X)
        torch.cuda.synchronize()
    got = X.float().cpu().numpy()
    assert np.isfinite(got).all()
    err = f_max = x_max = 0.0
    for r0 in range(0, rows, 65536):
        sl = slice(r0, min(r0 + 65536, rows))
        want = AO.action_fuse(inp["E"][sl], inp["actions"][sl], inp["table"], inp["W_gate"], inp["W_up"],
                              inp["W_down"])
        f_want = want - inp["E"][sl]
        err = max(err, float(np.abs(got[sl].astype(np.float64) - inp["E"][sl] - f_want).max()))
        f_max = max(f_max, float(np.abs(f_want).max()))
        x_max = max(x_max, float(np.abs(want).max()))
    bound = TOL["bf16"] * f_max + 2.0 ** -8 * x_max
    print(f"[action] {name} rows={rows} err={err:.3e} bound={bound:.3e}", flush=True)
    assert err <= bound, (err, bound)


F32_CASES = [
    # name, rows, d, d_a, d_ff, n_actions: K = d + d_a padded to 16 (72 -> 80, 136 -> 144), both widths,
    # d_ff multiples of 32, row counts around the 16-row product tiles and past one 32768-row pass
    ("f32_d128_da64_ff256", 3000, 128, 64, 256, 8),
    ("f32_d64_da8_ff96", 513, 64, 8, 96, 5),
    ("f32_d128_da8_ff32", 17, 128, 8, 32, 3),
    ("f32_d64_da0_ff64", 1, 64, 0, 64, 1),
    ("f32_d128_da128_ff512", 40000, 128, 128, 512, 1000),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_action_f32_parity(case):
    """float32 rows, gathered z and float32 matrix-core products: the whole of x within 1e-4 normwise
    (max |X - x| <= 1e-4 max |x|) and its FFN part within 1e-4 of max |x - e| as well."""
    name, rows, d, d_a, d_ff, n_act = case
    inp = W.make_action_inputs(rows, d, d_a, d_ff, n_act, seed=rows + 1)
    acts = inp["actions"].copy()
    acts[::13] = n_act + 5  # clamped to the last type
    with ActionFusion(_dev(inp["table"], torch.float32) if d_a else None, _dev(inp["W_gate"], torch.float32),
                      _dev(inp["W_up"], torch.float32), _dev(inp["W_down"], torch.float32), n_act) as af:
        got = af.fuse(_dev(inp["E"], torch.float32), _dev(acts, torch.int32)).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
    want = AO.action_fuse(inp["E"], np.clip(acts, 0, n_act - 1), inp["table"], inp["W_gate"], inp["W_up"],
                          inp["W_down"])
    f_want = want - inp["E"]
    err_x = float(np.abs(got - want).max()) / float(np.abs(want).max())
    err_f = float(np.abs((got - inp["E"]) - f_want).max()) / float(np.abs(f_want).max())
    print(f"[action] {name} x err={err_x:.3e} ffn err={err_f:.3e}", flush=True)
    assert err_x <= TOL["f32"] and err_f <= TOL["f32"], (err_x, err_f)
