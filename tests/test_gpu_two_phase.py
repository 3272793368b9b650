"""Parity of the two-phase pass (d = 128 with more than 512 prototypes, the
final configuration of the SequenceO1 page: about a thousand prototypes at
width 128, section 3.2) through the C ABI with the fp64 CPU oracle, with the
metric of the one-pass tests: normwise error per user (and on the row-centred
sketch) within 2e-2 for bfloat16 inputs.  The first phase writes each row's
log-sum-exp over every block of 256 prototypes, a merge forms the row's
log-sum-exp over all of them, and the second phase aggregates 2^(s' - L) per
block; the cases cover padded and full prototype counts, ragged and empty
users, a full 100 000-row user, rows whose scores leave the unshifted range
(the first phase's exact fallback), the mass identity at full size and
bitwise reproducibility."""
import numpy as np
import pytest
import torch

from oracle import sa_oracle as O
from sketch_attention_amd import SketchAttention
from sketch_attention_amd import workloads as W
from sa_testlib import run_gpu, to_device
from test_gpu_parity import _assert_mass_identity, _assert_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k,lengths", [
    (513, [1, 63, 64, 65, 2000]),          # one real prototype in the last block
    (600, [700, 0, 129, 3]),
    (768, [64, 1500]),                      # three full blocks
    (1000, [1, 999, 0, 4097]),
    (1024, [300, 5000, 17]),                # four full blocks, no padding
])
def test_two_phase_sweep(k, lengths):
    wl = W.make_workload(lengths=lengths, d=128, k=k, dtype="bf16", seed=11 * k, name=f"two-phase-{k}")
    got = run_gpu(wl)
    for u, n in enumerate(lengths):
        if n == 0:
            assert not got[u].any()
    _assert_parity(wl, got)


def test_two_phase_full_user_100k():
    wl = W.make_workload(lengths=[100000], d=128, k=1000, dtype="bf16", seed=1000, name="two-phase-100k",
                         x_kind="clusters", clusters=64, cluster_sigma=0.3)
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_two_phase_final_workload_sampled():
    wl = W.named_workload("final")
    got = run_gpu(wl)
    _assert_parity(wl, got, users=[0, 3])
    _assert_mass_identity(wl, got)


def test_two_phase_spike_rows_take_the_exact_fallback():
    """Rows scaled by 100 have scores of several hundred (log2 units): their
    unshifted per-block sums leave [2^-100, 2^100], so the first phase redoes
    those row blocks with a running maximum; the rows are picked with a gap of
    at least 1.7 log2 units between their two best prototypes before scaling
    (per the oracle's scores), so the bf16 rounding of the folded matrix
    cannot change which prototype takes their mass."""
    wl = W.make_workload(lengths=[3000, 700], d=128, k=1000, dtype="bf16", seed=21, name="two-phase-spikes")
    s = np.sort(O.affinity(wl.X, wl.P, wl.W_Q, wl.W_K, wl.tau), axis=0) / np.log(2.0)
    gap = s[-1] - s[-2]
    rows = []
    for u in range(wl.num_users):
        a, b = int(wl.offsets[u]), int(wl.offsets[u + 1])
        rows += [int(r) for r in np.nonzero(gap[a:b] >= 1.7)[0][:5] + a]
    assert len(rows) >= 6, rows
    for r in rows:
        wl.X[r] = W.round_to_bf16(wl.X[r] * 100.0)
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


def test_two_phase_is_bitwise_deterministic():
    wl = W.make_workload(lengths=[4000, 1, 2500], d=128, k=900, dtype="bf16", seed=44, name="two-phase-det")
    X, P, WQ, WK = to_device(wl)
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        a = sa.compress(X, wl.offsets).clone()
        b = sa.compress(X, wl.offsets)
        torch.cuda.synchronize()
    assert torch.equal(a, b)


# plan overrides of the two 32x32x16 passes: prototypes along the registers
# with the weights through LDS (sa_stream32.hpp), and along the lanes with the
# weights in registers (sa_wide.hpp)
WIDE_PLANS = {"stream32": "32,8,1,0,2,1,4,2", "lanes": "32,8,1,0,3,1,4,2"}


@pytest.mark.parametrize("plan", sorted(WIDE_PLANS))
@pytest.mark.parametrize("k,lengths", [(256, [1, 63, 64, 65, 3000, 0]), (200, [700, 129, 5]), (129, [2, 5000])])
def test_wide_products_one_pass(k, lengths, plan, monkeypatch):
    """The 32x32x16 passes as one-pass kernels for d = 128, k <= 256,
    selected by the plan override: parity with the oracle, padded and full
    prototype counts, ragged users."""
    monkeypatch.setenv("SA_PLAN", WIDE_PLANS[plan])
    wl = W.make_workload(lengths=lengths, d=128, k=k, dtype="bf16", seed=5 * k, name=f"wide-one-pass-{k}")
    got = run_gpu(wl)
    _assert_parity(wl, got)
    _assert_mass_identity(wl, got)


@pytest.mark.parametrize("plan", sorted(WIDE_PLANS))
def test_wide_products_exact_path(plan, monkeypatch):
    """Every tile of the 32x32x16 one-pass kernels overflows the unshifted
    softmax (hard assignment at tau = 4) and takes the exact pass; then only a
    few rows do, so exact and fast tiles alternate."""
    from test_gpu_parity import _hard_bf16_workload
    monkeypatch.setenv("SA_PLAN", WIDE_PLANS[plan])
    wl = _hard_bf16_workload([3000, 77, 1], d=128, k=256, tau=4.0, seed=23)
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)
    rng = np.random.default_rng(24)
    spikes = np.sort(rng.choice(5000, size=7, replace=False))
    wl = _hard_bf16_workload([5000], d=128, k=200, tau=4.0, seed=25, spike_rows=spikes)
    wl.X = W.round_to_bf16(wl.X * np.float32(0.05))
    wl.X[spikes] = W.round_to_bf16(wl.X[spikes] * np.float32(20.0))
    got = run_gpu(wl)
    assert np.isfinite(got).all()
    _assert_parity(wl, got)


@pytest.mark.parametrize("plan", sorted(WIDE_PLANS))
def test_wide_products_per_user_matrices(plan, monkeypatch):
    """Two refinement layers on the 32x32x16 one-pass kernels: the second
    layer's folded matrix is per user (reloaded when a group's tile list
    crosses a user boundary)."""
    from test_gpu_stack import _check
    monkeypatch.setenv("SA_PLAN", WIDE_PLANS[plan])
    wl = W.make_workload(lengths=[1500, 10, 0, 4097, 64], d=128, k=256, dtype="bf16", seed=26, name="wide-stack")
    layers = W.make_stack_layers(d=128, d_ff=256, layers=2, dtype="bf16", seed=27)
    _check(wl, layers)
