"""Input generators and the FLOP accounting (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import cost_model as CM
from sketch_attention_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0], np.float32)]).astype(np.float32)
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_named_shapes_and_recipes():
    wl = W.named_workload("tiny")
    assert (wl.X.shape, wl.k, wl.d, wl.dtype) == ((1024, 64), 16, 64, "f32")
    assert wl.tau == pytest.approx(1 / 8)
    wl = W.named_workload("recent", users=2)
    assert wl.X.shape == (20000, 128) and wl.k == 64 and wl.dtype == "bf16"
    assert np.array_equal(W.round_to_bf16(wl.X), wl.X)
    assert np.array_equal(W.round_to_bf16(wl.W_K), wl.W_K)
    assert abs(wl.W_Q.std() - 1 / math.sqrt(128)) < 0.01


def test_many_proto_prototypes_unit_norm():
    wl = W.named_workload("many_proto", users=1, lengths=[100])
    norms = np.sqrt((wl.P.astype(np.float64) ** 2).sum(axis=1))
    assert wl.k == 1024 and wl.d == 64
    assert np.allclose(norms, 1.0, atol=1e-2)      # unit before bf16 rounding


def test_ragged_lengths_and_duplicates():
    wl = W.named_workload("ragged", users=3)
    lens = np.diff(wl.offsets)
    assert len(lens) == 3 and lens.min() >= 1000 and lens.max() <= 100000
    for u in range(3):
        rows = wl.user_rows(u)
        n = rows.shape[0]
        uniq = np.unique(rows.view(np.uint32).reshape(n, -1), axis=0).shape[0]
        assert n - uniq == math.floor(0.2 * n)    # copies are exact and all distinct positions
    full = W.NAMED_WORKLOADS["ragged"]["lengths"]()
    assert len(full) == 64 and min(full) >= 1000 and max(full) <= 100000


def test_cluster_workload_is_clustered():
    wl = W.make_workload(lengths=[2000], d=16, k=4, x_kind="clusters", clusters=8, cluster_sigma=0.1, seed=3)
    X = wl.X.astype(np.float64)[:500]
    # rows sit within about sigma*sqrt(2d) of a same-cluster neighbour, far
    # closer than two independent N(0, I) rows (about sqrt(2d) apart)
    D2 = ((X[:, None, :] - X[None, :, :]) ** 2).sum(-1)
    np.fill_diagonal(D2, np.inf)
    nn = np.sqrt(D2.min(axis=1))
    assert np.median(nn) < 0.2 * math.sqrt(2 * 16)


def test_seeded_and_deterministic():
    a = W.named_workload("recent", users=1)
    b = W.named_workload("recent", users=1)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.P, b.P)


def test_empty_users_allowed():
    wl = W.make_workload(lengths=[0, 5, 0], d=64, k=3, seed=2)
    assert list(wl.offsets) == [0, 0, 5, 5] and wl.X.shape == (5, 64)


def test_cost_model_reproduces_figure1():
    with open(os.path.join(GOLDEN, "fig1_gflops.json")) as f:
        g = json.load(f)
    p = CM.CostParams(**g["params"])
    got = {}
    for pt in g["points"]:
        if pt["p_hit"] is None:
            v = CM.direct_stca_per_target(p, pt["reuse"]) / 1e9
        else:
            v = CM.sequenceo1_per_target(p, pt["reuse"], pt["p_hit"]) / 1e9
        digits = len(str(pt["gflop"]).split(".")[1])
        assert round(v, digits) == pytest.approx(pt["gflop"], abs=10 ** -digits / 2 + 1e-12), pt["what"]
        got[pt["what"]] = v
    r_train = got["direct STCA, training"] / got["SequenceO1, training"]
    r_serve = got["direct STCA, serving"] / got["SequenceO1, serving"]
    r_nomrlb = CM.direct_stca_per_target(p, 1) / CM.sequenceo1_per_target(p, 1, 0.5)
    assert [round(r, 2) for r in (r_train, r_serve, r_nomrlb)] == [x["value"] for x in g["ratios"]]


def test_sa_contraction_share():
    """The two n-long contractions dominate the SA miss cost at the paper's shape."""
    p = CM.CostParams()
    share = CM.sa_contraction_flops(p.k, p.d, p.n) * p.n_sa / CM.sa_miss_flops(p)
    assert 0.93 < share < 0.94
