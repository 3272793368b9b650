"""Matrix-product FLOP count of the SequenceO1 long-history branch.

TEST INFRASTRUCTURE ONLY (imported by the tests; never by the product path).

Source: SequenceO1 close-reading page, section 2.4 (cost formulas) and
section 3.5 / Figure 1 (top panels), which prints the resulting per-target
GFLOP counts at n = 100K.  The formulas below are this model's reading of
section 2.4, chosen because they reproduce every printed Figure 1 number to
all printed digits:

  SA miss cost per user   C_SA     = N_sa (2 n d^2 + 2 k d^2 + 4 k n d + 12 k d^2)
  per-target interaction  C_target = N_stca (4 h k D + 20 D^2)
  shared + adapter        C_shared + C_adapter = N_stca 12 k D^2 + 2 k d D
  SequenceO1 per target   C_target + (C_shared + C_adapter + (1 - p_hit) C_SA) / R
  direct STCA per target  N_stca (4 h n D + 20 D^2) + N_stca 12 n D^2 / R

with N_sa = 2 SA layers, d = 128, k = 1024 prototypes ("about a thousand",
section 3.2), N_stca = 4 layers, h = 16 heads, D = 1024 (section 2.4).

The term 4 k n d is the two n-long contractions of one SA layer (affinity
and aggregation, 2 k n d each).  The page excludes softmax, normalisation and
activations from the count, so throughput in FLOP/s for the compression
kernel is quoted against 4 k d per history row.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class CostParams:
    n: int = 100_000
    d: int = 128
    k: int = 1024
    n_sa: int = 2
    n_stca: int = 4
    heads: int = 16
    D: int = 1024


def sa_contraction_flops(k: int, d: int, n: int) -> float:
    """Affinity (2 k n d) plus aggregation (2 k n d) of one SA layer."""
    return 4.0 * k * n * d


def sa_miss_flops(p: CostParams) -> float:
    n, d, k = p.n, p.d, p.k
    return p.n_sa * (2 * n * d * d + 2 * k * d * d + sa_contraction_flops(k, d, n) + 12 * k * d * d)


def target_flops(p: CostParams) -> float:
    return p.n_stca * (4 * p.heads * p.k * p.D + 20 * p.D * p.D)


def shared_adapter_flops(p: CostParams) -> float:
    return p.n_stca * 12 * p.k * p.D * p.D + 2 * p.k * p.d * p.D


def sequenceo1_per_target(p: CostParams, reuse: float, p_hit: float) -> float:
    return target_flops(p) + (shared_adapter_flops(p) + (1.0 - p_hit) * sa_miss_flops(p)) / reuse


def direct_stca_per_target(p: CostParams, reuse: float) -> float:
    return (p.n_stca * (4 * p.heads * p.n * p.D + 20 * p.D * p.D)
            + p.n_stca * 12 * p.n * p.D * p.D / reuse)
