"""Shared helpers of the tests: error metrics and running the GPU path."""
import numpy as np
import torch

# Tolerances (normwise, per user): bf16 inputs with float32 accumulation and
# the float32 path.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def normwise_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| / max |want| over one user's k x d sketch."""
    den = float(np.max(np.abs(want)))
    num = float(np.max(np.abs(got.astype(np.float64) - want)))
    if den == 0.0:
        return num
    return num / den


def centred(a: np.ndarray) -> np.ndarray:
    """Sketch minus its mean row, so a near-uniform answer cannot pass on the common mean."""
    a = a.astype(np.float64)
    return a - a.mean(axis=0, keepdims=True)


# Unit roundoff of the weights as the aggregation product consumes them:
# each weight a_ji is rounded once to bfloat16 (relative error <= 2^-9) or
# used in float32.  Rounding every weight of row j perturbs the sketch row by
# at most u * sum_i a_ji |x_i|, i.e. by u times the sketch of |X| under the
# same weights; the row-centred comparison is allowed that much on top of its
# relative tolerance, because when all sketch rows are nearly equal (say k = 2
# with weights near 1/2) the centred sketch is tiny and the weight rounding
# alone exceeds any relative bound on it.
WEIGHT_ROUNDING = {"bf16": 2.0 ** -8, "f32": 2.0 ** -20}


def worst_errors(got: np.ndarray, want: np.ndarray):
    """(max over users of the normwise error, same on the centred sketches)."""
    e = max(normwise_err(g, w) for g, w in zip(got, want))
    c = max(normwise_err(centred(g), centred(w)) for g, w in zip(got, want))
    return e, c


def centred_within(got: np.ndarray, want: np.ndarray, abs_weighted: np.ndarray, tol: float, dtype: str) -> bool:
    """Centred check with the weight-rounding allowance described above."""
    gc, wc = centred(got), centred(want)
    err = float(np.max(np.abs(gc - wc)))
    return err <= tol * float(np.max(np.abs(wc))) + WEIGHT_ROUNDING[dtype] * float(np.max(abs_weighted))


def torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_device(wl, device="cuda"):
    dt = torch_dtype(wl.dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
    return t(wl.X), t(wl.P), t(wl.W_Q), t(wl.W_K)


def run_gpu(wl, device="cuda", X=None):
    """Compress a workload through the C ABI; returns float32 numpy [U, k, d]."""
    from sketch_attention_amd import SketchAttention
    Xd, P, WQ, WK = to_device(wl, device)
    if X is not None:
        Xd = X
    with SketchAttention(P, WQ, WK, wl.tau) as sa:
        out = sa.compress(Xd, wl.offsets)
        torch.cuda.synchronize()
    return out.cpu().numpy()
