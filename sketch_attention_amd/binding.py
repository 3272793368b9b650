"""Thin Python binding over libsa.so (include/sa.h), with the same names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their device pointers and the caller's HIP stream are passed
to the C ABI.  Every step of the computation runs in the library's HIP
kernels; there is no CPU fallback, and loading fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import numpy as np
import torch

from .build import LIB_PATH

SA_OK = 0
SA_ERR_INVALID_ARG = 1
SA_ERR_UNSUPPORTED = 2
SA_ERR_OUT_OF_MEMORY = 3
SA_ERR_DEVICE = 4

SA_F32 = 0
SA_BF16 = 1

SA_NORM_PROTOTYPES = 0  # Sketch Attention: softmax over the prototype axis
SA_NORM_HISTORY = 1     # the comparator: softmax over the history axis
_NORMS = {"prototypes": SA_NORM_PROTOTYPES, "history": SA_NORM_HISTORY}

_DTYPES = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}
_DTYPE_NAMES = {"f32": SA_F32, "bf16": SA_BF16}

EXPORTED = (
    "sa_create", "sa_create_ex", "sa_compress_batch", "sa_compress_batch_noalloc", "sa_reserve", "sa_destroy",
    "sa_status_string", "sa_check_config", "sa_check_batch",
    "sa_get_folded", "sa_set_kernel_timing", "sa_read_kernel_timing", "sa_describe_plan",
    "sa_stack_create", "sa_stack_compress_batch", "sa_stack_destroy", "sa_stack_set_kernel_timing",
    "sa_stack_read_kernel_timing",
    "sa_grad_check_config", "sa_grad_create", "sa_grad_compute", "sa_grad_destroy", "sa_grad_set_kernel_timing",
    "sa_grad_read_kernel_timing",
    "sa_action_check_config", "sa_action_create", "sa_action_fuse", "sa_action_compress_batch", "sa_action_destroy",
    "sa_action_set_kernel_timing", "sa_action_read_kernel_timing",
    "sa_measure_ceilings", "sa_measure_hbm_read",
)


class sa_layer_params(ctypes.Structure):
    """Mirror of the C struct sa_layer_params (device pointers)."""
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "W_Q", "W_K", "ln1_gain", "ln1_bias", "ffn_gate", "ffn_up", "ffn_down", "ln2_gain", "ln2_bias")]


class SAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {sa_status_string(status)} (status {status})")
        self.status = status


_lib = None

# Shape and dtype of every live handle, keyed by its address: the C ABI takes
# plain pointers and cannot check buffer sizes, so the binding checks every
# tensor against the handle it is used with before anything is enqueued.
_HANDLES: dict = {}


def _remember(handle: ctypes.c_void_p, kind: str, **info) -> None:
    _HANDLES[int(handle.value)] = dict(kind=kind, **info)


def _info(handle, kind: str) -> dict:
    key = handle.value if isinstance(handle, ctypes.c_void_p) else handle
    got = _HANDLES.get(int(key or 0))
    if got is None or got["kind"] != kind:
        raise ValueError(f"not a live {kind} handle")
    return got


def _forget(handle: ctypes.c_void_p) -> None:
    _HANDLES.pop(int(handle.value or 0), None)


def library() -> ctypes.CDLL:
    """Load libsa.so (once; SA_LIB_PATH selects another build).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SA_LIB_PATH") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing; run __graft_entry__.build() first "
                           "(this package has no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    p_i64 = ctypes.POINTER(ctypes.c_int64)
    p_i32 = ctypes.POINTER(ctypes.c_int32)
    p_f64 = ctypes.POINTER(ctypes.c_double)
    sig = {
        "sa_create": (i32, [ctypes.POINTER(vp), i32, i32, f32, i32, vp, vp, vp, vp]),
        "sa_create_ex": (i32, [ctypes.POINTER(vp), i32, i32, f32, i32, vp, vp, vp, i32, vp]),
        "sa_compress_batch": (i32, [vp, vp, vp, i32, vp, vp]),
        "sa_compress_batch_noalloc": (i32, [vp, vp, vp, i32, vp, vp]),
        "sa_reserve": (i32, [vp, i64, i32, i32, vp]),
        "sa_destroy": (None, [vp]),
        "sa_status_string": (ctypes.c_char_p, [i32]),
        "sa_check_config": (i32, [i32, i32, f32, i32]),
        "sa_check_batch": (i32, [i32, p_i64, i32]),
        "sa_get_folded": (i32, [vp, vp, vp]),
        "sa_set_kernel_timing": (i32, [vp, i32]),
        "sa_read_kernel_timing": (i32, [vp, p_f64, p_f64, p_i64]),
        "sa_describe_plan": (i32, [vp, i64, p_i32, p_i32, p_i32, p_i32, p_i32]),
        "sa_stack_create": (i32, [ctypes.POINTER(vp), i32, i32, i32, i32, f32, i32, vp,
                                  ctypes.POINTER(sa_layer_params), vp]),
        "sa_stack_compress_batch": (i32, [vp, vp, vp, i32, vp, vp]),
        "sa_stack_destroy": (None, [vp]),
        "sa_stack_set_kernel_timing": (i32, [vp, i32]),
        "sa_stack_read_kernel_timing": (i32, [vp, p_f64, p_f64, p_i64]),
        "sa_grad_check_config": (i32, [i32, i32, f32, i32]),
        "sa_grad_create": (i32, [ctypes.POINTER(vp), i32, i32, f32, i32, vp, vp, vp, vp]),
        "sa_grad_compute": (i32, [vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]),
        "sa_grad_destroy": (None, [vp]),
        "sa_grad_set_kernel_timing": (i32, [vp, i32]),
        "sa_grad_read_kernel_timing": (i32, [vp, p_f64, p_f64, p_i64]),
        "sa_action_check_config": (i32, [i32, i32, i32, i32, i32]),
        "sa_action_create": (i32, [ctypes.POINTER(vp), i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "sa_action_fuse": (i32, [vp, vp, vp, i64, vp, vp]),
        "sa_action_compress_batch": (i32, [vp, vp, vp, vp, vp, i32, vp, vp]),
        "sa_action_destroy": (None, [vp]),
        "sa_action_set_kernel_timing": (i32, [vp, i32]),
        "sa_action_read_kernel_timing": (i32, [vp, p_f64, p_i64]),
        "sa_measure_ceilings": (i32, [p_f64, p_f64, p_f64, p_f64, p_f64, vp]),
        "sa_measure_hbm_read": (i32, [p_f64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def sa_status_string(status: int) -> str:
    return library().sa_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != SA_OK:
        raise SAError(status, what)


def _stream_ptr(stream: Optional[torch.cuda.Stream], device: torch.device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _offsets_array(offsets) -> np.ndarray:
    if isinstance(offsets, torch.Tensor):
        if offsets.is_cuda:
            raise ValueError("offsets are read on the host: pass a CPU tensor, numpy array or list")
        offsets = offsets.numpy()
    return np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))


def _i64_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _device_tensor(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def sa_check_config(d: int, k: int, tau: float, dtype: Union[str, torch.dtype]) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else _DTYPE_NAMES.get(dtype, 99)
    return int(library().sa_check_config(int(d), int(k), float(tau), code))


def sa_check_batch(k: int, offsets) -> int:
    offs = _offsets_array(offsets)
    if offs.size == 0:
        return SA_ERR_INVALID_ARG
    return int(library().sa_check_batch(int(k), _i64_ptr(offs), int(offs.size - 1)))


def sa_create(P: torch.Tensor, W_Q: torch.Tensor, W_K: torch.Tensor, tau: float,
              stream: Optional[torch.cuda.Stream] = None, norm: str = "prototypes") -> ctypes.c_void_p:
    """Fold the weights into a new handle (see include/sa.h); norm "history"
    selects the comparator (sa_create_ex with SA_NORM_HISTORY)."""
    if norm not in _NORMS:
        raise ValueError("norm must be 'prototypes' or 'history'")
    for t, n in ((P, "P"), (W_Q, "W_Q"), (W_K, "W_K")):
        _device_tensor(t, n)
    if P.dtype not in _DTYPES or W_Q.dtype != P.dtype or W_K.dtype != P.dtype:
        raise ValueError("P, W_Q, W_K must share dtype float32 or bfloat16")
    if P.dim() != 2:
        raise ValueError("P must be [k, d]")
    k, d = P.shape
    if tuple(W_Q.shape) != (d, d) or tuple(W_K.shape) != (d, d):
        raise ValueError("W_Q and W_K must be [d, d]")
    h = ctypes.c_void_p()
    with torch.cuda.device(P.device):
        if norm == "prototypes":
            st = library().sa_create(ctypes.byref(h), int(d), int(k), float(tau), _DTYPES[P.dtype],
                                     ctypes.c_void_p(P.data_ptr()), ctypes.c_void_p(W_Q.data_ptr()),
                                     ctypes.c_void_p(W_K.data_ptr()), _stream_ptr(stream, P.device))
        else:
            st = library().sa_create_ex(ctypes.byref(h), int(d), int(k), float(tau), _DTYPES[P.dtype],
                                        ctypes.c_void_p(P.data_ptr()), ctypes.c_void_p(W_Q.data_ptr()),
                                        ctypes.c_void_p(W_K.data_ptr()), _NORMS[norm], _stream_ptr(stream, P.device))
    _check(st, "sa_create")
    _remember(h, "sa", k=int(k), d=int(d), dtype=P.dtype, device=P.device)
    return h


def sa_compress_batch(handle: ctypes.c_void_p, X: torch.Tensor, offsets, out: torch.Tensor,
                      stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue the compression of a packed batch into `out` ([U, k, d] float32).

    The library selects the handle's device itself, so no device context is
    entered here; pointers go to ctypes as plain integers."""
    if isinstance(offsets, np.ndarray) and offsets.dtype == np.int64 and offsets.ndim == 1 and \
            offsets.flags["C_CONTIGUOUS"]:
        offs = offsets
    else:
        offs = _offsets_array(offsets)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    info = _info(handle, "sa")
    _check_batch_tensors(info, X, offs, out)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    st = library().sa_compress_batch(handle, X.data_ptr(), offs.ctypes.data, offs.size - 1, out.data_ptr(),
                                     stream.cuda_stream)
    _check(st, "sa_compress_batch")


def _bound_call(fn, name: str, args: tuple, keep: tuple):
    """A callable that re-issues fn(*args) and raises on a non-OK status; keep
    holds the objects whose memory the pointers in args refer to."""
    def run() -> None:
        st = fn(*args)
        if st != 0:
            _check(st, name)
    run.keep = keep
    return run


def sa_compress_batch_bound(handle: ctypes.c_void_p, X: torch.Tensor, offsets, out: torch.Tensor,
                            stream: Optional[torch.cuda.Stream] = None):
    """Check the arguments of sa_compress_batch once and return a callable that
    enqueues that same call again (same buffers, offsets and stream) with no
    further Python-side work: for loops that re-run one batch layout over
    buffers that stay alive (the callable keeps X, out and the offsets)."""
    offs = np.array(_offsets_array(offsets), dtype=np.int64, copy=True)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    _check_batch_tensors(_info(handle, "sa"), X, offs, out)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    args = (handle, X.data_ptr(), offs.ctypes.data, offs.size - 1, out.data_ptr(), stream.cuda_stream)
    return _bound_call(library().sa_compress_batch, "sa_compress_batch", args, (X, offs, out, stream))


def sa_compress_batch_noalloc(handle: ctypes.c_void_p, X: torch.Tensor, offsets, out: torch.Tensor,
                              stream: Optional[torch.cuda.Stream] = None) -> None:
    """As sa_compress_batch, through the entry point that allocates nothing
    (its workspace is the library's fixed per-GPU array; see include/sa.h)."""
    offs = _offsets_array(offsets)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    _check_batch_tensors(_info(handle, "sa"), X, offs, out)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    st = library().sa_compress_batch_noalloc(handle, X.data_ptr(), offs.ctypes.data, offs.size - 1, out.data_ptr(),
                                             stream.cuda_stream)
    _check(st, "sa_compress_batch_noalloc")


def sa_reserve(handle: ctypes.c_void_p, max_rows: int, max_users: int, freeze: bool = True,
               stream: Optional[torch.cuda.Stream] = None) -> None:
    """Size (and with freeze, fix) the handle's workspace for calls of up to max_rows rows and max_users users
    (see include/sa.h)."""
    info = _info(handle, "sa")
    if stream is None:
        stream = torch.cuda.current_stream(info["device"])
    _check(library().sa_reserve(handle, int(max_rows), int(max_users), 1 if freeze else 0, stream.cuda_stream),
           "sa_reserve")


def _check_batch_tensors(info: dict, X: torch.Tensor, offs: np.ndarray, out: torch.Tensor) -> None:
    """X [offsets[-1], d] in the handle's dtype, out float32 [U, k, d], both contiguous on the GPU
    (shapes are checked first, so a wrong size is reported as such)."""
    k, d = info["k"], info["d"]
    if X.dim() != 2 or X.shape[0] != int(offs[-1]) or X.shape[1] != d:
        raise ValueError(f"X must be [offsets[-1], {d}]")
    if X.dtype != info["dtype"]:
        raise ValueError(f"X dtype {X.dtype} differs from the handle's {info['dtype']}")
    if out.dtype != torch.float32 or tuple(out.shape) != (offs.size - 1, k, d):
        raise ValueError(f"out must be float32 [{offs.size - 1}, {k}, {d}]")
    _device_tensor(X, "X")
    _device_tensor(out, "out")


def sa_destroy(handle: Optional[ctypes.c_void_p]) -> None:
    if handle is not None and handle.value:
        _forget(handle)
        library().sa_destroy(handle)


def sa_get_folded(handle: ctypes.c_void_p, dst: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    info = _info(handle, "sa")
    if dst.dtype != torch.float32 or tuple(dst.shape) != (info["k"], info["d"]):
        raise ValueError(f"dst must be float32 [{info['k']}, {info['d']}]")
    _device_tensor(dst, "dst")
    with torch.cuda.device(dst.device):
        _check(library().sa_get_folded(handle, ctypes.c_void_p(dst.data_ptr()), _stream_ptr(stream, dst.device)),
               "sa_get_folded")


def sa_set_kernel_timing(handle: ctypes.c_void_p, enable: bool) -> None:
    _check(library().sa_set_kernel_timing(handle, 1 if enable else 0), "sa_set_kernel_timing")


def sa_read_kernel_timing(handle: ctypes.c_void_p):
    """Returns (fused_ms_total, reduce_ms_total, fused_launches) since the last read."""
    f, r, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(library().sa_read_kernel_timing(handle, ctypes.byref(f), ctypes.byref(r), ctypes.byref(n)),
           "sa_read_kernel_timing")
    return f.value, r.value, n.value


def sa_describe_plan(handle: ctypes.c_void_p, total_rows: int) -> dict:
    vals = [ctypes.c_int32() for _ in range(5)]
    _check(library().sa_describe_plan(handle, int(total_rows), *[ctypes.byref(v) for v in vals]), "sa_describe_plan")
    keys = ("groups", "waves_k", "waves_rows", "tile_rows", "k_padded")
    return {k: v.value for k, v in zip(keys, vals)}


class SketchAttention:
    """Owns one handle: the folded weights of one (P, W_Q, W_K, tau)."""

    def __init__(self, P: torch.Tensor, W_Q: torch.Tensor, W_K: torch.Tensor, tau: float,
                 stream: Optional[torch.cuda.Stream] = None, norm: str = "prototypes"):
        self.handle = sa_create(P, W_Q, W_K, tau, stream, norm)
        self.norm = norm
        self.k, self.d = int(P.shape[0]), int(P.shape[1])
        self.dtype = P.dtype
        self.device = P.device
        self.tau = float(tau)

    def compress(self, X: torch.Tensor, offsets, out: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        if X.dtype != self.dtype:
            raise ValueError(f"X dtype {X.dtype} differs from the weights' {self.dtype}")
        if X.dim() != 2 or X.shape[1] != self.d:
            raise ValueError(f"X must be [N, {self.d}]")
        offs = _offsets_array(offsets)
        if out is None:
            out = torch.empty((offs.size - 1, self.k, self.d), dtype=torch.float32, device=X.device)
        sa_compress_batch(self.handle, X, offs, out, stream)
        return out

    def reserve(self, max_rows: int, max_users: int, freeze: bool = True,
                stream: Optional[torch.cuda.Stream] = None) -> None:
        """Workspace for calls of up to max_rows rows and max_users users; with freeze it never moves again
        (for HIP graph capture of compress)."""
        sa_reserve(self.handle, max_rows, max_users, freeze, stream)

    def folded(self) -> torch.Tensor:
        dst = torch.empty((self.k, self.d), dtype=torch.float32, device=self.device)
        sa_get_folded(self.handle, dst)
        return dst

    def plan(self, total_rows: int) -> dict:
        return sa_describe_plan(self.handle, total_rows)

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            sa_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- stacked refinement

LAYER_FIELDS = ("W_Q", "W_K", "ln1_gain", "ln1_bias", "ffn_gate", "ffn_up", "ffn_down", "ln2_gain", "ln2_bias")


def sa_stack_create(P: torch.Tensor, layers: Sequence[dict], tau: float,
                    stream: Optional[torch.cuda.Stream] = None) -> ctypes.c_void_p:
    """Copy the weights of a refinement stack into a new handle (see include/sa.h).

    `layers` holds one dict per layer with the sa_layer_params fields as GPU
    tensors: W_Q, W_K [d, d] in P's dtype; ln gains/biases [d], ffn_gate and
    ffn_up [d, d_ff], ffn_down [d_ff, d] in float32."""
    _device_tensor(P, "P")
    if P.dtype not in _DTYPES or P.dim() != 2:
        raise ValueError("P must be a [k, d] float32 or bfloat16 tensor")
    k, d = P.shape
    if len(layers) < 1:
        raise ValueError("at least one layer")
    d_ff = int(layers[0]["ffn_gate"].shape[1])
    arr = (sa_layer_params * len(layers))()
    for i, lay in enumerate(layers):
        for name in LAYER_FIELDS:
            t = lay[name]
            _device_tensor(t, f"layers[{i}].{name}")
            want_dtype = P.dtype if name in ("W_Q", "W_K") else torch.float32
            if t.dtype != want_dtype:
                raise ValueError(f"layers[{i}].{name} must be {want_dtype}")
            shape = {"W_Q": (d, d), "W_K": (d, d), "ffn_gate": (d, d_ff), "ffn_up": (d, d_ff),
                     "ffn_down": (d_ff, d)}.get(name, (d,))
            if tuple(t.shape) != shape:
                raise ValueError(f"layers[{i}].{name} must be {list(shape)}")
            setattr(arr[i], name, t.data_ptr())
    h = ctypes.c_void_p()
    with torch.cuda.device(P.device):
        st = library().sa_stack_create(ctypes.byref(h), int(d), int(k), d_ff, len(layers), float(tau), _DTYPES[P.dtype],
                                       ctypes.c_void_p(P.data_ptr()), arr, _stream_ptr(stream, P.device))
    _check(st, "sa_stack_create")
    _remember(h, "stack", k=int(k), d=int(d), dtype=P.dtype)
    return h


def sa_stack_compress_batch(handle: ctypes.c_void_p, X: torch.Tensor, offsets, out: torch.Tensor,
                            stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue X~(L) of every user of a packed batch into `out` ([U, k, d] float32)."""
    offs = _offsets_array(offsets)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    _check_batch_tensors(_info(handle, "stack"), X, offs, out)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    st = library().sa_stack_compress_batch(handle, X.data_ptr(), offs.ctypes.data, offs.size - 1, out.data_ptr(),
                                           stream.cuda_stream)
    _check(st, "sa_stack_compress_batch")


def sa_stack_compress_batch_bound(handle: ctypes.c_void_p, X: torch.Tensor, offsets, out: torch.Tensor,
                                  stream: Optional[torch.cuda.Stream] = None):
    """As sa_compress_batch_bound, for sa_stack_compress_batch."""
    offs = np.array(_offsets_array(offsets), dtype=np.int64, copy=True)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    _check_batch_tensors(_info(handle, "stack"), X, offs, out)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    args = (handle, X.data_ptr(), offs.ctypes.data, offs.size - 1, out.data_ptr(), stream.cuda_stream)
    return _bound_call(library().sa_stack_compress_batch, "sa_stack_compress_batch", args, (X, offs, out, stream))


def sa_stack_destroy(handle: Optional[ctypes.c_void_p]) -> None:
    if handle is not None and handle.value:
        _forget(handle)
        library().sa_stack_destroy(handle)


def sa_stack_set_kernel_timing(handle: ctypes.c_void_p, enable: bool) -> None:
    _check(library().sa_stack_set_kernel_timing(handle, 1 if enable else 0), "sa_stack_set_kernel_timing")


def sa_stack_read_kernel_timing(handle: ctypes.c_void_p):
    """Returns (fused_ms_total, reduce_ms_total, fused_launches) since the last read."""
    f, r, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(library().sa_stack_read_kernel_timing(handle, ctypes.byref(f), ctypes.byref(r), ctypes.byref(n)),
           "sa_stack_read_kernel_timing")
    return f.value, r.value, n.value


class SketchStack:
    """Owns one refinement-stack handle (section 2.2 of the SequenceO1 close reading)."""

    def __init__(self, P: torch.Tensor, layers: Sequence[dict], tau: float,
                 stream: Optional[torch.cuda.Stream] = None):
        self.handle = sa_stack_create(P, layers, tau, stream)
        self.k, self.d = int(P.shape[0]), int(P.shape[1])
        self.dtype = P.dtype

    def compress(self, X: torch.Tensor, offsets, out: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        if X.dtype != self.dtype or X.dim() != 2 or X.shape[1] != self.d:
            raise ValueError(f"X must be [N, {self.d}] {self.dtype}")
        offs = _offsets_array(offsets)
        if out is None:
            out = torch.empty((offs.size - 1, self.k, self.d), dtype=torch.float32, device=X.device)
        sa_stack_compress_batch(self.handle, X, offs, out, stream)
        return out

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            sa_stack_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------ backward pass
def sa_grad_check_config(d: int, k: int, tau: float, dtype: Union[str, torch.dtype]) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else _DTYPE_NAMES.get(dtype, 99)
    return int(library().sa_grad_check_config(int(d), int(k), float(tau), code))


def sa_grad_create(P: torch.Tensor, W_Q: torch.Tensor, W_K: torch.Tensor, tau: float,
                   stream: Optional[torch.cuda.Stream] = None) -> ctypes.c_void_p:
    """Prepare the weights of the backward pass (bfloat16 or float32; see include/sa.h)."""
    for t, n in ((P, "P"), (W_Q, "W_Q"), (W_K, "W_K")):
        _device_tensor(t, n)
    if P.dtype not in _DTYPES or W_Q.dtype != P.dtype or W_K.dtype != P.dtype or P.dim() != 2:
        raise ValueError("P [k, d], W_Q and W_K [d, d] must share one dtype")
    k, d = P.shape
    if tuple(W_Q.shape) != (d, d) or tuple(W_K.shape) != (d, d):
        raise ValueError("W_Q and W_K must be [d, d]")
    h = ctypes.c_void_p()
    with torch.cuda.device(P.device):
        st = library().sa_grad_create(ctypes.byref(h), int(d), int(k), float(tau), _DTYPES[P.dtype],
                                      ctypes.c_void_p(P.data_ptr()), ctypes.c_void_p(W_Q.data_ptr()),
                                      ctypes.c_void_p(W_K.data_ptr()), _stream_ptr(stream, P.device))
    _check(st, "sa_grad_create")
    _remember(h, "grad", k=int(k), d=int(d), dtype=P.dtype)
    return h


def sa_grad_compute(handle: ctypes.c_void_p, X: torch.Tensor, offsets, grad_sketch: torch.Tensor,
                    grad_X: torch.Tensor, grad_P: torch.Tensor, grad_W_Q: torch.Tensor, grad_W_K: torch.Tensor,
                    stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue the gradients of one packed batch (argument meaning as in include/sa.h)."""
    offs = _offsets_array(offsets)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    info = _info(handle, "grad")
    k, d, U = info["k"], info["d"], offs.size - 1
    if X.dim() != 2 or X.shape[0] != int(offs[-1]) or X.shape[1] != d or X.dtype != info["dtype"]:
        raise ValueError(f"X must be [offsets[-1], {d}] {info['dtype']}")
    if tuple(grad_X.shape) != tuple(X.shape) or grad_X.dtype != X.dtype:
        raise ValueError("grad_X must match X")
    if grad_sketch.dtype != torch.float32 or tuple(grad_sketch.shape) != (U, k, d):
        raise ValueError(f"grad_sketch must be float32 [{U}, {k}, {d}]")
    for t, n, shape in ((grad_P, "grad_P", (k, d)), (grad_W_Q, "grad_W_Q", (d, d)), (grad_W_K, "grad_W_K", (d, d))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape:
            raise ValueError(f"{n} must be float32 {list(shape)}")
    for t, n in ((X, "X"), (grad_sketch, "grad_sketch"), (grad_X, "grad_X"), (grad_P, "grad_P"),
                 (grad_W_Q, "grad_W_Q"), (grad_W_K, "grad_W_K")):
        _device_tensor(t, n)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    st = library().sa_grad_compute(handle, X.data_ptr(), offs.ctypes.data, offs.size - 1, grad_sketch.data_ptr(),
                                   grad_X.data_ptr(), grad_P.data_ptr(), grad_W_Q.data_ptr(), grad_W_K.data_ptr(),
                                   stream.cuda_stream)
    _check(st, "sa_grad_compute")


def sa_grad_destroy(handle: Optional[ctypes.c_void_p]) -> None:
    if handle is not None and handle.value:
        _forget(handle)
        library().sa_grad_destroy(handle)


def sa_grad_set_kernel_timing(handle: ctypes.c_void_p, enable: bool) -> None:
    _check(library().sa_grad_set_kernel_timing(handle, 1 if enable else 0), "sa_grad_set_kernel_timing")


def sa_grad_read_kernel_timing(handle: ctypes.c_void_p):
    """Returns (stats_ms_total, dx_ms_total, calls) since the last read."""
    a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(library().sa_grad_read_kernel_timing(handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)),
           "sa_grad_read_kernel_timing")
    return a.value, b.value, n.value


class SketchAttentionGrad:
    """Owns one backward handle: gradients of the sketches of one (P, W_Q, W_K, tau)."""

    def __init__(self, P: torch.Tensor, W_Q: torch.Tensor, W_K: torch.Tensor, tau: float,
                 stream: Optional[torch.cuda.Stream] = None):
        self.handle = sa_grad_create(P, W_Q, W_K, tau, stream)
        self.k, self.d = int(P.shape[0]), int(P.shape[1])
        self.dtype = P.dtype
        self.device = P.device

    def backward(self, X: torch.Tensor, offsets, grad_sketch: torch.Tensor,
                 stream: Optional[torch.cuda.Stream] = None):
        """Returns (grad_X, grad_P, grad_W_Q, grad_W_K) as new tensors."""
        if X.dtype != self.dtype or X.dim() != 2 or X.shape[1] != self.d:
            raise ValueError(f"X must be [N, {self.d}] {self.dtype}")
        dev = X.device
        gX = torch.empty_like(X)
        gP = torch.empty((self.k, self.d), dtype=torch.float32, device=dev)
        gQ = torch.empty((self.d, self.d), dtype=torch.float32, device=dev)
        gK = torch.empty((self.d, self.d), dtype=torch.float32, device=dev)
        sa_grad_compute(self.handle, X, offsets, grad_sketch, gX, gP, gQ, gK, stream)
        return gX, gP, gQ, gK

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            sa_grad_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------ action fusion
def sa_action_check_config(d: int, d_a: int, d_ff: int, n_actions: int, dtype: Union[str, torch.dtype]) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else _DTYPE_NAMES.get(dtype, 99)
    return int(library().sa_action_check_config(int(d), int(d_a), int(d_ff), int(n_actions), code))


def sa_action_create(table: Optional[torch.Tensor], W_gate: torch.Tensor, W_up: torch.Tensor, W_down: torch.Tensor,
                     n_actions: int, stream: Optional[torch.cuda.Stream] = None) -> ctypes.c_void_p:
    """Pack the action-fusion weights (see include/sa.h); table may be None when d_a == 0."""
    for t, n in ((W_gate, "W_gate"), (W_up, "W_up"), (W_down, "W_down")):
        _device_tensor(t, n)
    if table is not None:
        _device_tensor(table, "action_table")
    d_ff, d = W_down.shape
    k_in = W_gate.shape[0]
    d_a = k_in - d
    if tuple(W_up.shape) != (k_in, d_ff) or W_gate.shape[1] != d_ff or d_a < 0:
        raise ValueError("W_gate, W_up must be [d + d_a, d_ff] and W_down [d_ff, d]")
    if d_a > 0 and (table is None or tuple(table.shape) != (n_actions, d_a)):
        raise ValueError("action_table must be [n_actions, d_a]")
    dt = W_down.dtype
    if dt not in _DTYPES or any(t.dtype != dt for t in (W_gate, W_up) + ((table,) if d_a > 0 else ())):
        raise ValueError("weights and table must share one dtype")
    h = ctypes.c_void_p()
    dev = W_down.device
    with torch.cuda.device(dev):
        st = library().sa_action_create(ctypes.byref(h), int(d), int(d_a), int(d_ff), int(n_actions), _DTYPES[dt],
                                        ctypes.c_void_p(table.data_ptr() if d_a > 0 else 0),
                                        ctypes.c_void_p(W_gate.data_ptr()), ctypes.c_void_p(W_up.data_ptr()),
                                        ctypes.c_void_p(W_down.data_ptr()), _stream_ptr(stream, dev))
    _check(st, "sa_action_create")
    _remember(h, "action", d=int(d), dtype=dt)
    return h


def sa_action_fuse(handle: ctypes.c_void_p, E: torch.Tensor, actions: torch.Tensor, X: torch.Tensor,
                   stream: Optional[torch.cuda.Stream] = None) -> None:
    info = _info(handle, "action")
    if E.dim() != 2 or E.shape[1] != info["d"] or E.dtype != info["dtype"]:
        raise ValueError(f"E must be [rows, {info['d']}] {info['dtype']}")
    if actions.dtype != torch.int32 or actions.dim() != 1 or actions.shape[0] != E.shape[0]:
        raise ValueError("actions must be int32 [rows]")
    if tuple(X.shape) != tuple(E.shape) or X.dtype != E.dtype:
        raise ValueError("X must match E")
    for t, n in ((E, "E"), (actions, "actions"), (X, "X")):
        _device_tensor(t, n)
    if stream is None:
        stream = torch.cuda.current_stream(E.device)
    _check(library().sa_action_fuse(handle, E.data_ptr(), actions.data_ptr(), int(E.shape[0]), X.data_ptr(),
                                    stream.cuda_stream), "sa_action_fuse")


def sa_action_compress_batch(action: ctypes.c_void_p, handle: ctypes.c_void_p, E: torch.Tensor,
                             actions: torch.Tensor, offsets, out: torch.Tensor,
                             stream: Optional[torch.cuda.Stream] = None) -> None:
    """out[u] = the sketch of user u's rows x_i = e_i + FFN([e_i; a_i]), formed inside the sketch kernel
    (X never written; see include/sa.h)."""
    ainfo = _info(action, "action")
    offs = _offsets_array(offsets)
    if offs.ndim != 1 or offs.size < 1:
        raise ValueError("offsets must be a 1-D array of length num_users + 1")
    if E.dim() != 2 or E.shape[1] != ainfo["d"] or E.dtype != ainfo["dtype"]:
        raise ValueError(f"E must be [rows, {ainfo['d']}] {ainfo['dtype']}")
    if actions.dtype != torch.int32 or actions.dim() != 1 or actions.shape[0] != E.shape[0]:
        raise ValueError("actions must be int32 [rows]")
    _check_batch_tensors(_info(handle, "sa"), E, offs, out)
    _device_tensor(actions, "actions")
    if stream is None:
        stream = torch.cuda.current_stream(E.device)
    _check(library().sa_action_compress_batch(action, handle, E.data_ptr(), actions.data_ptr(), offs.ctypes.data,
                                              offs.size - 1, out.data_ptr(), stream.cuda_stream),
           "sa_action_compress_batch")


def sa_action_destroy(handle: Optional[ctypes.c_void_p]) -> None:
    if handle is not None and handle.value:
        _forget(handle)
        library().sa_action_destroy(handle)


def sa_action_set_kernel_timing(handle: ctypes.c_void_p, enable: bool) -> None:
    _check(library().sa_action_set_kernel_timing(handle, 1 if enable else 0), "sa_action_set_kernel_timing")


def sa_action_read_kernel_timing(handle: ctypes.c_void_p):
    """Returns (ms_total, launches) since the last read."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(library().sa_action_read_kernel_timing(handle, ctypes.byref(ms), ctypes.byref(n)),
           "sa_action_read_kernel_timing")
    return ms.value, n.value


class ActionFusion:
    """Owns one action-fusion handle: x = e + SwiGLU-FFN([e; table[action]]) (section 2.2)."""

    def __init__(self, table: Optional[torch.Tensor], W_gate: torch.Tensor, W_up: torch.Tensor,
                 W_down: torch.Tensor, n_actions: int, stream: Optional[torch.cuda.Stream] = None):
        self.handle = sa_action_create(table, W_gate, W_up, W_down, n_actions, stream)
        self.d = int(W_down.shape[1])

    def fuse(self, E: torch.Tensor, actions: torch.Tensor, out: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        if out is None:
            out = torch.empty_like(E)
        sa_action_fuse(self.handle, E, actions, out, stream)
        return out

    def compress(self, sa: "SketchAttention", E: torch.Tensor, actions: torch.Tensor, offsets,
                 out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """The sketches ([U, k, d] float32) of the fused rows, without writing X."""
        offs = _offsets_array(offsets)
        if out is None:
            out = torch.empty((offs.size - 1, sa.k, sa.d), dtype=torch.float32, device=E.device)
        sa_action_compress_batch(self.handle, sa.handle, E, actions, offs, out, stream)
        return out

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            sa_action_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------ device ceilings
def sa_measure_ceilings(stream: Optional[torch.cuda.Stream] = None) -> dict:
    """Measured ceilings of the current GPU (see include/sa.h): bf16 matrix-core
    TFLOP/s (16x16x32 and 32x32x16 products), float32 FMA TFLOP/s, hardware exp2
    per second, streaming-copy GB/s."""
    vals = [ctypes.c_double() for _ in range(5)]
    dev = torch.device("cuda", torch.cuda.current_device())
    _check(library().sa_measure_ceilings(*[ctypes.byref(v) for v in vals], _stream_ptr(stream, dev)),
           "sa_measure_ceilings")
    keys = ("mfma_bf16_tflops", "mfma_bf16_32x32_tflops", "valu_fma_tflops", "exp2_per_sec", "copy_gbs")
    return {k: v.value for k, v in zip(keys, vals)}


def sa_measure_hbm_read(stream: Optional[torch.cuda.Stream] = None) -> float:
    """GB/s of a read-only stream over 1 GiB on the current GPU (see include/sa.h)."""
    v = ctypes.c_double()
    dev = torch.device("cuda", torch.cuda.current_device())
    _check(library().sa_measure_hbm_read(ctypes.byref(v), _stream_ptr(stream, dev)), "sa_measure_hbm_read")
    return v.value
