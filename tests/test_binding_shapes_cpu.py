"""The binding checks every tensor against the handle it is used with before
anything reaches the C ABI (which takes plain pointers and cannot check
sizes).  The handles here are registry entries only: no library call is made,
every case must raise ValueError first."""
import ctypes

import numpy as np
import pytest
import torch

from sketch_attention_amd import binding as B

K, D = 16, 64


@pytest.fixture
def handles():
    made = {}
    for addr, kind in ((0x1000, "sa"), (0x2000, "stack"), (0x3000, "grad")):
        h = ctypes.c_void_p(addr)
        B._remember(h, kind, k=K, d=D, dtype=torch.bfloat16)
        made[kind] = h
    h = ctypes.c_void_p(0x4000)
    B._remember(h, "action", d=D, dtype=torch.bfloat16)
    made["action"] = h
    yield made
    for h in made.values():
        B._forget(h)


def _x(n, d=D, dt=torch.bfloat16):
    return torch.zeros((n, d), dtype=dt)


OFFS = np.array([0, 3, 10], dtype=np.int64)


@pytest.mark.parametrize("fn", ["sa", "stack"])
@pytest.mark.parametrize("X,out,what", [
    (_x(10, 32), torch.zeros((2, K, D)), "X must be"),                     # narrow rows
    (_x(9), torch.zeros((2, K, D)), "X must be"),                          # fewer rows than offsets[-1]
    (_x(10, dt=torch.float32), torch.zeros((2, K, D)), "dtype"),           # dtype of another handle
    (_x(10), torch.zeros((2, K - 1, D)), "out must be"),                   # undersized sketch buffer
    (_x(10), torch.zeros((1, K, D)), "out must be"),                       # too few users
    (_x(10), torch.zeros((2, K, D), dtype=torch.bfloat16), "out must be"),  # wrong output dtype
])
def test_compress_rejects_mismatched_tensors(handles, fn, X, out, what):
    call = B.sa_compress_batch if fn == "sa" else B.sa_stack_compress_batch
    with pytest.raises(ValueError, match=what):
        call(handles[fn], X, OFFS, out)
    # the bound form (arguments checked once, then re-issued) checks the same things up front
    bind = B.sa_compress_batch_bound if fn == "sa" else B.sa_stack_compress_batch_bound
    with pytest.raises(ValueError, match=what):
        bind(handles[fn], X, OFFS, out)


def test_compress_shapes_ok_reach_device_check(handles):
    # right shapes on the CPU: the next check (GPU tensors) is what fails
    with pytest.raises(ValueError, match="GPU tensor"):
        B.sa_compress_batch(handles["sa"], _x(10), OFFS, torch.zeros((2, K, D)))


def test_handle_kind_is_checked(handles):
    with pytest.raises(ValueError, match="not a live sa handle"):
        B.sa_compress_batch(handles["grad"], _x(10), OFFS, torch.zeros((2, K, D)))
    with pytest.raises(ValueError, match="not a live"):
        B.sa_compress_batch(ctypes.c_void_p(0x9999), _x(10), OFFS, torch.zeros((2, K, D)))


def _grad_args(**over):
    a = dict(X=_x(10), grad_sketch=torch.zeros((2, K, D)), grad_X=_x(10), grad_P=torch.zeros((K, D)),
             grad_W_Q=torch.zeros((D, D)), grad_W_K=torch.zeros((D, D)))
    a.update(over)
    return a


@pytest.mark.parametrize("over,what", [
    (dict(X=_x(10, 32)), "X must be"),
    (dict(grad_X=_x(9)), "grad_X must match"),
    (dict(grad_sketch=torch.zeros((2, K, D - 1))), "grad_sketch must be"),
    (dict(grad_sketch=torch.zeros((3, K, D))), "grad_sketch must be"),
    (dict(grad_P=torch.zeros((K - 1, D))), "grad_P must be"),
    (dict(grad_W_Q=torch.zeros((D, D - 1))), "grad_W_Q must be"),
    (dict(grad_W_K=torch.zeros((D, D), dtype=torch.bfloat16)), "grad_W_K must be"),
])
def test_grad_rejects_mismatched_tensors(handles, over, what):
    a = _grad_args(**over)
    with pytest.raises(ValueError, match=what):
        B.sa_grad_compute(handles["grad"], a["X"], OFFS, a["grad_sketch"], a["grad_X"], a["grad_P"], a["grad_W_Q"],
                          a["grad_W_K"])


@pytest.mark.parametrize("E,acts,X,what", [
    (_x(5, 32), torch.zeros(5, dtype=torch.int32), _x(5, 32), "E must be"),
    (_x(5), torch.zeros(4, dtype=torch.int32), _x(5), "actions must be"),
    (_x(5), torch.zeros(5, dtype=torch.int64), _x(5), "actions must be"),
    (_x(5), torch.zeros(5, dtype=torch.int32), _x(4), "X must match"),
])
def test_action_rejects_mismatched_tensors(handles, E, acts, X, what):
    with pytest.raises(ValueError, match=what):
        B.sa_action_fuse(handles["action"], E, acts, X)


def test_folded_buffer_shape(handles):
    with pytest.raises(ValueError, match="dst must be"):
        B.sa_get_folded(handles["sa"], torch.zeros((K, D - 1)))


@pytest.mark.parametrize("E,acts,out,what", [
    (_x(10, 32), torch.zeros(10, dtype=torch.int32), torch.zeros((2, K, D)), "E must be"),         # narrow rows
    (_x(10, dt=torch.float32), torch.zeros(10, dtype=torch.int32), torch.zeros((2, K, D)), "E must be"),
    (_x(10), torch.zeros(10, dtype=torch.int64), torch.zeros((2, K, D)), "actions must be"),       # id dtype
    (_x(10), torch.zeros(9, dtype=torch.int32), torch.zeros((2, K, D)), "actions must be"),        # id count
    (_x(9), torch.zeros(9, dtype=torch.int32), torch.zeros((2, K, D)), "X must be"),               # rows vs offsets
    (_x(10), torch.zeros(10, dtype=torch.int32), torch.zeros((2, K - 1, D)), "out must be"),       # sketch buffer
])
def test_action_compress_rejects_mismatched_tensors(handles, E, acts, out, what):
    with pytest.raises(ValueError, match=what):
        B.sa_action_compress_batch(handles["action"], handles["sa"], E, acts, OFFS, out)
