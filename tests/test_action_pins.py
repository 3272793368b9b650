"""Pins for the action-fusion oracle (SequenceO1 close reading, section 2.2):
x_i = e_i + SwiGLU-FFN([e_i ; a_i]).  Each pin checks an implementation so
that planted mistakes can be shown to be caught."""
import math

import numpy as np
import pytest

from oracle import action_oracle as AO


def _rand(seed, n=7, d=3, d_a=2, d_ff=4, n_act=3):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((n, d))
    acts = rng.integers(0, n_act, size=n)
    T = rng.standard_normal((n_act, d_a))
    Wg = rng.standard_normal((d + d_a, d_ff))
    Wu = rng.standard_normal((d + d_a, d_ff))
    Wd = rng.standard_normal((d_ff, d))
    return E, acts, T, Wg, Wu, Wd


def pin_zero_down_projection(impl):
    E, acts, T, Wg, Wu, Wd = _rand(1)
    return np.allclose(impl(E, acts, T, Wg, Wu, 0 * Wd), E, atol=0)


def pin_hand_value(impl):
    # d = d_a = d_ff = 1: z = [e, a], x = e + silu(g.z) (u.z) w
    e, a, g, u, w = 0.7, -1.3, (0.5, 2.0), (-1.0, 0.25), 1.5
    gz = g[0] * e + g[1] * a
    uz = u[0] * e + u[1] * a
    want = e + gz / (1 + math.exp(-gz)) * uz * w
    got = impl(np.array([[e]]), np.array([0]), np.array([[a]]), np.array([[g[0]], [g[1]]]),
               np.array([[u[0]], [u[1]]]), np.array([[w]]))
    return abs(float(got[0, 0]) - want) < 1e-12


def pin_equal_inputs_equal_rows(impl):
    E, acts, T, Wg, Wu, Wd = _rand(2)
    E[4] = E[1]
    acts[4] = acts[1]
    x = impl(E, acts, T, Wg, Wu, Wd)
    return np.array_equal(x[4], x[1])


def pin_rows_independent(impl):
    E, acts, T, Wg, Wu, Wd = _rand(3)
    perm = np.random.default_rng(9).permutation(E.shape[0])
    return np.allclose(impl(E[perm], acts[perm], T, Wg, Wu, Wd), impl(E, acts, T, Wg, Wu, Wd)[perm], atol=1e-12)


def pin_linear_in_down(impl):
    E, acts, T, Wg, Wu, Wd = _rand(4)
    x1 = impl(E, acts, T, Wg, Wu, Wd) - E
    x2 = impl(E, acts, T, Wg, Wu, 2.5 * Wd) - E
    return np.allclose(x2, 2.5 * x1, atol=1e-12) and np.abs(x1).max() > 1e-3


def pin_zero_inputs(impl):
    E, acts, T, Wg, Wu, Wd = _rand(5)
    return np.allclose(impl(0 * E, acts, 0 * T, Wg, Wu, Wd), 0, atol=0)


def pin_index_loops(impl):
    E, acts, T, Wg, Wu, Wd = _rand(6, n=4, d=2, d_a=3, d_ff=2, n_act=2)
    n, d = E.shape
    want = np.zeros((n, d))
    for i in range(n):
        z = list(E[i]) + list(T[acts[i]])
        h = []
        for f in range(Wg.shape[1]):
            gs = sum(z[t] * Wg[t, f] for t in range(len(z)))
            us = sum(z[t] * Wu[t, f] for t in range(len(z)))
            h.append(gs / (1.0 + math.exp(-gs)) * us)
        for c in range(d):
            want[i, c] = E[i, c] + sum(h[f] * Wd[f, c] for f in range(len(h)))
    return np.allclose(impl(E, acts, T, Wg, Wu, Wd), want, atol=1e-12)


PINS = [pin_zero_down_projection, pin_hand_value, pin_equal_inputs_equal_rows, pin_rows_independent,
        pin_linear_in_down, pin_zero_inputs, pin_index_loops]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_action_pin(pin):
    assert pin(AO.action_fuse)


def _mutant(kind):
    def impl(E, acts, T, Wg, Wu, Wd):
        E = np.asarray(E, dtype=np.float64)
        A = np.asarray(T, dtype=np.float64)[np.asarray(acts)]
        if kind == "no_action":
            A = 0 * A
        Z = np.concatenate([E, A], axis=1)
        g, u = Z @ Wg, Z @ Wu
        if kind == "gate_up_swapped":
            g, u = u, g
        act = 1 / (1 + np.exp(-g)) if kind == "sigmoid" else g / (1 + np.exp(-g))
        x = (act * u) @ Wd
        return x if kind == "no_residual" else E + x
    return impl


@pytest.mark.parametrize("kind", ["no_residual", "no_action", "gate_up_swapped", "sigmoid"])
def test_planted_mistake_is_caught(kind):
    assert all(pin(_mutant("none")) for pin in PINS)
    assert not all(pin(_mutant(kind)) for pin in PINS), kind
