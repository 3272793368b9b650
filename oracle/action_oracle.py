"""Plain fp64 CPU oracle for the action fusion that produces the history rows.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the HIP library shares no code
with it.

SequenceO1 close-reading page, section 2.2: each behaviour's row is built
from the item embedding e_i of its video and the embedding a_i of its action
type; the two are concatenated, a SwiGLU-gated feed-forward network maps the
concatenation back to the item width, and the result is added to e_i:

    x_i = e_i + FFN([e_i ; a_i]),   FFN(z) = (silu(z W_gate) * (z W_up)) W_down

Only these rows x_i enter the history matrix that the sketch compresses.  The
page gives neither the action embedding width nor the FFN width; here the
action types index a table of n_act embeddings of width d_a, and the gated
layer has width d_ff (both parameters).  Computed literally in float64: the
concatenation is formed, the three products taken as written.

Pins (tests under "not gpu"): W_down = 0 gives x = e; a hand value at
d = d_a = d_ff = 1; rows with equal (e, action) give equal x; rows are
independent (permuting them permutes x); the FFN is linear in W_down; zero
embedding and zero action row give x = 0; brute-force index loops on tiny
inputs; planted mistakes (no residual, action part dropped, gate and up
swapped, sigmoid for silu) are caught.
"""
from __future__ import annotations

import numpy as np

from .refine_oracle import silu

__all__ = ["action_fuse"]


def action_fuse(E, actions, A_table, W_gate, W_up, W_down) -> np.ndarray:
    """x_i = e_i + (silu(z_i W_gate) * (z_i W_up)) W_down with z_i = [e_i ; A_table[actions[i]]].

    E [n, d], actions [n] integer ids into A_table [n_act, d_a],
    W_gate and W_up [d + d_a, d_ff], W_down [d_ff, d]; float64 [n, d]."""
    E = np.asarray(E, dtype=np.float64)
    acts = np.asarray(actions, dtype=np.int64)
    A = np.asarray(A_table, dtype=np.float64)[acts]
    Z = np.concatenate([E, A], axis=1)
    H = silu(Z @ np.asarray(W_gate, dtype=np.float64)) * (Z @ np.asarray(W_up, dtype=np.float64))
    return E + H @ np.asarray(W_down, dtype=np.float64)
