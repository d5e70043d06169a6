"""Plain CPU oracle of a Gated DeltaNet layer's recurrence over the kept rows
(test infrastructure: only tests/, the smoke check and the benchmark's CPU leg
use it).

Why it is here ([KO] "성능 결과"; [PT] "Resultados em modelos maiores"; [IT]
"Vantaggi in velocità e memoria"): TokenGate also runs on a hybrid model
whose Gated DeltaNet layers are interleaved with full-attention layers, and it
prunes those recurrent layers too, where attention-only pruning methods
cannot.  Above the gate a Gated DeltaNet layer therefore runs its recurrence
over the kept rows only, in their original order: a dropped token never
enters the state.  The pages give no formula for the layer itself.

The recurrence is written from its published definition (Yang, Kautz and
Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR
2025: the gated delta rule), per value head h with a matrix state S
[dv, dk], a log-decay g_t (alpha_t = exp(g_t) <= 1) and a write strength
beta_t in [0, 1]:

    S  <- alpha_t S                         decay the whole memory
    S  <- S + beta_t (v_t - S k_t) k_t^T    delta rule: move the value stored
                                            at key k_t towards v_t
    o_t = scale * S q_t

Readings (the pages are silent): q and k arrive L2-normalised per head, as
the layer's own normalisation leaves them (so the write is a projection step);
``scale`` defaults to 1/sqrt(dk); value heads share q/k heads in groups
(value head h reads q/k head h // (Hv / Hk)); the gate's score bias acts on
the attention layers only, so the recurrence takes no score.

Everything is float64 numpy, one token at a time.  Pins:
tests/test_oracle_gdn_pins.py (zero write keeps the decayed state; a unit
write overwrites the value at its key; orthonormal keys reduce it to causal
linear attention, with and without decay, against torch; the unrolled product
of transition matrices; a chunked (WY) formulation on ragged chunks; state
carried across a split sequence; GQA grouping; pruning equals a full-length
run in which dropped tokens neither write nor decay).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["gated_delta_rule"]


def gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None, return_state=False):
    """Sequential gated delta rule.

    q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv] (log decay, write
    strength); initial_state [Hv, dv, dk] (zeros when None).
    Returns o [T, Hv, dv] float64 (and the final state [Hv, dv, dk] if asked).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    t_len, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    assert k.shape == (t_len, hk, dk) and v.shape == (t_len, hv, dv)
    assert g.shape == (t_len, hv) and beta.shape == (t_len, hv) and hv % hk == 0
    group = hv // hk
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    state = (np.zeros((hv, dv, dk)) if initial_state is None
             else np.array(initial_state, dtype=np.float64, copy=True))
    out = np.zeros((t_len, hv, dv))
    for h in range(hv):
        s = state[h]
        kh = h // group
        for t in range(t_len):
            s *= math.exp(g[t, h])
            kt = k[t, kh]
            s += beta[t, h] * np.outer(v[t, h] - s @ kt, kt)
            out[t, h] = scale * (s @ q[t, kh])
    return (out, state) if return_state else out
