"""Pins of the Gated DeltaNet oracle (oracle/gated_deltanet.py) against things
other than itself: closed forms of the recurrence, torch's causal linear
attention (the special case of orthonormal keys), the unrolled product of the
recurrence's transition matrices, a chunked (WY) formulation of the same
recurrence, and invariants (state carried across a split, head grouping,
pruning as skipped tokens).  A slip in the oracle (decay after the write
instead of before, a missing beta, the delta taken against the undecayed
state, q and k swapped, a wrong head group) fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

from oracle import gated_deltanet as G


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(seed, t, hk=2, hv=4, dk=8, dv=6):
    rng = np.random.default_rng(seed)
    q = _unit(rng.standard_normal((t, hk, dk)))
    k = _unit(rng.standard_normal((t, hk, dk)))
    v = rng.standard_normal((t, hv, dv))
    g = -rng.uniform(0.0, 0.4, (t, hv))
    beta = rng.uniform(0.0, 1.0, (t, hv))
    return q, k, v, g, beta


def test_zero_write_keeps_the_decayed_state():
    """beta = 0: nothing is written, the state only decays:
    o_t = scale * exp(g_1 + ... + g_t) S_0 q_t."""
    q, k, v, g, _ = _case(1, 9)
    s0 = np.random.default_rng(2).standard_normal((4, 6, 8))
    out, st = G.gated_delta_rule(q, k, v, g, np.zeros_like(g), initial_state=s0, return_state=True)
    scale = 1 / math.sqrt(8)
    for h in range(4):
        for t in range(9):
            want = scale * math.exp(g[: t + 1, h].sum()) * (s0[h] @ q[t, h // 2])
            assert np.allclose(out[t, h], want, rtol=1e-13, atol=1e-15)
        assert np.allclose(st[h], math.exp(g[:, h].sum()) * s0[h], rtol=1e-13)


def test_unit_write_overwrites_the_value_at_its_key():
    """alpha = 1, beta = 1, one unit key written twice: the second write
    replaces the first, S = v_2 k^T, and reading at k returns v_2."""
    rng = np.random.default_rng(3)
    key = _unit(rng.standard_normal(5))
    v = rng.standard_normal((2, 1, 3))
    k = np.stack([key, key])[:, None, :]
    q = np.stack([key, _unit(rng.standard_normal(5))])[:, None, :]
    out, st = G.gated_delta_rule(q, k, v, np.zeros((2, 1)), np.ones((2, 1)), scale=1.0,
                                 return_state=True)
    assert np.allclose(st[0], np.outer(v[1, 0], key), atol=1e-14)
    assert np.allclose(st[0] @ key, v[1, 0], atol=1e-14)
    assert np.allclose(out[0, 0], v[0, 0], atol=1e-14)                 # read back at t = 0
    assert np.allclose(out[1, 0], v[1, 0] * (key @ q[1, 0]), atol=1e-14)


@pytest.mark.parametrize("decay", [False, True])
def test_orthonormal_keys_reduce_to_causal_linear_attention(decay):
    """Orthonormal keys (T <= dk): S_{t-1} k_t = 0, so every write adds
    beta_t v_t k_t^T and o_t = scale sum_{s<=t} (prod_{s<r<=t} alpha_r) beta_s
    (k_s.q_t) v_s, a decay-masked causal linear attention computed here with
    torch's tril / matmul."""
    rng = np.random.default_rng(4)
    t, dk, dv = 12, 16, 5
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[:t][:, None, :]
    q = _unit(rng.standard_normal((t, 1, dk)))
    v = rng.standard_normal((t, 1, dv))
    beta = rng.uniform(0.2, 1.0, (t, 1))
    g = -rng.uniform(0.0, 0.5, (t, 1)) if decay else np.zeros((t, 1))
    out = G.gated_delta_rule(q, k, v, g, beta)
    tq, tk, tv = (torch.from_numpy(x[:, 0]) for x in (q, k, v))
    cg = torch.cumsum(torch.from_numpy(g[:, 0]), 0)
    mask = torch.tril(torch.exp(cg[:, None] - cg[None, :]))       # prod over (s, t] of alpha
    att = torch.tril(tq @ tk.T) * mask * torch.from_numpy(beta[:, 0])[None, :]
    ref = (att @ tv).numpy() / math.sqrt(dk)
    assert np.allclose(out[:, 0], ref, rtol=1e-12, atol=1e-14)


def test_unrolled_product_of_transition_matrices():
    """S_t = S_{t-1} M_t + beta_t v_t k_t^T with M_t = alpha_t (I - beta_t k_t k_t^T),
    so S_t = S_0 M_1...M_t + sum_s beta_s v_s k_s^T M_{s+1}...M_t; every prefix
    state is built from that sum of products and o_t = scale S_t q_t."""
    q, k, v, g, beta = _case(5, 7, hk=1, hv=1, dk=6, dv=4)
    s0 = np.random.default_rng(6).standard_normal((1, 4, 6))
    out, st = G.gated_delta_rule(q, k, v, g, beta, initial_state=s0, return_state=True)
    eye = np.eye(6)
    m = [math.exp(g[t, 0]) * (eye - beta[t, 0] * np.outer(k[t, 0], k[t, 0])) for t in range(7)]

    def prod(a, b):
        r = eye.copy()
        for j in range(a, b):
            r = r @ m[j]
        return r

    for t in range(7):
        s = s0[0] @ prod(0, t + 1)
        for u in range(t + 1):
            s = s + beta[u, 0] * np.outer(v[u, 0], k[u, 0]) @ prod(u + 1, t + 1)
        assert np.allclose(out[t, 0], (s @ q[t, 0]) / math.sqrt(6), rtol=1e-12, atol=1e-14)
    assert np.allclose(st[0], s, rtol=1e-12, atol=1e-14)


def _chunked(q, k, v, g, beta, chunk, scale):
    """The recurrence in chunks (WY form): inside a chunk with start state S,
    cumulative log decay c_i and Gam_i = exp(c_i), the written deltas
    u_i = beta_i (v_i - alpha_i S_{i-1} k_i) solve (I + A) U = diag(beta) V -
    diag(beta Gam) K S^T with A_ij = beta_i exp(c_i - c_j) k_i.k_j (j < i); then
    O = scale (diag(Gam) Q S^T + (exp(c_i - c_j) q_i.k_j)_{j<=i} U) and the next
    state is Gam_last S + U^T diag(exp(c_last - c)) K."""
    t_len, hk, dk = q.shape
    hv, dv = v.shape[1:]
    out = np.zeros((t_len, hv, dv))
    for h in range(hv):
        kh = h // (hv // hk)
        s = np.zeros((dv, dk))
        for c0 in range(0, t_len, chunk):
            sl = slice(c0, min(c0 + chunk, t_len))
            Q, K, V, b = q[sl, kh], k[sl, kh], v[sl, h], beta[sl, h]
            c = np.cumsum(g[sl, h])
            n = c.size
            dec = np.exp(c[:, None] - c[None, :])
            A = np.tril(b[:, None] * dec * (K @ K.T), -1)
            rhs = b[:, None] * V - (b * np.exp(c))[:, None] * (K @ s.T)
            U = np.linalg.solve(np.eye(n) + A, rhs)
            P = np.tril(dec * (Q @ K.T))
            out[sl, h] = scale * (np.exp(c)[:, None] * (Q @ s.T) + P @ U)
            s = math.exp(c[-1]) * s + U.T @ (np.exp(c[-1] - c)[:, None] * K)
    return out


@pytest.mark.parametrize("chunk", [1, 3, 4, 64])
def test_chunked_formulation_equals_the_sequential_recurrence(chunk):
    q, k, v, g, beta = _case(7, 13)
    out = G.gated_delta_rule(q, k, v, g, beta)
    ref = _chunked(q, k, v, g, beta, chunk, 1 / math.sqrt(8))
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_state_carries_across_a_split_sequence():
    q, k, v, g, beta = _case(8, 11)
    whole, s_end = G.gated_delta_rule(q, k, v, g, beta, return_state=True)
    a, s_mid = G.gated_delta_rule(q[:4], k[:4], v[:4], g[:4], beta[:4], return_state=True)
    b, s_two = G.gated_delta_rule(q[4:], k[4:], v[4:], g[4:], beta[4:], initial_state=s_mid,
                                  return_state=True)
    assert np.allclose(np.concatenate([a, b]), whole, rtol=1e-13, atol=1e-15)
    assert np.allclose(s_two, s_end, rtol=1e-13, atol=1e-15)


def test_value_heads_share_query_key_heads_in_groups():
    """Hv = 2 Hk: value head h reads q/k head h // 2, which equals giving every
    value head its own copy of that q/k head."""
    q, k, v, g, beta = _case(9, 6, hk=2, hv=4)
    out = G.gated_delta_rule(q, k, v, g, beta)
    rep = G.gated_delta_rule(np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1), v, g, beta)
    assert np.array_equal(out, rep)


def test_pruned_rows_equal_rows_that_neither_write_nor_decay():
    """Running over the kept rows only equals a full-length run in which every
    dropped row has beta = 0 and g = 0 (it leaves the state untouched), read
    at the kept rows: the pruned recurrence skips the dropped tokens."""
    q, k, v, g, beta = _case(10, 15)
    keep = np.array([0, 2, 3, 7, 8, 11, 14])
    pruned = G.gated_delta_rule(q[keep], k[keep], v[keep], g[keep], beta[keep])
    g2, b2 = np.zeros_like(g), np.zeros_like(beta)
    g2[keep], b2[keep] = g[keep], beta[keep]
    full = G.gated_delta_rule(q, k, v, g2, b2)
    assert np.allclose(full[keep], pruned, rtol=1e-13, atol=1e-15)
    # and keeping every row is the plain full-length recurrence
    assert np.array_equal(G.gated_delta_rule(q, k, v, g, beta),
                          G.gated_delta_rule(q[np.arange(15)], k, v, g, beta))
