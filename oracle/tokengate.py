"""Plain CPU oracle of the TokenGate gated prefill (test infrastructure).

What the method computes, in the order the coverage pages give it ([KO] "작동
방식"; [FR] lede; [IT] "Come funziona"; source tags are defined in
``oracle/__init__.py``):

  1. layers below the gate layer run over all N tokens (not modelled here: the
     post-attention residual of the gate layer is an input);
  2. at the gate layer a small MLP gives every token a score computed from its
     post-attention residual;
  3. a top-K selector keeps the best-scoring tokens of the *document* part of
     the prompt; the question is never pruned;
  4. only the kept rows go up: the layers above the gate see K tokens and build
     no KV entries for the dropped ones;
  5. above the gate, attention is *token-gated*: each kept key's score is added
     to the attention logits as a bias, with a learned gain and temperature per
     head ([KO] "작동 방식"; [PT] "TokenGate “ensina”…"; [ABS]).

Everything here is numpy in float64, written for a reader to check by eye; no
blocking or fusion beyond splitting query rows into blocks to bound memory,
which does not change any value.

Readings of points the pages leave open (each is also listed in the design
notes of the repository):

  * logit form: q.k / (sqrt(d) * tau_h) + g_h * s_j, with s_j the raw gate
    output of key j (the pages only say "score as a bias, per-head gain and
    temperature");
  * gate MLP: z = W1 h + b1, a = GELU(z) with the exact erf form, s = w2.a + b2,
    no normalisation inside the gate; every row is scored (question rows too,
    since their scores are their own key bias above the gate);
  * selection total order: scores are compared as float32 through a monotone
    32-bit key; -0.0 equals +0.0; NaN ranks below -inf; ties go to the lower
    token index; the kept set is therefore unique;
  * kept rows stay in ascending original order, so causality in compacted
    order equals causality in original positions; kept tokens keep their
    original RoPE positions (applied to q/k before attention);
  * the bias applies only to layers above the gate (the pages place it there).

Pins (tests in ``tests/test_oracle_pins.py``):
  gelu_erf         -- torch's erf GELU and x*Phi(x) from scipy.stats; limits.
  gate_scores      -- H_g = 1 detector special case vs torch GELU; linear
                      regime closed form; pure-Python loop brute force.
  score_keys       -- order agreement with Python float comparison on a
                      hand-built list incl. +-inf, +-0, NaN, denormals.
  topk_select      -- brute force over all k-subsets on tiny inputs (the unique
                      dominating subset); invariants; golden fixture.
  compact_rows     -- bytewise definition on random bytes.
  gated_attention  -- torch SDPA (fp64) with K=N, g=0, tau=1; masking identity
                      vs torch SDPA with an additive float mask on the full-N
                      problem; two-key closed form; first-row identity; a
                      dominant bias on one key returns that key's v; shift
                      invariance; temperature equivalence; golden fixture.
  gated_attention_bwd
                   -- central finite differences of gated_attention (every
                      input element, tiny sizes, float64); torch autograd
                      through torch SDPA (fp64) with the bias as an additive
                      float mask and q divided by tau; the score gradient sums
                      to zero (a common shift of all scores changes nothing).
  full_attention   -- torch SDPA (fp64, causal, GQA by repetition).
  qk_norm_rope     -- transformers' Qwen3 apply_rotary_pos_emb (with this
                      function's cos/sin) and Qwen3RMSNorm; Qwen3RotaryEmbedding's
                      cos/sin at small positions; position 0 is the identity;
                      rotation keeps each pair's norm; q.k after RoPE depends
                      only on the position difference.
  gated_decode     -- torch SDPA (fp64) for one query with the additive float
                      bias and the head's scale; equals the last row of
                      gated_attention when the new token is the last row;
                      one key returns its v; a dominant bias selects one key.
No function is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

__all__ = [
    "gelu_erf",
    "gate_scores",
    "score_keys",
    "kept_count",
    "topk_select",
    "compact_rows",
    "gated_attention",
    "gated_attention_bwd",
    "full_attention",
    "qk_norm_rope",
    "gated_decode",
    "gated_prefill",
]


# ---------------------------------------------------------------------------
# Gate: a small MLP scores every token from its post-attention residual
# ([KO] "작동 방식"; [FR] lede; [IT] "Come funziona").
# ---------------------------------------------------------------------------

def gelu_erf(x):
    """Exact GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def gate_scores(h, w1, b1, w2, b2, row_block: int = 4096):
    """Score s_i = w2 . GELU(W1 h_i + b1) + b2 for every row i.

    h  [N, H]     post-attention residual at the gate layer
    w1 [Hg, H]    first layer (out x in, as a linear layer stores it)
    b1 [Hg], w2 [Hg], b2 scalar
    Returns float64 [N].  Rows are processed in blocks only to bound memory.
    """
    h = np.asarray(h)
    w1 = np.asarray(w1, dtype=np.float64)
    b1 = np.asarray(b1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    n = h.shape[0]
    out = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, row_block):
        hb = h[r0:r0 + row_block].astype(np.float64)
        z = hb @ w1.T + b1
        out[r0:r0 + row_block] = gelu_erf(z) @ w2 + float(b2)
    return out


# ---------------------------------------------------------------------------
# Selection: top-K over the document part only; the question is always kept
# ([KO] "작동 방식"; [PT] "TokenGate “ensina”…"; [IT] "Come funziona").
# ---------------------------------------------------------------------------

def score_keys(scores_f32):
    """Map float32 scores to uint32 keys whose unsigned order is the total order.

    Non-negative floats get their sign bit set; negative floats are bit-flipped
    (so a larger magnitude sorts lower); -0.0 is first turned into +0.0 and any
    NaN maps to key 0, below -inf.
    """
    s = np.ascontiguousarray(np.asarray(scores_f32, dtype=np.float32))
    bits = s.view(np.uint32).copy()
    bits[bits == np.uint32(0x80000000)] = 0
    neg = (bits >> np.uint32(31)) == 1
    keys = np.where(neg, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)
    keys[np.isnan(s)] = 0
    return keys


def kept_count(n: int, doc_begin: int, doc_end: int, k_doc: int) -> int:
    """Rows that survive: min(K, N_doc) document rows plus every other row."""
    n_doc = doc_end - doc_begin
    return min(k_doc, n_doc) + (n - n_doc)


def topk_select(scores_f32, doc_begin: int, doc_end: int, k_doc: int):
    """Kept row indices, ascending, as int32.

    Document rows [doc_begin, doc_end) are ranked by (score key descending,
    index ascending) and the first min(K, N_doc) are kept; every row outside
    the document is kept.  The selection is decided in float32, the precision
    the scores are handed over in.
    """
    keys = score_keys(scores_f32)
    n = keys.shape[0]
    assert 0 <= doc_begin <= doc_end <= n and k_doc >= 0
    doc = np.arange(doc_begin, doc_end, dtype=np.int64)
    # np.lexsort: last key is primary.  Primary = key descending, i.e. the
    # complement ascending; secondary = index ascending.
    order = np.lexsort((doc, np.uint32(0xFFFFFFFF) - keys[doc_begin:doc_end]))
    k = min(k_doc, doc.size)
    chosen = doc[order[:k]]
    others = np.concatenate([np.arange(0, doc_begin), np.arange(doc_end, n)])
    return np.sort(np.concatenate([chosen, others])).astype(np.int32)


# ---------------------------------------------------------------------------
# Compaction: only kept rows go up; no KV rows exist for the dropped tokens
# ([KO] "작동 방식"; [FR] lede).
# ---------------------------------------------------------------------------

def compact_rows(idx, src):
    """dst[i] = src[idx[i]] (a copy of whole rows)."""
    return np.array(np.asarray(src)[np.asarray(idx, dtype=np.int64)], copy=True)


# ---------------------------------------------------------------------------
# Token-gated attention above the gate ([KO] "작동 방식"; [PT] "TokenGate
# “ensina”…"; [ABS]; [IT] "Come funziona").
# ---------------------------------------------------------------------------

def gated_attention(q, k, v, key_score, gain, tau, rows=None, return_lse=False,
                    row_block: int = 256):
    """Causal GQA attention with a per-key score bias.

    q [M, Hq, d]; k, v [M, Hkv, d]; key_score [M]; gain, tau [Hq].
    For query head h (KV head h // (Hq/Hkv)) and query row i:
        logit_ij = q_i.k_j / (sqrt(d) tau_h) + gain_h * key_score_j,  j <= i
        out_i    = sum_j softmax_j(logit_i.) v_j
    ``rows``: optional subset of query rows (each row depends only on keys
    0..i, so a subset is exact).  Returns float64 out [R, Hq, d] and, if asked,
    the natural-log log-sum-exp [Hq, R].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    m, hq, d = q.shape
    hkv = k.shape[1]
    assert k.shape == (m, hkv, d) and v.shape == (m, hkv, d) and hq % hkv == 0
    group = hq // hkv
    s = np.asarray(key_score, dtype=np.float64).reshape(m)
    gain = np.asarray(gain, dtype=np.float64).reshape(hq)
    tau = np.asarray(tau, dtype=np.float64).reshape(hq)
    rows = np.arange(m, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    r = rows.size
    out = np.zeros((r, hq, d), dtype=np.float64)
    lse = np.zeros((hq, r), dtype=np.float64)
    for h in range(hq):
        g = h // group
        kh = k[:, g, :].astype(np.float64)
        vh = v[:, g, :].astype(np.float64)
        scale = 1.0 / (math.sqrt(d) * tau[h])
        for b0 in range(0, r, row_block):
            rb = rows[b0:b0 + row_block]
            kend = int(rb.max()) + 1
            qb = q[rb, h, :].astype(np.float64)
            logits = (qb @ kh[:kend].T) * scale + gain[h] * s[None, :kend]
            j = np.arange(kend)[None, :]
            logits = np.where(j <= rb[:, None], logits, -np.inf)
            mx = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - mx)
            l = p.sum(axis=1, keepdims=True)
            out[b0:b0 + row_block, h, :] = (p @ vh[:kend]) / l
            lse[h, b0:b0 + row_block] = (mx + np.log(l))[:, 0]
    return (out, lse) if return_lse else out


def gated_attention_bwd(q, k, v, key_score, gain, tau, dout, row_block: int = 256):
    """Gradients of the token-gated attention above, for training the gate
    through the bias ([KO] "작동 방식": the score enters the logits as a bias, so
    the loss reaches the gate's scores through it; [ABS]).

    Given dout = dLoss/dout [M, Hq, d], returns float64 arrays
        dq [M, Hq, d], dk [M, Hkv, d], dv [M, Hkv, d],
        dscore [M], dgain [Hq], dtau [Hq].
    Chain rule, head by head, with the softmax recomputed from the inputs:
        p_ij      = softmax_j(logit_i.)            (causal: p_ij = 0 for j > i)
        dp_ij     = dout_i . v_j
        dlogit_ij = p_ij (dp_ij - sum_l p_il dp_il)   (softmax Jacobian)
        dq_i     += sum_j dlogit_ij k_j / (sqrt(d) tau_h)
        dk_j     += sum_i dlogit_ij q_i / (sqrt(d) tau_h)
        dv_j     += sum_i p_ij dout_i
        dscore_j += gain_h sum_i dlogit_ij
        dgain_h   = sum_ij dlogit_ij key_score_j
        dtau_h    = sum_ij dlogit_ij q_i.k_j * (-1 / (sqrt(d) tau_h^2))
    (K/V rows are shared by the heads of a group, so their gradients sum over
    those heads.)
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    m, hq, d = q.shape
    hkv = k.shape[1]
    assert k.shape == (m, hkv, d) and v.shape == (m, hkv, d) and hq % hkv == 0
    dout = np.asarray(dout, dtype=np.float64).reshape(m, hq, d)
    group = hq // hkv
    s = np.asarray(key_score, dtype=np.float64).reshape(m)
    gain = np.asarray(gain, dtype=np.float64).reshape(hq)
    tau = np.asarray(tau, dtype=np.float64).reshape(hq)
    dq = np.zeros((m, hq, d), dtype=np.float64)
    dk = np.zeros((m, hkv, d), dtype=np.float64)
    dv = np.zeros((m, hkv, d), dtype=np.float64)
    dscore = np.zeros(m, dtype=np.float64)
    dgain = np.zeros(hq, dtype=np.float64)
    dtau = np.zeros(hq, dtype=np.float64)
    for h in range(hq):
        g = h // group
        kh = k[:, g, :].astype(np.float64)
        vh = v[:, g, :].astype(np.float64)
        scale = 1.0 / (math.sqrt(d) * tau[h])
        for b0 in range(0, m, row_block):
            rb = np.arange(b0, min(b0 + row_block, m))
            kend = int(rb[-1]) + 1
            qb = q[rb, h, :].astype(np.float64)
            dob = dout[rb, h, :]
            qk = qb @ kh[:kend].T
            logits = qk * scale + gain[h] * s[None, :kend]
            visible = np.arange(kend)[None, :] <= rb[:, None]
            logits = np.where(visible, logits, -np.inf)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = dob @ vh[:kend].T
            dlogit = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[rb, h, :] += (dlogit @ kh[:kend]) * scale
            dk[:kend, g, :] += (dlogit.T @ qb) * scale
            dv[:kend, g, :] += p.T @ dob
            dscore[:kend] += gain[h] * dlogit.sum(axis=0)
            dgain[h] += (dlogit * s[None, :kend]).sum()
            dtau[h] += (dlogit * qk).sum() * (-1.0 / (math.sqrt(d) * tau[h] ** 2))
    return dict(dq=dq, dk=dk, dv=dv, dscore=dscore, dgain=dgain, dtau=dtau)


def full_attention(q, k, v, rows=None, return_lse=False):
    """Unpruned causal GQA attention over all N rows: the gated form with
    gain 0 and temperature 1, i.e. softmax(q.k / sqrt(d)) v."""
    n, hq, _ = np.asarray(q).shape
    return gated_attention(q, k, v, np.zeros(n), np.zeros(hq), np.ones(hq),
                           rows=rows, return_lse=return_lse)


# ---------------------------------------------------------------------------
# The upper layers' query/key prologue at the kept tokens' own positions
# ([KO] "작동 방식": only the kept tokens go up, as the tokens they are; their
# positions are their original ones).  Qwen3's per-head RMS normalisation of
# q and k followed by rotary position embedding (rotate-half) is model
# plumbing, not on the pages: written here from its definition.
# ---------------------------------------------------------------------------

def qk_norm_rope(x, positions, norm_weight=None, eps=1e-6, theta=1.0e6):
    """x [n, heads, d] -> RoPE(RMSNorm(x) * w) at the given positions, float64.

    RMSNorm over each head vector: x / sqrt(mean(x^2) + eps) * w (skipped when
    ``norm_weight`` is None).  RoPE, rotate-half form: for f < d/2 with angle
    a = position * theta^(-2f/d),
        out[f]       = y[f] cos a - y[f + d/2] sin a
        out[f + d/2] = y[f + d/2] cos a + y[f] sin a.
    """
    x = np.asarray(x, dtype=np.float64)
    n, heads, d = x.shape
    assert d % 2 == 0
    if norm_weight is not None:
        w = np.asarray(norm_weight, dtype=np.float64).reshape(d)
        x = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64).reshape(n)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------
# One decode step over the pruned KV cache ([KO] lede: time to first token;
# [KO] "작동 방식": above the gate only the kept tokens have KV entries, and
# their scores bias the logits there).
# ---------------------------------------------------------------------------

def gated_decode(q, k, v, key_score, gain, tau, return_lse=False):
    """One new query row per head against every cached key, with the score bias.

    q [Hq, d] (the new token's queries); k, v [n, Hkv, d] (the cache: the kept
    rows plus the new token's own row, appended by the caller); key_score [n];
    gain, tau [Hq].  For query head h (KV head h // (Hq/Hkv)):
        logit_j = q.k_j / (sqrt(d) tau_h) + gain_h * key_score_j,  0 <= j < n
        out     = sum_j softmax_j(logit) v_j
    (every cached row precedes or is the new token, so no key is masked).
    Returns float64 out [Hq, d] and, if asked, the natural-log log-sum-exp [Hq].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    hq, d = q.shape
    n, hkv, _ = k.shape
    assert k.shape == (n, hkv, d) and v.shape == (n, hkv, d) and hq % hkv == 0 and n > 0
    group = hq // hkv
    s = np.asarray(key_score, dtype=np.float64).reshape(n)
    gain = np.asarray(gain, dtype=np.float64).reshape(hq)
    tau = np.asarray(tau, dtype=np.float64).reshape(hq)
    out = np.zeros((hq, d), dtype=np.float64)
    lse = np.zeros(hq, dtype=np.float64)
    for h in range(hq):
        g = h // group
        logits = (k[:, g, :].astype(np.float64) @ q[h].astype(np.float64)) / (math.sqrt(d) * tau[h])
        logits = logits + gain[h] * s
        mx = logits.max()
        p = np.exp(logits - mx)
        l = p.sum()
        out[h] = (p @ v[:, g, :].astype(np.float64)) / l
        lse[h] = mx + math.log(l)
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------------------
# The three-stage forward ([KO] "작동 방식"; [FR] lede).
# ---------------------------------------------------------------------------

def gated_prefill(h, w1, b1, w2, b2, doc_begin, doc_end, k_doc, layers,
                  scores_f32=None, layer_ids=None, rows=None):
    """Score -> select -> compact -> token-gated attention for each upper layer.

    ``layers``: list of (q, k, v, gain, tau) where q/k/v are full-N rows of the
    upper layer (positions already encoded at the original ids); the kept rows
    are taken with the selected indices.  ``scores_f32``: optional float32
    scores to select on (the precision the selection is decided in); by default
    the oracle's own scores rounded to float32.
    Returns dict(scores, idx, h_kept, s_kept, outs={layer: out}).
    """
    s64 = gate_scores(h, w1, b1, w2, b2)
    s32 = s64.astype(np.float32) if scores_f32 is None else np.asarray(scores_f32, np.float32)
    idx = topk_select(s32, doc_begin, doc_end, k_doc)
    h_kept = compact_rows(idx, h)
    s_kept = compact_rows(idx, s32).astype(np.float64)
    outs = {}
    ids = range(len(layers)) if layer_ids is None else layer_ids
    for li in ids:
        q, k, v, gain, tau = layers[li]
        outs[li] = gated_attention(compact_rows(idx, q), compact_rows(idx, k),
                                   compact_rows(idx, v), s_kept, gain, tau, rows=rows)
    return dict(scores=s64, idx=idx, h_kept=h_kept, s_kept=s_kept, outs=outs)
