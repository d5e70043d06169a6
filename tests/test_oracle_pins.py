"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a library routine (torch's erf
GELU, torch's scaled-dot-product attention, scipy's normal CDF), a closed form,
a brute-force enumeration on tiny inputs, or an invariant the coverage pages
state (question never pruned, exactly K document tokens kept, bias only on kept
keys).  A plausible slip in the oracle (dropped bias term, temperature on the
wrong side, a wrong head group, an off-by-one causal mask, a wrong tie order)
fails at least one of them.
"""

import itertools
import math

import numpy as np
import pytest
import scipy.stats
import torch
import torch.nn.functional as F

from learned_token_pruning_tg_amd import inputs
from oracle import tokengate as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------- GELU / gate

def test_gelu_matches_torch_erf_gelu_and_x_phi():
    x = np.linspace(-9, 9, 4001)
    ref_t = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    ref_phi = x * scipy.stats.norm.cdf(x)
    got = O.gelu_erf(x)
    assert np.max(np.abs(got - ref_t)) < 1e-14
    assert np.max(np.abs(got - ref_phi)) < 1e-14
    assert O.gelu_erf(0.0) == 0.0
    assert abs(O.gelu_erf(12.0) - 12.0) < 1e-15
    assert abs(O.gelu_erf(-12.0)) < 1e-30


def test_gate_detector_special_case_is_gelu_of_first_feature():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((50, 7))
    w1 = np.zeros((1, 7)); w1[0, 0] = 1.0
    s = O.gate_scores(h, w1, np.zeros(1), np.ones(1), 0.0)
    ref = F.gelu(torch.from_numpy(h[:, 0]), approximate="none").numpy()
    assert np.max(np.abs(s - ref)) < 1e-14


def test_gate_matches_torch_mlp():
    rng = np.random.default_rng(1)
    n, hdim, hg = 37, 24, 11
    h = rng.standard_normal((n, hdim)); w1 = rng.standard_normal((hg, hdim)) * 0.3
    b1 = rng.standard_normal(hg); w2 = rng.standard_normal(hg); b2 = 0.7
    lin1 = torch.nn.Linear(hdim, hg, dtype=torch.float64)
    lin2 = torch.nn.Linear(hg, 1, dtype=torch.float64)
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1)); lin1.bias.copy_(torch.from_numpy(b1))
        lin2.weight.copy_(torch.from_numpy(w2)[None]); lin2.bias.fill_(b2)
        ref = lin2(F.gelu(lin1(torch.from_numpy(h)), approximate="none"))[:, 0].numpy()
    assert np.max(np.abs(O.gate_scores(h, w1, b1, w2, b2, row_block=8) - ref)) < 1e-12


def test_gate_linear_and_dead_regimes():
    # b1 >> 0: GELU(z) = z, so s = (w2 W1) h + w2.b1 + b2; b1 << 0: s = b2.
    rng = np.random.default_rng(2)
    h = rng.standard_normal((20, 9)); w1 = rng.standard_normal((5, 9)) * 0.1
    w2 = rng.standard_normal(5)
    s = O.gate_scores(h, w1, np.full(5, 60.0), w2, -1.5)
    ref = h @ (w2 @ w1) + 60.0 * w2.sum() - 1.5
    assert np.max(np.abs(s - ref)) < 1e-10
    s = O.gate_scores(h, w1, np.full(5, -60.0), w2, -1.5)
    assert np.max(np.abs(s + 1.5)) < 1e-30


def test_gate_brute_force_loops():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((4, 5)); w1 = rng.standard_normal((3, 5))
    b1 = rng.standard_normal(3); w2 = rng.standard_normal(3); b2 = 0.25
    for i in range(4):
        acc = b2
        for j in range(3):
            z = b1[j] + sum(w1[j, c] * h[i, c] for c in range(5))
            acc += w2[j] * z * 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))
        assert abs(O.gate_scores(h, w1, b1, w2, b2)[i] - acc) < 1e-13


# --------------------------------------------------------------------------- keys / top-K

def _beats(a, ia, b, ib):
    """Total order of the selection: larger score first, NaN last, -0 == +0,
    ties to the lower index.  Written with Python float comparisons."""
    an, bn = math.isnan(a), math.isnan(b)
    if an and bn:
        return ia < ib
    if an != bn:
        return bn
    if a != b:
        return a > b
    return ia < ib


def test_score_keys_order_matches_float_order():
    vals = [float("-inf"), -3.4e38, -1.0, -1e-45, -0.0, 0.0, 1e-45, 1e-38, 0.5, 1.0,
            3.4e38, float("inf")]
    vals32 = np.array(vals, dtype=np.float32)
    keys = O.score_keys(vals32)
    for i in range(len(vals)):
        for j in range(len(vals)):
            a, b = float(vals32[i]), float(vals32[j])
            assert (keys[i] > keys[j]) == (a > b), (a, b)
            assert (keys[i] == keys[j]) == (a == b), (a, b)
    nan = O.score_keys(np.array([np.nan, -np.inf], dtype=np.float32))
    assert nan[0] < nan[1]


def _brute_force_topk(scores, db, de, k):
    doc = list(range(db, de))
    k = min(k, len(doc))
    winners = []
    for sub in itertools.combinations(doc, k):
        kept = set(sub)
        dropped = [j for j in doc if j not in kept]
        if all(_beats(float(scores[a]), a, float(scores[b]), b) for a in kept for b in dropped):
            winners.append(sub)
    assert len(winners) == 1, "the total order must make the kept set unique"
    others = [i for i in range(len(scores)) if not (db <= i < de)]
    return sorted(list(winners[0]) + others)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    n = 10
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, -1.0, 1.0, 0.5, 2.0], dtype=np.float32)
    scores = rng.choice(pool, size=n) if seed % 2 else np.round(rng.standard_normal(n), 0)
    scores = scores.astype(np.float32)
    db, de = int(rng.integers(0, 3)), int(rng.integers(6, n + 1))
    for k in range(0, de - db + 2):
        got = O.topk_select(scores, db, de, k)
        assert got.dtype == np.int32
        assert got.tolist() == _brute_force_topk(scores, db, de, k)


def test_topk_invariants_on_tiny_workload():
    w = inputs.WORKLOADS["tiny"]
    g = inputs.gate_inputs(w)
    s = O.gate_scores(g["h"], g["w1"], g["b1"], g["w2"], g["b2"]).astype(np.float32)
    for k in (0, 1, 64, 128, 447, 448, 1000):
        idx = O.topk_select(s, w.doc_begin, w.doc_end, k)
        assert idx.size == O.kept_count(w.n, w.doc_begin, w.doc_end, k)
        assert np.all(np.diff(idx) > 0)
        doc_kept = idx[idx < w.n_doc]
        assert doc_kept.size == min(k, w.n_doc)                       # exactly K document rows
        assert set(range(w.n_doc, w.n)) <= set(idx.tolist())           # question never pruned
        dropped = np.setdiff1d(np.arange(w.n_doc), doc_kept)
        if doc_kept.size and dropped.size:                             # threshold separation
            assert s[doc_kept].min() >= s[dropped].max()
        # equals a full stable sort
        order = sorted(range(w.n_doc), key=lambda i: (-float(s[i]), i))[:min(k, w.n_doc)]
        assert sorted(order) == doc_kept.tolist()


def test_topk_special_cases():
    s = np.full(12, 0.25, dtype=np.float32)
    assert O.topk_select(s, 2, 9, 3).tolist() == [0, 1, 2, 3, 4, 9, 10, 11]   # all ties: lowest
    assert O.topk_select(s, 0, 12, 0).tolist() == []
    assert O.topk_select(s, 4, 4, 5).tolist() == list(range(12))               # empty document
    assert O.topk_select(s, 0, 12, 99).tolist() == list(range(12))
    assert O.topk_select(np.zeros(0, np.float32), 0, 0, 3).tolist() == []


# --------------------------------------------------------------------------- compaction

def test_compact_rows_bytewise():
    rng = np.random.default_rng(4)
    src = rng.integers(0, 256, size=(40, 13), dtype=np.uint8)
    idx = np.array([0, 3, 4, 17, 39], dtype=np.int32)
    dst = O.compact_rows(idx, src)
    for r, i in enumerate(idx):
        assert dst[r].tobytes() == src[i].tobytes()
    dst[0, 0] ^= 1
    assert src[0, 0] != dst[0, 0]        # a copy, not a view


# --------------------------------------------------------------------------- attention

def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch SDPA in float64 on [n, heads, d] arrays; KV heads repeated for GQA."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


def _rand_qkv(rng, n, hq, hkv, d):
    return (rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)),
            rng.standard_normal((n, hkv, d)))


def test_attention_k_equals_n_no_gain_is_causal_sdpa():
    rng = np.random.default_rng(5)
    q, k, v = _rand_qkv(rng, 70, 4, 2, 16)
    s = rng.standard_normal(70) * 3
    got = O.gated_attention(q, k, v, s, np.zeros(4), np.ones(4), row_block=16)
    assert np.max(np.abs(got - _sdpa(q, k, v, causal=True))) < 1e-12
    assert np.max(np.abs(O.full_attention(q, k, v) - _sdpa(q, k, v, causal=True))) < 1e-12


def test_gated_attention_masking_identity_vs_sdpa():
    """Gated attention over the kept rows == full-N attention whose mask is
    gain_h * s_j on kept keys (j <= i) and -inf elsewhere, at scale 1/(sqrt(d) tau_h),
    read at the kept query rows.  Pins bias placement, temperature and GQA grouping."""
    rng = np.random.default_rng(6)
    n, hq, hkv, d = 48, 4, 2, 8
    q, k, v = _rand_qkv(rng, n, hq, hkv, d)
    s = rng.standard_normal(n).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq); tau = rng.uniform(0.8, 1.2, hq)
    idx = O.topk_select(s, 0, 40, 13)
    got = O.gated_attention(q[idx], k[idx], v[idx], s[idx].astype(np.float64), gain, tau)
    kept = np.zeros(n, bool); kept[idx] = True
    causal = np.tril(np.ones((n, n), bool))
    for h in range(hq):
        mask = np.where(causal & kept[None, :], gain[h] * s[None, :].astype(np.float64), -np.inf)
        g = h // (hq // hkv)
        ref = _sdpa(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], mask=mask,
                    scale=1.0 / (math.sqrt(d) * tau[h]))
        assert np.max(np.abs(got[:, h] - ref[idx, 0])) < 1e-12


# ----------------------------------------------------------- attention backward

def _bwd_case(seed, m=6, hq=4, hkv=2, d=4, row_block=256):
    rng = np.random.default_rng(seed)
    q, k, v = _rand_qkv(rng, m, hq, hkv, d)
    s = rng.standard_normal(m) * 1.5
    gain = rng.uniform(0.5, 1.5, hq); tau = rng.uniform(0.8, 1.2, hq)
    dout = rng.standard_normal((m, hq, d))
    return q, k, v, s, gain, tau, dout


def test_attention_bwd_finite_differences_every_input():
    """Central differences of sum(dout * gated_attention(...)) in float64, for
    every element of q, k, v, the scores, the gains and the temperatures.
    row_block=2 also exercises the row blocking of both functions."""
    q, k, v, s, gain, tau, dout = _bwd_case(11)
    args = dict(q=q, k=k, v=v, key_score=s, gain=gain, tau=tau)
    got = O.gated_attention_bwd(q, k, v, s, gain, tau, dout, row_block=2)
    names = dict(q="dq", k="dk", v="dv", key_score="dscore", gain="dgain", tau="dtau")
    eps = 1e-6
    for arg, gname in names.items():
        base = args[arg]
        fd = np.zeros_like(base)
        for ix in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[ix] += eps; minus[ix] -= eps
            lp = np.sum(dout * O.gated_attention(**{**args, arg: plus}, row_block=3))
            lm = np.sum(dout * O.gated_attention(**{**args, arg: minus}, row_block=3))
            fd[ix] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(got[gname] - fd)) / max(np.max(np.abs(fd)), 1e-3)
        assert err < 1e-6, (gname, err)


def test_attention_bwd_matches_torch_autograd_through_sdpa():
    """torch autograd (float64) through torch SDPA, one head at a time: q/tau_h
    at scale 1/sqrt(d), the bias gain_h * s_j as an additive float mask with -inf
    above the diagonal; K/V rows gathered per head so their gradients sum over
    the group."""
    m, hq, hkv, d = 37, 4, 2, 16
    q, k, v, s, gain, tau, dout = _bwd_case(12, m, hq, hkv, d)
    got = O.gated_attention_bwd(q, k, v, s, gain, tau, dout, row_block=16)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, ts, tg, tt = T(q), T(k), T(v), T(s), T(gain), T(tau)
    causal = torch.tril(torch.ones(m, m, dtype=torch.bool))
    loss = 0
    for h in range(hq):
        g = h // (hq // hkv)
        mask = torch.where(causal, tg[h] * ts[None, :], torch.tensor(-math.inf, dtype=torch.float64))
        o = F.scaled_dot_product_attention((tq[:, h] / tt[h])[None], tk[:, g][None], tv[:, g][None],
                                           attn_mask=mask[None], scale=1.0 / math.sqrt(d))
        loss = loss + (o[0] * torch.from_numpy(dout[:, h])).sum()
    loss.backward()
    for gname, t in dict(dq=tq, dk=tk, dv=tv, dscore=ts, dgain=tg, dtau=tt).items():
        assert np.max(np.abs(got[gname] - t.grad.numpy())) < 1e-10, gname


def test_attention_bwd_score_gradient_sums_to_zero():
    """Adding one constant to every score moves each row's logits together, so
    the output and hence the loss do not change: sum_j dscore_j = 0; with all
    scores equal the gains get no gradient either."""
    q, k, v, s, gain, tau, dout = _bwd_case(13, 40, 4, 1, 8)
    got = O.gated_attention_bwd(q, k, v, s, gain, tau, dout, row_block=8)
    assert abs(got["dscore"].sum()) < 1e-10 * np.abs(got["dscore"]).sum()
    flat = O.gated_attention_bwd(q, k, v, np.full(40, 0.7), gain, tau, dout)
    assert np.max(np.abs(flat["dgain"])) < 1e-10


def _term_sums_by_loops(q, k, v, s, gain, tau, dout):
    """The GPU bars' term-magnitude sums written as plain loops over every
    (head, query row, key): softmax p_ij from its definition, dp_ij = dout_i.v_j,
    D_i = sum_j p_ij dp_ij, A_i = sum_f |dout_if out_if| with out_i = sum_j p_ij v_j,
    mag_ij = p_ij (|dp_ij - D_i| + A_i)."""
    m, hq, d = q.shape
    group = hq // k.shape[1]
    sc = np.zeros(m); sg = np.zeros(hq); st = np.zeros(hq)
    for h in range(hq):
        g = h // group
        c = 1.0 / (math.sqrt(d) * tau[h])
        for i in range(m):
            lg = [sum(q[i, h, f] * k[j, g, f] for f in range(d)) * c + gain[h] * s[j]
                  for j in range(i + 1)]
            top = max(lg)
            e = [math.exp(x - top) for x in lg]
            p = [x / sum(e) for x in e]
            dp = [sum(dout[i, h, f] * v[j, g, f] for f in range(d)) for j in range(i + 1)]
            dsum = sum(p[j] * dp[j] for j in range(i + 1))
            out = [sum(p[j] * v[j, g, f] for j in range(i + 1)) for f in range(d)]
            a = sum(abs(dout[i, h, f] * out[f]) for f in range(d))
            for j in range(i + 1):
                mag = p[j] * (abs(dp[j] - dsum) + a)
                qk = sum(q[i, h, f] * k[j, g, f] for f in range(d))
                sc[j] += abs(gain[h]) * mag
                sg[h] += mag * abs(s[j])
                st[h] += mag * abs(qk) / (math.sqrt(d) * tau[h] ** 2)
    return dict(dscore=sc, dgain=sg, dtau=st)


@pytest.mark.parametrize("row_block", [1, 3, 256])
def test_bwd_bound_sums_match_plain_loops(row_block):
    """tests/bwd_bounds.py (the GPU bars of the score, gain and temperature
    gradients) against plain loops; and the sums dominate the oracle's
    gradients they describe (|sum dS x| <= sum |dS| |x| with |dS_ij| <=
    p_ij |dp_ij - D_i|)."""
    from bwd_bounds import term_magnitude_sums
    q, k, v, s, gain, tau, dout = _bwd_case(14, 7, 4, 2, 5)
    got = term_magnitude_sums(q, k, v, s, gain, tau, dout, row_block=row_block)
    ref = _term_sums_by_loops(q, k, v, s, gain, tau, dout)
    grads = O.gated_attention_bwd(q, k, v, s, gain, tau, dout)
    for name in ("dscore", "dgain", "dtau"):
        assert np.allclose(got[name], ref[name], rtol=1e-12, atol=0), name
        assert np.all(got[name] >= np.abs(grads[name])), name


def test_attention_two_key_closed_form_and_first_row():
    rng = np.random.default_rng(7)
    d = 6
    q, k, v = _rand_qkv(rng, 2, 1, 1, d)
    s = np.array([0.8, -0.3]); gain = np.array([1.3]); tau = np.array([0.9])
    out, lse = O.gated_attention(q, k, v, s, gain, tau, return_lse=True)
    assert np.array_equal(out[0, 0], v[0, 0])                      # a single visible key
    l0 = q[1, 0] @ k[0, 0] / (math.sqrt(d) * 0.9) + 1.3 * 0.8
    l1 = q[1, 0] @ k[1, 0] / (math.sqrt(d) * 0.9) + 1.3 * -0.3
    p0 = 1.0 / (1.0 + math.exp(l1 - l0))
    assert np.max(np.abs(out[1, 0] - (p0 * v[0, 0] + (1 - p0) * v[1, 0]))) < 1e-14
    assert abs(lse[0, 1] - (max(l0, l1) + math.log1p(math.exp(-abs(l0 - l1))))) < 1e-13
    l00 = q[0, 0] @ k[0, 0] / (math.sqrt(d) * 0.9) + 1.3 * 0.8
    assert abs(lse[0, 0] - l00) < 1e-13


def test_attention_dominant_bias_selects_one_key():
    """gain * s_j -> +inf for a single key j drives every row that sees it to
    v_j (the softmax collapses onto that key); rows before j are untouched."""
    rng = np.random.default_rng(12)
    n, d, j = 12, 8, 5
    q, k, v = _rand_qkv(rng, n, 2, 1, d)
    s = np.zeros(n); s[j] = 1.0
    base = O.gated_attention(q, k, v, s, np.array([0.0, 0.0]), np.ones(2))
    big = O.gated_attention(q, k, v, s, np.array([60.0, 80.0]), np.ones(2))
    for i in range(n):
        for h in range(2):
            if i >= j:
                assert np.max(np.abs(big[i, h] - v[j, 0])) < 1e-12
            else:
                assert np.array_equal(big[i, h], base[i, h])   # key j is not visible yet


def test_decode_vs_sdpa_one_query_with_bias():
    """One query per head against n cached keys == torch SDPA with the additive
    float bias gain_h * s_j and scale 1/(sqrt(d) tau_h), GQA by repetition."""
    rng = np.random.default_rng(21)
    n, hq, hkv, d = 37, 8, 2, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((n, hkv, d)); v = rng.standard_normal((n, hkv, d))
    s = rng.standard_normal(n) * 2
    gain = rng.uniform(0.5, 1.5, hq); tau = rng.uniform(0.8, 1.2, hq)
    got, lse = O.gated_decode(q, k, v, s, gain, tau, return_lse=True)
    for h in range(hq):
        g = h // (hq // hkv)
        ref = _sdpa(q[None, h:h + 1], k[:, g:g + 1], v[:, g:g + 1],
                    mask=(gain[h] * s)[None, :], scale=1.0 / (math.sqrt(d) * tau[h]))
        assert np.max(np.abs(got[h] - ref[0, 0])) < 1e-12
        logits = torch.from_numpy(k[:, g] @ q[h] / (math.sqrt(d) * tau[h]) + gain[h] * s)
        assert abs(lse[h] - torch.logsumexp(logits, 0).item()) < 1e-12


def test_decode_is_the_last_row_of_prefill_attention():
    """With the new token appended as the last cached row, its decode output is
    the last row of causal gated attention over the cache (that row sees every key)."""
    rng = np.random.default_rng(22)
    n, hq, hkv, d = 29, 4, 2, 8
    q, k, v = _rand_qkv(rng, n, hq, hkv, d)
    s = rng.standard_normal(n)
    gain = rng.uniform(0.5, 1.5, hq); tau = rng.uniform(0.8, 1.2, hq)
    pre, pre_lse = O.gated_attention(q, k, v, s, gain, tau, return_lse=True)
    dec, dec_lse = O.gated_decode(q[-1], k, v, s, gain, tau, return_lse=True)
    assert np.max(np.abs(dec - pre[-1])) < 1e-13
    assert np.max(np.abs(dec_lse - pre_lse[:, -1])) < 1e-13


def test_decode_single_key_and_dominant_bias():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((2, 8)); k = rng.standard_normal((6, 1, 8)); v = rng.standard_normal((6, 1, 8))
    one = O.gated_decode(q, k[:1], v[:1], np.array([0.7]), np.ones(2), np.ones(2))
    assert np.array_equal(one, np.repeat(v[:1, 0], 2, axis=0))      # softmax of one logit is 1
    s = np.zeros(6); s[3] = 1.0
    big = O.gated_decode(q, k, v, s, np.array([70.0, 90.0]), np.ones(2))
    assert np.max(np.abs(big - v[3, 0][None, :])) < 1e-12


def test_qk_norm_rope_vs_transformers_qwen3():
    """The rotation convention against transformers' Qwen3 apply_rotary_pos_emb
    (fed this oracle's own angles), the normalisation against Qwen3RMSNorm, and
    the frequency table against Qwen3RotaryEmbedding at small positions (it
    computes in float32)."""
    from transformers import Qwen3Config
    from transformers.models.qwen3 import modeling_qwen3 as q3
    rng = np.random.default_rng(31)
    n, heads, d, theta, eps = 9, 3, 16, 1.0e6, 1e-6
    x = rng.standard_normal((n, heads, d)) * 2
    w = rng.uniform(0.5, 1.5, d)
    pos = rng.integers(0, 1500, n)
    got = O.qk_norm_rope(x, pos, w, eps=eps, theta=theta)
    # RMSNorm (float32 inside the library)
    norm = q3.Qwen3RMSNorm(d, eps=eps).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(w))
        xn = norm(torch.from_numpy(x)).numpy()
    # rotation with the oracle's cos/sin in the library's [n, 1, d] layout
    ang = pos[:, None].astype(np.float64) * theta ** (-2.0 * np.arange(d // 2) / d)[None, :]
    cos = torch.from_numpy(np.cos(np.concatenate([ang, ang], -1)))[None]
    sin = torch.from_numpy(np.sin(np.concatenate([ang, ang], -1)))[None]
    xt = torch.from_numpy(xn).permute(1, 0, 2)[None]            # [1, heads, n, d]
    rq, _ = q3.apply_rotary_pos_emb(xt, xt, cos, sin)
    ref = rq[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - ref)) < 1e-5 * np.max(np.abs(ref))   # the norm ran in float32
    no_norm = O.qk_norm_rope(x, pos, None, theta=theta)
    rq2, _ = q3.apply_rotary_pos_emb(torch.from_numpy(x).permute(1, 0, 2)[None],
                                     torch.from_numpy(x).permute(1, 0, 2)[None], cos, sin)
    assert np.max(np.abs(no_norm - rq2[0].permute(1, 0, 2).numpy())) < 1e-12
    # the library's own frequency table (float32) at these positions
    cfg = Qwen3Config(head_dim=d, rope_parameters={"rope_type": "default", "rope_theta": theta},
                      max_position_embeddings=4096)
    rot = q3.Qwen3RotaryEmbedding(cfg)
    c32, s32 = rot(torch.zeros(1, dtype=torch.float32), torch.from_numpy(pos)[None])
    assert np.max(np.abs(c32[0].double().numpy() - cos[0].numpy())) < 2e-4
    assert np.max(np.abs(s32[0].double().numpy() - sin[0].numpy())) < 2e-4


def test_qk_norm_rope_invariants():
    rng = np.random.default_rng(32)
    n, heads, d = 6, 2, 32
    x = rng.standard_normal((n, heads, d))
    # position 0: rotation is the identity
    assert np.max(np.abs(O.qk_norm_rope(x, np.zeros(n), None) - x)) < 1e-15
    # each (f, f + d/2) pair keeps its length
    y = O.qk_norm_rope(x, rng.integers(0, 10 ** 5, n), None)
    h = d // 2
    assert np.max(np.abs((y[..., :h] ** 2 + y[..., h:] ** 2) - (x[..., :h] ** 2 + x[..., h:] ** 2))) < 1e-9
    # q.k after rotation depends only on the position difference
    q = rng.standard_normal((1, 1, d)); k = rng.standard_normal((1, 1, d))
    dots = [np.sum(O.qk_norm_rope(q, [p + 37], None) * O.qk_norm_rope(k, [p], None))
            for p in (0, 11, 5000, 123456)]
    assert np.max(np.abs(np.array(dots) - dots[0])) < 1e-9
    # RMSNorm with unit weight gives unit root-mean-square
    z = O.qk_norm_rope(x * 7, np.zeros(n), np.ones(d), eps=0.0)
    assert np.max(np.abs(np.sqrt(np.mean(z ** 2, axis=-1)) - 1)) < 1e-12


def test_attention_uniform_logits_lse_and_mean():
    # q = 0 and s = 0: every visible key has logit 0, so lse_i = log(i+1) and
    # out_i is the running mean of v.
    rng = np.random.default_rng(8)
    v = rng.standard_normal((9, 1, 4))
    out, lse = O.gated_attention(np.zeros((9, 2, 4)), rng.standard_normal((9, 1, 4)), v,
                                 np.zeros(9), np.ones(2), np.ones(2), return_lse=True)
    for i in range(9):
        assert abs(lse[1, i] - math.log(i + 1)) < 1e-14
        assert np.max(np.abs(out[i, 1] - v[:i + 1, 0].mean(axis=0))) < 1e-14


def test_attention_shift_invariance_and_temperature_equivalence():
    rng = np.random.default_rng(9)
    q, k, v = _rand_qkv(rng, 33, 2, 1, 8)
    const = np.full(33, 2.5)
    a = O.gated_attention(q, k, v, const, np.array([0.1, 1.4]), np.array([1.0, 1.1]))
    b = O.gated_attention(q, k, v, const, np.array([3.0, -2.0]), np.array([1.0, 1.1]))
    assert np.max(np.abs(a - b)) < 1e-12                  # a constant bias cancels
    tau = np.array([0.7, 1.3]); s = rng.standard_normal(33)
    c = O.gated_attention(q, k, v, s, np.array([1.0, 1.0]), tau)
    d2 = O.gated_attention(q / tau[None, :, None], k, v, s, np.array([1.0, 1.0]), np.ones(2))
    assert np.max(np.abs(c - d2)) < 1e-12                 # temperature divides q.k only


def test_attention_rows_subset_is_exact():
    rng = np.random.default_rng(10)
    q, k, v = _rand_qkv(rng, 50, 2, 2, 8)
    s = rng.standard_normal(50)
    full = O.gated_attention(q, k, v, s, np.ones(2), np.ones(2))
    rows = np.array([0, 7, 49, 23])
    sub = O.gated_attention(q, k, v, s, np.ones(2), np.ones(2), rows=rows, row_block=3)
    assert np.max(np.abs(full[rows] - sub)) < 1e-13


def test_original_positions_are_load_bearing():
    """With RoPE at original positions the gated output equals the masked
    full-N computation; re-encoding the kept rows at positions 0..M-1 does not."""
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.qkv_template(w, 0)
    rng = np.random.default_rng(11)
    s = rng.standard_normal(w.n).astype(np.float32)
    idx = O.topk_select(s, 0, w.n_doc, 32)
    gain = np.ones(w.n_q_heads); tau = np.ones(w.n_q_heads)
    kept = O.gated_attention(q[idx], k[idx], v[idx], s[idx], gain, tau)
    # undo the original-position encoding and re-encode at compacted positions
    def reenc(x):
        raw = inputs.apply_rope(x[idx].astype(np.float32), -idx.astype(np.float64))
        return inputs.apply_rope(raw, np.arange(idx.size))
    other = O.gated_attention(reenc(q), reenc(k), v[idx], s[idx], gain, tau)
    assert np.max(np.abs(kept - other)) > 1e-2


def test_gated_prefill_chain_invariants():
    w = inputs.WORKLOADS["tiny"]
    g = inputs.gate_inputs(w, random_bias=True)
    gain, tau = inputs.layer_params(w)
    layers = []
    for li in range(w.n_layers):
        q, k, v = inputs.qkv_template(w, inputs.template_of_layer(w, li))
        layers.append((q, k, v, gain[li], tau[li]))
    r = O.gated_prefill(g["h"], g["w1"], g["b1"], g["w2"], g["b2"], w.doc_begin, w.doc_end,
                        w.k_doc, layers)
    assert r["idx"].size == w.kept
    assert np.array_equal(r["h_kept"], g["h"][r["idx"]])
    for li in range(w.n_layers):
        assert r["outs"][li].shape == (w.kept, w.n_q_heads, w.head_dim)
        assert np.all(np.abs(r["outs"][li]) <= 3.5 + 1e-9)   # convex combination of clipped V
    # the planted spans are what a detector-unit gate prefers
    spans = np.concatenate([np.arange(s0, s0 + w.span_len) for s0 in g["span_starts"]])
    assert np.isin(spans, r["idx"]).mean() > 0.8


def test_golden_tiny_regression():
    """Regression fixture written by tests/golden/make_golden.py (oracle only)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_gated_prefill.json")
    with open(path) as f:
        gold = json.load(f)
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_golden", os.path.join(os.path.dirname(path), "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    now = mod.tiny_fixture()
    assert now["idx"] == gold["idx"]
    for key in ("scores", "out_layer0", "out_layer1"):
        assert np.max(np.abs(np.array(now[key]) - np.array(gold[key]))) < 1e-12, key
