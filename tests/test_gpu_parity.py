"""GPU parity: every HIP entry point against the CPU oracle, through the C ABI.

Bars: top-K indices and compacted bytes bit-exact (top-K is fed the GPU's own
float32 scores, so both sides decide on identical values); scores within 1e-3
relative; attention outputs within max-abs 1e-2 and relative-L2 5e-3 of the
float64 oracle.  The fp32 tiny workload runs on bf16-rounded copies, and the
oracle is given the same rounded values.
"""

import numpy as np
import pytest
import torch

from learned_token_pruning_tg_amd import inputs, tg
from oracle import tokengate as O

from gpu_util import (check_attn, check_scores, dev_bf16, dev_f32, host_bf16, say)

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _sample_rows(m, rng, extra=(), n_random=40):
    base = {0, 1, 2, m // 2, m - 2, m - 1, 63, 64, 127, 128, 129, 255, 256}
    base |= set(int(x) for x in extra)
    base |= set(int(x) for x in rng.integers(0, m, size=n_random))
    return np.array(sorted(r for r in base if 0 <= r < m), dtype=np.int64)


# --------------------------------------------------------------------------- gate

@pytest.mark.parametrize("random_bias", [False, True])
def test_gate_tiny(random_bias):
    w = W["tiny"]
    g = inputs.gate_inputs(w, random_bias=random_bias)
    h = inputs.round_bf16(g["h"]); w1 = inputs.round_bf16(g["w1"])
    say(f"gate tiny random_bias={random_bias}")
    s = tg.gate_score(dev_bf16(h), dev_bf16(w1), dev_f32(g["b1"]), dev_f32(g["w2"]), g["b2"])
    torch.cuda.synchronize()
    check_scores(s.cpu().numpy(), O.gate_scores(h, w1, g["b1"], g["w2"], g["b2"]), "gate tiny")


@pytest.mark.parametrize("n,hidden,hg,ld", [(1000, 256, 96, 264), (1, 64, 32, 64),
                                           (130, 512, 512, 520), (64, 128, 64, 128),
                                           (333, 192, 200, 200), (77, 64, 1, 64),
                                           (300, 128, 384, 136), (66000, 64, 256, 64),
                                           (40000, 64, 300, 72), (33000, 128, 512, 128),
                                           (33023, 192, 257, 200), (49999, 64, 450, 72)])
def test_gate_ragged_strided(n, hidden, hg, ld):
    rng = np.random.default_rng(n + hg)
    base = inputs.round_bf16(rng.standard_normal((n, ld)).astype(np.float32))
    w1 = inputs.round_bf16((rng.standard_normal((hg, hidden)) * 0.08).astype(np.float32))
    b1 = (rng.standard_normal(hg) * 0.5).astype(np.float32)
    w2 = rng.standard_normal(hg).astype(np.float32)
    say(f"gate ragged n={n} hidden={hidden} hg={hg} ld={ld}")
    hd = dev_bf16(base)[:, :hidden]
    s = tg.gate_score(hd, dev_bf16(w1), dev_f32(b1), dev_f32(w2), -0.25)
    torch.cuda.synchronize()
    check_scores(s.cpu().numpy(), O.gate_scores(base[:, :hidden], w1, b1, w2, -0.25), "gate ragged")


@pytest.mark.parametrize("n", [16384, 65536 + 37])
def test_gate_qwen_shapes_and_determinism(n):
    w = W["qwen3-1.7b-16k"]
    wk = w.with_n(n, n - 256, 2048)
    g = inputs.gate_inputs(wk, random_bias=True)
    say(f"gate qwen n={n}")
    hd = dev_bf16(g["h"]); w1d = dev_bf16(g["w1"])
    s1 = tg.gate_score(hd, w1d, dev_f32(g["b1"]), dev_f32(g["w2"]), g["b2"])
    # into a buffer that holds NaNs: every score is written afresh
    s2 = tg.gate_score(hd, w1d, dev_f32(g["b1"]), dev_f32(g["w2"]), g["b2"],
                       out=torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    a, b = s1.cpu().numpy(), s2.cpu().numpy()
    assert a.tobytes() == b.tobytes()                     # deterministic
    # every row: work-groups start their K loops at staggered offsets, so each
    # row's sum order depends on its work-group
    ref = O.gate_scores(g["h"], g["w1"], g["b1"], g["w2"], g["b2"])
    check_scores(a, ref, f"gate qwen n={n}")


# --------------------------------------------------------------------------- top-K

def _topk_gpu(s32, db, de, k):
    """Indices from tg_topk_select, checked equal to those of
    tg_topk_select_scores, whose gathered scores must be s32[idx] bit for bit
    (NaN payloads and signed zeros included)."""
    say(f"topk n={s32.size} doc=[{db},{de}) k={k}")
    sd = dev_f32(s32)
    out = tg.topk_select(sd, db, de, k)
    m = tg.kept_count(s32.size, db, de, k)
    ks = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda")
    out2 = tg.topk_select(sd, db, de, k, kept_scores=ks)
    torch.cuda.synchronize()
    idx = out.cpu().numpy()
    assert np.array_equal(out2.cpu().numpy(), idx)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), s32[idx].view(np.uint32))
    return idx


def test_topk_tiny_on_gpu_scores():
    w = W["tiny"]
    g = inputs.gate_inputs(w)
    s = tg.gate_score(dev_bf16(g["h"]), dev_bf16(g["w1"]), dev_f32(g["b1"]), dev_f32(g["w2"]),
                      g["b2"])
    s32 = s.cpu().numpy()
    for k in (0, 1, 17, 128, 447, 448, 1000):
        assert np.array_equal(_topk_gpu(s32, 0, w.n_doc, k), O.topk_select(s32, 0, w.n_doc, k))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_special_values_and_ties(seed):
    rng = np.random.default_rng(seed)
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1e-45, -1e-45, 0.5, -2.0, 3.0],
                    dtype=np.float32)
    s32 = rng.choice(pool, size=5000).astype(np.float32)
    for db, de in ((100, 4900), (0, 5000), (2500, 2500), (0, 1)):
        for k in (0, 1, 2, 999, 1000, de - db - 1, de - db, 6000):
            if k < 0:
                continue
            assert np.array_equal(_topk_gpu(s32, db, de, k), O.topk_select(s32, db, de, k)), \
                (seed, db, de, k)


@pytest.mark.parametrize("n,db,de,k", [(131072, 0, 130816, 8192), (131072, 1000, 130000, 8192),
                                       (65536, 0, 65280, 1024), (65536, 0, 65280, 16384),
                                       (16384, 0, 16128, 2048), (70001, 3, 69999, 33333),
                                       (16385, 1, 16384, 8000), (24576, 0, 24320, 4096),
                                       (20000, 100, 19900, 1),
                                       (2 * 1024 * 2048 + 4099, 517, 2 * 1024 * 2048, 300007)])
def test_topk_large_quantised(n, db, de, k):
    rng = np.random.default_rng(n + k)
    s32 = (np.round(rng.standard_normal(n) * 64) / 64).astype(np.float32)   # many exact ties
    a = _topk_gpu(s32, db, de, k)
    assert np.array_equal(a, O.topk_select(s32, db, de, k))
    assert np.array_equal(a, _topk_gpu(s32, db, de, k))                     # deterministic


def test_topk_long_special_values_and_shared_workspace():
    # The multi-work-group path on NaN/inf/signed-zero/tie-heavy scores, its two
    # trivial budgets (0 and all), and one workspace reused across calls of
    # different lengths (nothing may carry over between calls).
    rng = np.random.default_rng(7)
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1e-45, -1e-45, 0.5, -2.0, 3.0],
                    dtype=np.float32)
    ws = tg.topk_workspace(300000)
    for n, db, de in ((300000, 17, 299990), (120001, 0, 120001), (40000, 5000, 35000)):
        s32 = rng.choice(pool, size=n).astype(np.float32)
        sd = dev_f32(s32)
        for k in (0, 1, 12345, de - db - 1, de - db, de - db + 7):
            say(f"topk long n={n} doc=[{db},{de}) k={k}")
            out = tg.topk_select(sd, db, de, k, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), O.topk_select(s32, db, de, k)), (n, db, de, k)


def test_topk_special_values_above_single_group_limit():
    # Just above the one-work-group limit (16384 rows): the multi-work-group
    # path with few row ranges, on NaN/inf/signed-zero/tie-heavy scores.
    rng = np.random.default_rng(11)
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1e-45, -1e-45, 0.5, -2.0, 3.0],
                    dtype=np.float32)
    s32 = rng.choice(pool, size=24000).astype(np.float32)
    for db, de in ((0, 24000), (16000, 17000), (300, 23999)):
        for k in (0, 1, 2399, 2400, de - db - 1, de - db):
            assert np.array_equal(_topk_gpu(s32, db, de, k), O.topk_select(s32, db, de, k)), \
                (db, de, k)


def test_topk_all_equal():
    s32 = np.full(9000, 1.25, dtype=np.float32)
    assert np.array_equal(_topk_gpu(s32, 10, 8990, 4000), O.topk_select(s32, 10, 8990, 4000))


# --------------------------------------------------------------------------- compaction

# rows of 4096 and 2048 B (16-byte units, blocks of 8 and 16 rows), 1204 B
# (4-byte units, blocks of 6), 1500 B (byte units, one row per block), 40000 B
# (past a block's 32 KiB: the flattened path) and narrow rows
@pytest.mark.parametrize("row_shape,dtype", [((2048,), torch.bfloat16), ((), torch.float32),
                                             ((3,), torch.int16), ((3,), torch.float32),
                                             ((8, 128), torch.bfloat16), ((5,), torch.uint8),
                                             ((301,), torch.float32), ((1500,), torch.uint8),
                                             ((20000,), torch.bfloat16)])
def test_compact_bytewise(row_shape, dtype):
    rng = np.random.default_rng(len(row_shape))
    rows = 3000
    src = torch.from_numpy(rng.integers(0, 255, size=(rows,) + row_shape).astype(np.uint8))
    if dtype != torch.uint8:
        nbytes = int(np.prod(row_shape or (1,))) * torch.empty((), dtype=dtype).element_size()
        raw = rng.integers(0, 256, size=(rows, nbytes), dtype=np.uint8)
        src = torch.from_numpy(raw).view(dtype).reshape((rows,) + row_shape)
    idx = np.sort(rng.choice(rows, size=777, replace=False)).astype(np.int32)
    say(f"compact row_shape={row_shape} dtype={dtype}")
    out = tg.compact(torch.from_numpy(idx).cuda(), src.cuda())
    torch.cuda.synchronize()
    got = out.cpu().contiguous().view(torch.uint8).numpy().reshape(777, -1)
    ref = src[torch.from_numpy(idx).long()].contiguous().view(torch.uint8).numpy().reshape(777, -1)
    assert got.tobytes() == ref.tobytes()


def test_compact_strided_and_out_of_range_indices():
    rng = np.random.default_rng(9)
    big = torch.from_numpy(rng.standard_normal((500, 40)).astype(np.float32)).cuda()
    src = big[:, 4:36]                       # row stride 160 B, rows of 128 B
    assert not src.is_contiguous() and src[0].is_contiguous()
    idx = torch.tensor([5, -1, 499, 500, 0, 7], dtype=torch.int32).cuda()
    out = torch.full((6, 32), -7.0, device="cuda")
    say("compact strided + invalid idx")
    tg.compact(idx, src, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy(); s = src.cpu().numpy()
    for r, i in enumerate([5, -1, 499, 500, 0, 7]):
        if 0 <= i < 500:
            assert np.array_equal(o[r], s[i])
        else:
            assert np.all(o[r] == -7.0)      # skipped row left unwritten


# --------------------------------------------------------------------------- attention

def _rand_attn(rng, m, hq, hkv, d):
    q = inputs.round_bf16(np.clip(rng.standard_normal((m, hq, d)), -3.5, 3.5).astype(np.float32))
    k = inputs.round_bf16(np.clip(rng.standard_normal((m, hkv, d)), -3.5, 3.5).astype(np.float32))
    v = inputs.round_bf16(np.clip(rng.standard_normal((m, hkv, d)), -3.5, 3.5).astype(np.float32))
    s = (rng.standard_normal(m) * 1.5).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    return q, k, v, s, gain, tau


@pytest.mark.parametrize("m,hq,hkv,d", [(1, 4, 2, 64), (2, 4, 2, 128), (63, 4, 2, 64),
                                        (64, 4, 4, 128), (65, 8, 1, 128), (127, 4, 2, 64),
                                        (129, 16, 8, 128), (200, 4, 2, 64), (515, 16, 8, 128),
                                        (1000, 2, 1, 128), (2304, 16, 8, 128), (3000, 1, 1, 64),
                                        (5000, 2, 1, 128), (1800, 8, 1, 128), (2600, 8, 4, 64),
                                        (2000, 16, 8, 128), (3000, 16, 8, 128)])
def test_gated_attention_ragged(m, hq, hkv, d):
    rng = np.random.default_rng(m * 7 + d)
    q, k, v, s, gain, tau = _rand_attn(rng, m, hq, hkv, d)
    say(f"gated attn m={m} hq={hq} hkv={hkv} d={d}")
    out, lse = tg.gated_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s), dev_f32(gain),
                                 dev_f32(tau), want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.gated_attention(q, k, v, s, gain, tau, return_lse=True)
    check_attn(host_bf16(out), ref, f"gated m={m} d={d}")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3
    # a second call gives the same bits (split key ranges merge in a fixed order)
    again = tg.gated_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s), dev_f32(gain),
                              dev_f32(tau))
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    # first row sees only key 0: output is v_0 of its KV group, exactly
    g = hq // hkv
    got0 = host_bf16(out)[0]
    for h in range(hq):
        assert np.array_equal(got0[h], v[0, h // g])


@pytest.mark.parametrize("m,hq,hkv", [(200, 4, 2), (2304, 16, 8)])
def test_gated_attention_dominant_bias(m, hq, hkv):
    # one key with a huge biased logit: every row that sees it returns its v
    # (the softmax collapses onto it); exact up to the fp16 step of v in the
    # P.V product, which only bites below fp16's normal range (|v| < 6.1e-5,
    # error < 6e-8).  Rows before it are ordinary attention.
    rng = np.random.default_rng(m + 5)
    q, k, v, _, _, tau = _rand_attn(rng, m, hq, hkv, 128)
    j = m // 3
    s = np.zeros(m, np.float32); s[j] = 1.0
    gain = np.full(hq, 80.0, np.float32)
    say(f"dominant bias m={m} hq={hq}")
    out = host_bf16(tg.gated_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s),
                                      dev_f32(gain), dev_f32(tau)))
    torch.cuda.synchronize()
    g = hq // hkv
    for h in range(hq):
        assert np.max(np.abs(out[j:, h] - v[j, h // g][None, :])) <= 1e-6
    rows = np.arange(0, j)
    ref = O.gated_attention(q, k, v, s, gain, tau, rows=rows)
    check_attn(out[rows], ref, "rows before the dominant key")


@pytest.mark.parametrize("m,hq,hkv,d", [(2304, 16, 8, 128), (1500, 4, 2, 64)])
def test_full_attention_split_keys(m, hq, hkv, d):
    # unbiased kernel on a short prefix: its longest query tiles are split
    # along the keys and merged
    rng = np.random.default_rng(m + d)
    q, k, v, _, _, _ = _rand_attn(rng, m, hq, hkv, d)
    say(f"full attn split m={m} hq={hq} d={d}")
    out, lse = tg.full_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.full_attention(q, k, v, return_lse=True)
    check_attn(host_bf16(out), ref, f"full m={m} d={d}")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3


@pytest.mark.parametrize("m,d", [(300, 128), (777, 64)])
def test_no_gain_unit_temperature_equals_full(m, d):
    rng = np.random.default_rng(m)
    q, k, v, s, _, _ = _rand_attn(rng, m, 4, 2, d)
    say(f"gated(g=0,tau=1) vs full m={m} d={d}")
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    a = tg.gated_attn_fwd(qd, kd, vd, dev_f32(s), dev_f32(np.zeros(4)), dev_f32(np.ones(4)))
    b, lse = tg.full_attn_fwd(qd, kd, vd, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref, ref_lse = O.full_attention(q, k, v, return_lse=True)
    check_attn(host_bf16(b), ref, "full")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3


def test_tiny_workload_chain_all_layers():
    w = W["tiny"]
    g = inputs.gate_inputs(w, random_bias=True)
    h = inputs.round_bf16(g["h"]); w1 = inputs.round_bf16(g["w1"])
    gain, tau = inputs.layer_params(w)
    say("tiny chain")
    hd = dev_bf16(h)
    s_d = tg.gate_score(hd, dev_bf16(w1), dev_f32(g["b1"]), dev_f32(g["w2"]), g["b2"])
    idx_d = tg.topk_select(s_d, w.doc_begin, w.doc_end, w.k_doc)
    h_kept = tg.compact(idx_d, hd)
    s_kept = tg.compact(idx_d, s_d)
    torch.cuda.synchronize()
    s32 = s_d.cpu().numpy(); idx = idx_d.cpu().numpy()
    check_scores(s32, O.gate_scores(h, w1, g["b1"], g["w2"], g["b2"]), "tiny scores")
    assert np.array_equal(idx, O.topk_select(s32, w.doc_begin, w.doc_end, w.k_doc))
    assert np.array_equal(host_bf16(h_kept), h[idx])
    assert np.array_equal(s_kept.cpu().numpy(), s32[idx])
    for li in range(w.n_layers):
        q, k, v = (inputs.round_bf16(x) for x in inputs.qkv_template(w, inputs.template_of_layer(w, li)))
        qk, kk, vk = (tg.compact(idx_d, dev_bf16(x)) for x in (q, k, v))
        out = tg.gated_attn_fwd(qk, kk, vk, s_kept, dev_f32(gain[li]), dev_f32(tau[li]))
        torch.cuda.synchronize()
        ref = O.gated_attention(q[idx], k[idx], v[idx], s32[idx], gain[li], tau[li])
        check_attn(host_bf16(out), ref, f"tiny layer {li}")


# --------------------------------------------------------------------------- full-size chains

def _chain(w, layers, n_rows=None, full_rows=32):
    """Gate -> top-K -> compaction -> gated attention at full size, checked in
    full (every gate score, indices, compacted bytes; every gated-attention
    output and LSE when n_rows is None) or on sampled rows (attention when
    n_rows is given; the full-N baseline)."""
    rng = np.random.default_rng(w.seed)
    g = inputs.gate_inputs(w)
    gain, tau = inputs.layer_params(w)
    say(f"chain {w.name}: gate/top-K/compact")
    hd = dev_bf16(g["h"])
    s_d = tg.gate_score(hd, dev_bf16(g["w1"]), dev_f32(g["b1"]), dev_f32(g["w2"]), g["b2"])
    # the step's own launch sequence: top-K also gathers s', then h is compacted
    s_kept = torch.empty(w.kept, dtype=torch.float32, device="cuda")
    idx_d = tg.topk_select(s_d, w.doc_begin, w.doc_end, w.k_doc, kept_scores=s_kept)
    h_kept = tg.compact(idx_d, hd)
    torch.cuda.synchronize()
    s32 = s_d.cpu().numpy(); idx = idx_d.cpu().numpy()
    check_scores(s32, O.gate_scores(g["h"], g["w1"], g["b1"], g["w2"], g["b2"]),
                 f"{w.name} scores")
    assert idx.size == w.kept
    assert np.array_equal(idx, O.topk_select(s32, w.doc_begin, w.doc_end, w.k_doc))
    assert host_bf16(h_kept).tobytes() == g["h"][idx].tobytes()
    assert np.array_equal(s_kept.cpu().numpy(), s32[idx])
    del hd, h_kept
    kept_doc = min(w.k_doc, w.n_doc)
    for li in layers:
        t = inputs.template_of_layer(w, li)
        q, k, v = inputs.qkv_template(w, t)
        qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
        say(f"chain {w.name}: gated attention layer {li} (M={w.kept})")
        qk, kk, vk = (tg.compact(idx_d, x) for x in (qd, kd, vd))
        out, lse = tg.gated_attn_fwd(qk, kk, vk, s_kept, dev_f32(gain[li]), dev_f32(tau[li]),
                                     want_lse=True)
        torch.cuda.synchronize()
        if n_rows is None:
            r = np.arange(w.kept)
        else:
            r = _sample_rows(w.kept, rng, extra=(kept_doc - 1, kept_doc, kept_doc + 1),
                             n_random=n_rows)
        ref, ref_lse = O.gated_attention(q[idx], k[idx], v[idx], s32[idx], gain[li], tau[li],
                                         rows=r, return_lse=True)
        check_attn(host_bf16(out)[r], ref, f"{w.name} layer {li}")
        assert np.max(np.abs(lse.cpu().numpy()[:, r] - ref_lse)) < 2e-3
        if li == layers[0] and full_rows:
            say(f"chain {w.name}: full attention (N={w.n})")
            fo = tg.full_attn_fwd(qd, kd, vd)
            torch.cuda.synchronize()
            fr = _sample_rows(w.n, rng, extra=(w.n_doc - 1, w.n_doc), n_random=full_rows)
            check_attn(host_bf16(fo)[fr], O.full_attention(q, k, v, rows=fr), f"{w.name} full")
            del fo
        del qd, kd, vd, qk, kk, vk, out


def test_chain_qwen_16k():
    _chain(W["qwen3-1.7b-16k"], layers=[0, 26])


def test_chain_qwen_32k():
    _chain(W["qwen3-1.7b-32k"], layers=[0, 26])


def test_chain_qwen_128k():
    _chain(W["qwen3-1.7b-128k"], layers=[0, 26], full_rows=16)


@pytest.mark.parametrize("k_doc", inputs.SWEEP_BUDGETS)
def test_chain_qwen_64k_budget_sweep(k_doc):
    w = W["qwen3-1.7b-64k-sweep"].with_budget(k_doc)
    _chain(w, layers=[0], n_rows=24, full_rows=0)


def test_budget_n_with_no_gain_is_full_prefill_64k():
    """K = N, gain 0, temperature 1: the gated path is the plain full prefill."""
    w = W["qwen3-1.7b-64k-sweep"]
    q, k, v = inputs.qkv_template(w, 0)
    say("64k K=N equivalence")
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    s = dev_f32(np.random.default_rng(3).standard_normal(w.n))
    a = tg.gated_attn_fwd(qd, kd, vd, s, dev_f32(np.zeros(16)), dev_f32(np.ones(16)))
    b = tg.full_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
