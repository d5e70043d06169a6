"""GPU parity of the decode step over the pruned KV cache (tg_gated_decode_fwd)
against the CPU oracle, through the C ABI.

Bars as for attention: outputs within max-abs 1e-2 and relative-L2 5e-3 of the
float64 oracle; the log-sum-exp within 2e-3; repeated calls bit-identical.
"""

import numpy as np
import pytest
import torch

from learned_token_pruning_tg_amd import inputs, tg
from oracle import tokengate as O

from gpu_util import check_attn, dev_bf16, dev_f32, host_bf16, say

pytestmark = pytest.mark.gpu


def _rand_cache(rng, n, hq, hkv, d):
    r = lambda *shape: inputs.round_bf16(np.clip(rng.standard_normal(shape), -3.5, 3.5)
                                         .astype(np.float32))
    q, k, v = r(hq, d), r(n, hkv, d), r(n, hkv, d)
    s = (rng.standard_normal(n) * 1.5).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    return q, k, v, s, gain, tau


@pytest.mark.parametrize("n,hq,hkv,d,bias", [
    (1, 16, 8, 128, True), (2, 4, 2, 64, True), (31, 4, 4, 64, False), (65, 8, 1, 128, True),
    (300, 16, 4, 128, True), (1000, 8, 8, 128, True), (2304, 16, 8, 128, True),
    (5000, 16, 2, 64, True), (8448, 16, 8, 128, True), (16383, 16, 8, 128, False)])
def test_decode_vs_oracle(n, hq, hkv, d, bias):
    rng = np.random.default_rng(n * 3 + hq + d)
    q, k, v, s, gain, tau = _rand_cache(rng, n, hq, hkv, d)
    say(f"decode n={n} hq={hq} hkv={hkv} d={d} bias={bias}")
    args = (dev_f32(s), dev_f32(gain), dev_f32(tau)) if bias else (None, None, None)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, lse = tg.gated_decode(qd, kd, vd, *args, want_lse=True)
    torch.cuda.synchronize()
    if bias:
        ref, ref_lse = O.gated_decode(q, k, v, s, gain, tau, return_lse=True)
    else:
        ref, ref_lse = O.gated_decode(q, k, v, np.zeros(n), np.zeros(hq), np.ones(hq),
                                      return_lse=True)
    check_attn(host_bf16(out), ref, f"decode n={n}")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3
    again = tg.gated_decode(qd, kd, vd, *args)
    torch.cuda.synchronize()
    assert torch.equal(again, out)                                   # deterministic


def test_decode_gate_layer_over_all_rows_128k():
    """The gate layer's decode: plain attention over all 131072 rows."""
    rng = np.random.default_rng(77)
    n, hq, hkv, d = 131072, 16, 8, 128
    q, k, v, _, _, _ = _rand_cache(rng, n, hq, hkv, d)
    say(f"decode plain n={n}")
    out = tg.gated_decode(dev_bf16(q), dev_bf16(k), dev_bf16(v))
    torch.cuda.synchronize()
    ref = O.gated_decode(q, k, v, np.zeros(n), np.zeros(hq), np.ones(hq))
    check_attn(host_bf16(out), ref, "decode plain 128k")


def test_decode_equals_last_row_of_prefill_on_gpu():
    """Appending the new token as the last cached row: the decode output is the
    last row of the prefill attention (both on the GPU, both vs the oracle)."""
    rng = np.random.default_rng(78)
    m, hq, hkv, d = 2304, 16, 8, 128
    q = inputs.round_bf16(np.clip(rng.standard_normal((m, hq, d)), -3.5, 3.5).astype(np.float32))
    _, k, v, s, gain, tau = _rand_cache(rng, m, hq, hkv, d)
    say("decode vs prefill last row m=2304")
    pre = tg.gated_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s), dev_f32(gain),
                            dev_f32(tau))
    dec = tg.gated_decode(dev_bf16(q[-1]), dev_bf16(k), dev_bf16(v), dev_f32(s), dev_f32(gain),
                          dev_f32(tau))
    torch.cuda.synchronize()
    check_attn(host_bf16(dec), host_bf16(pre)[-1], "decode vs prefill last row")


def test_decode_dominant_bias_and_shared_workspace():
    rng = np.random.default_rng(79)
    hq, hkv, d = 16, 8, 128
    ws = tg.decode_workspace(9000, hq, hkv, d)
    for n, j in ((9000, 4321), (700, 0), (64, 63)):
        q, k, v, _, _, tau = _rand_cache(rng, n, hq, hkv, d)
        s = np.zeros(n, np.float32); s[j] = 1.0
        gain = np.full(hq, 90.0, np.float32)
        say(f"decode dominant bias n={n} j={j}")
        out = tg.gated_decode(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(s), dev_f32(gain),
                              dev_f32(tau), workspace=ws)
        torch.cuda.synchronize()
        want = np.repeat(v[j], hq // hkv, axis=0)                    # head h reads KV head h // 2
        assert np.max(np.abs(host_bf16(out) - want)) < 1e-6
