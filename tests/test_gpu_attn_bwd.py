"""GPU parity of the token-gated attention backward (tg_gated_attn_bwd) against
the float64 oracle, through the C ABI.

The backward consumes the GPU training forward's own fp32 output and
log-sum-exp, as a training step would.  Bars, from the arithmetic: every
gradient is a sum of products whose operands were rounded to bf16 (relative
error <= 2^-9 each: q, k, v, dout are bf16 inputs; P and dS enter the dv, dk
and dq products as bf16), accumulated in fp32, and dq, dk, dv are rounded to
bf16 once more; D = dout.out is formed from the forward's fp32 output.  With random signs the errors add in
quadrature, so a gradient tensor's relative L2 error is a few times 2^-9
(~2e-3); the bar is the attention outputs' relative L2 of 5e-3, and every
element must lie within 2^-5 of the tensor's largest magnitude.

The score, gain and temperature gradients are fp32 sums of fp32 dS terms, and
they cancel (each softmax row of dS sums to zero), so a relative bar does not
fit them.  Their terms' errors come from D = dout.out formed from the forward's
output, which differs from the exact output by well under 2^-8 relative per
element (the forward's fp16 P): |dD_i| <= 2^-8 A_i with
A_i = sum_f |dout_if out_if|, hence |d dS_ij| <= 2^-8 p_ij A_i, and the
summation bound gives |error| <= 2^-8 * the term-magnitude sum
(p_ij (|dp_ij - D_i| + A_i) in place of dS_ij; tests/bwd_bounds.py).  The bar
is 2^-7 times that sum, per element.  The score gradient, the one that reaches
the gate, is also held to relative L2 5e-3 as a whole vector.
"""

import numpy as np
import pytest
import torch

from learned_token_pruning_tg_amd import inputs, tg
from oracle import tokengate as O

from bwd_bounds import term_magnitude_sums
from gpu_util import dev_bf16, dev_f32, host_bf16, say

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
MAX_FRAC = 2.0 ** -5


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    scale = max(np.abs(ref).max(), 1e-30)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    worst = np.abs(got - ref).max() / scale
    print(f"  {what}: rel-L2 {rel:.2e}, max err / max|ref| {worst:.2e}", flush=True)
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    assert worst <= MAX_FRAC, f"{what}: max err {worst:.3e} of the largest magnitude"


def _case(rng, n, hq, hkv, d):
    r = lambda *shape: inputs.round_bf16(np.clip(rng.standard_normal(shape), -3.5, 3.5)
                                         .astype(np.float32))
    q, k, v = r(n, hq, d), r(n, hkv, d), r(n, hkv, d)
    dout = inputs.round_bf16((rng.standard_normal((n, hq, d)) * 0.5).astype(np.float32))
    s = (rng.standard_normal(n) * 1.5).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    return q, k, v, dout, s, gain, tau


def _gpu_bwd(q, k, v, dout, s, gain, tau, workspace=None):
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    sd, gd, td = dev_f32(s), dev_f32(gain), dev_f32(tau)
    _, lse, out32 = tg.gated_attn_fwd_train(qd, kd, vd, sd, gd, td)
    g = tg.gated_attn_bwd(qd, kd, vd, sd, gd, td, out32, lse, dev_bf16(dout), workspace=workspace)
    torch.cuda.synchronize()
    return g, (qd, kd, vd, sd, gd, td, out32, lse)


def _host(g):
    return dict(dq=host_bf16(g["dq"]), dk=host_bf16(g["dk"]), dv=host_bf16(g["dv"]),
                dscore=g["dscore"].cpu().numpy(), dgain=g["dgain"].cpu().numpy(),
                dtau=g["dtau"].cpu().numpy())


def check_sum(got, ref, scale, what, rel_l2=None):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    ratio = np.abs(got - ref) / np.maximum(scale, 1e-30)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"  {what}: max |err| / term-magnitude sum {ratio.max():.2e}, rel-L2 {rel:.2e}",
          flush=True)
    assert ratio.max() <= 2.0 ** -7, f"{what}: error {ratio.max():.3e} of its term-magnitude sum"
    if rel_l2 is not None:
        assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e}"


def _compare(got, ref, bounds, what):
    for name in ("dq", "dk", "dv"):
        check_grad(got[name], ref[name], f"{what} {name}")
    for name in ("dscore", "dgain", "dtau"):
        check_sum(got[name], ref[name], bounds[name], f"{what} {name}",
                  rel_l2=REL_L2 if name == "dscore" else None)


def _oracle(q, k, v, s, gain, tau, dout):
    return (O.gated_attention_bwd(q, k, v, s, gain, tau, dout),
            term_magnitude_sums(q, k, v, s, gain, tau, dout))


@pytest.mark.parametrize("n,hq,hkv,d", [
    (2, 2, 1, 128), (3, 4, 2, 64), (31, 4, 4, 64), (33, 2, 1, 128), (129, 4, 2, 128),
    (300, 16, 8, 128), (700, 8, 2, 64), (1000, 16, 4, 128), (2304, 16, 8, 128),
    (600, 16, 2, 64), (4352, 16, 8, 128)])
def test_attn_bwd_vs_oracle(n, hq, hkv, d):
    rng = np.random.default_rng(1000 + n + hq + d)
    q, k, v, dout, s, gain, tau = _case(rng, n, hq, hkv, d)
    say(f"attn bwd n={n} hq={hq} hkv={hkv} d={d}")
    g, _ = _gpu_bwd(q, k, v, dout, s, gain, tau)
    _compare(_host(g), *_oracle(q, k, v, s, gain, tau, dout), f"n={n}")


def test_attn_bwd_deterministic_and_shared_workspace():
    rng = np.random.default_rng(31)
    hq, hkv, d = 16, 8, 128
    ws = tg.attn_bwd_workspace(3000, hq, hkv, d)
    for n in (3000, 517):
        q, k, v, dout, s, gain, tau = _case(rng, n, hq, hkv, d)
        say(f"attn bwd determinism n={n}")
        g1, args = _gpu_bwd(q, k, v, dout, s, gain, tau, workspace=ws)
        g2 = tg.gated_attn_bwd(*args, dev_bf16(dout), workspace=ws)
        torch.cuda.synchronize()
        for name in g1:
            assert torch.equal(g1[name], g2[name]), name
        if n == 517:
            _compare(_host(g2), *_oracle(q, k, v, s, gain, tau, dout), "n=517 reused ws")


def test_attn_bwd_full_size_one_kv_group():
    """8448 kept rows (the 128k-token workload), 16 query heads over 8 KV heads,
    in the launch configuration of the full problem.  Gains are zero outside
    KV group 0, so the score gradient comes from heads 0 and 1 only and the
    oracle runs on that group alone: dq of heads 0-1, dk/dv of KV head 0, the
    score gradient, and gain/temperature gradients of heads 0-1, all compared
    in full; the other heads' outputs must be finite."""
    rng = np.random.default_rng(32)
    n, hq, hkv, d = 8448, 16, 8, 128
    q, k, v, dout, s, gain, tau = _case(rng, n, hq, hkv, d)
    gain[2:] = 0.0
    say(f"attn bwd full size n={n}")
    got = _host(_gpu_bwd(q, k, v, dout, s, gain, tau)[0])
    for name in got:
        assert np.all(np.isfinite(got[name])), name
    ref = _oracle(q[:, :2], k[:, :1], v[:, :1], s, gain[:2], tau[:2], dout[:, :2])
    sub = dict(dq=got["dq"][:, :2], dk=got["dk"][:, :1], dv=got["dv"][:, :1],
               dscore=got["dscore"], dgain=got["dgain"][:2], dtau=got["dtau"][:2])
    _compare(sub, *ref, "n=8448 group 0")


def test_attn_bwd_single_row():
    """One row: its softmax is 1 on its own key, so dS = 0 (up to the rounding
    of dout.v against dout.out), dq = dk = 0, dv = dout, and the score, gain and
    temperature gradients vanish."""
    rng = np.random.default_rng(34)
    q, k, v, dout, s, gain, tau = _case(rng, 1, 16, 8, 128)
    say("attn bwd n=1")
    got = _host(_gpu_bwd(q, k, v, dout, s, gain, tau)[0])
    # each KV head's dv is the sum of its two query heads' dout, rounded to bf16
    want = inputs.round_bf16(dout[0].reshape(8, 2, 128).sum(axis=1, dtype=np.float32))
    assert np.array_equal(got["dv"][0], want)
    for name in ("dq", "dk", "dscore", "dgain", "dtau"):
        assert np.max(np.abs(got[name])) <= 1e-4, name
