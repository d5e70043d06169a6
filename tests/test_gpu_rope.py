"""GPU parity of the fused gather + QK-norm + RoPE prologue (tg_qk_norm_rope)
against the CPU oracle.  Bar, from the arithmetic: the output is a bf16
rounding (relative error <= 2^-9) of fp32 arithmetic on bf16-exact inputs, and
unlike attention outputs it is not bounded by 4, so the bar is relative: every
element within 2^-8 * max(|ref|, 1) of the float64 oracle, and relative-L2
within 5e-3."""

import numpy as np
import pytest
import torch

from learned_token_pruning_tg_amd import inputs, tg
from oracle import tokengate as O

from gpu_util import dev_bf16, dev_f32, host_bf16, say


def check_rope(got, ref, what):
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    err = np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= 2.0 ** -8, f"{what}: max scaled error {err.max():.3e}"
    assert rel <= 5e-3, f"{what}: rel-L2 {rel:.3e}"

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_src,n,heads,d,norm,gather", [
    (1, 1, 8, 128, True, False), (300, 300, 16, 128, True, False), (300, 77, 8, 64, False, True),
    (16384, 2304, 16, 128, True, True), (131072, 8448, 8, 128, True, True),
    (5000, 5000, 3, 64, True, False), (1000, 333, 32, 128, True, True),
    (300, 50, 80, 128, True, True), (700, 123, 40, 64, False, True)])
def test_qk_norm_rope_vs_oracle(n_src, n, heads, d, norm, gather):
    rng = np.random.default_rng(n + heads + d)
    x = inputs.round_bf16((rng.standard_normal((n_src, heads, d)) * 1.7).astype(np.float32))
    rows = np.sort(rng.choice(n_src, n, replace=False)).astype(np.int32) if gather else None
    pos = (rows if gather else rng.integers(0, 131072, n)).astype(np.int32)
    w = rng.uniform(0.5, 1.5, d).astype(np.float32) if norm else None
    say(f"qk_norm_rope n_src={n_src} n={n} heads={heads} d={d} norm={norm} gather={gather}")
    out = tg.qk_norm_rope(dev_bf16(x), torch.from_numpy(pos).cuda(),
                          rows=None if rows is None else torch.from_numpy(rows).cuda(),
                          norm_weight=None if w is None else dev_f32(w))
    torch.cuda.synchronize()
    ref = O.qk_norm_rope(x if rows is None else x[rows], pos, w)
    check_rope(host_bf16(out), ref, "qk_norm_rope")


def test_qk_norm_rope_in_place_and_skipped_rows():
    rng = np.random.default_rng(5)
    n, heads, d = 200, 4, 128
    x = inputs.round_bf16(rng.standard_normal((n, heads, d)).astype(np.float32))
    pos = rng.integers(0, 70000, n).astype(np.int32)
    xd = dev_bf16(x)
    say("qk_norm_rope in place")
    tg.qk_norm_rope(xd, torch.from_numpy(pos).cuda(), out=xd)
    torch.cuda.synchronize()
    check_rope(host_bf16(xd), O.qk_norm_rope(x, pos, None), "in place")
    # out-of-range rows leave their output rows untouched
    rows = torch.tensor([3, -1, 199, 200], dtype=torch.int32).cuda()
    out = torch.full((4, heads, d), 5.0, dtype=torch.bfloat16).cuda()
    src = dev_bf16(x)
    tg.qk_norm_rope(src, torch.tensor([3, 0, 199, 0], dtype=torch.int32).cuda(), rows=rows, out=out)
    torch.cuda.synchronize()
    o = host_bf16(out)
    assert np.all(o[1] == 5.0) and np.all(o[3] == 5.0)
    check_rope(o[[0, 2]], O.qk_norm_rope(x[[3, 199]], np.array([3, 199]), None), "gathered rows")
