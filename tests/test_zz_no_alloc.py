"""The allocation-free top-K (tg_topk_select_noalloc) against the workspace
entry point (tg_topk_select), through the C ABI.

Two calls in a row on the library's static scratch, the second smaller (the
array keeps the first call's contents, so the second call's result shows that
every word it reads was cleared or written within the call), plus a
one-work-group size that uses no scratch.  Bar: bit-exact indices (integer
work), and the oracle's top-K on the same float32 scores.
"""

import numpy as np
import pytest
import torch

from learned_token_pruning_tg_amd import tg
from oracle import tokengate as O

from gpu_util import dev_f32, say

pytestmark = pytest.mark.gpu


def _scores(rng, n):
    s = rng.standard_normal(n).astype(np.float32)
    # heavy ties and special values, so the tie budget and the key order matter
    s[rng.integers(0, n, n // 8)] = 0.5
    s[rng.integers(0, n, 64)] = -0.0
    s[rng.integers(0, n, 16)] = np.inf
    s[rng.integers(0, n, 16)] = np.nan
    return s


def test_noalloc_topk_matches_workspace_entry_point_twice():
    rng = np.random.default_rng(77)
    # 131072 rows (the long-context workload's size), then a smaller
    # multi-work-group size, then a one-work-group size
    for n, n_doc, k in ((131072, 130816, 8192), (40000, 39000, 3000), (9000, 8800, 700)):
        s = _scores(rng, n)
        sd = dev_f32(s)
        say(f"noalloc topk n={n} doc={n_doc} k={k}")
        want = tg.topk_select(sd, 0, n_doc, k)
        got = tg.topk_select_noalloc(sd, 0, n_doc, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want), n
        assert np.array_equal(got.cpu().numpy(), O.topk_select(s, 0, n_doc, k)), n


def test_noalloc_topk_trivial_budgets():
    rng = np.random.default_rng(78)
    n = 50000
    s = dev_f32(_scores(rng, n))
    for db, de, k in ((100, 49000, 0), (0, 50000, 50000), (0, 50000, 60000), (2000, 2000, 5)):
        say(f"noalloc topk trivial doc=[{db},{de}) k={k}")
        want = tg.topk_select(s, db, de, k)
        got = tg.topk_select_noalloc(s, db, de, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (db, de, k)
