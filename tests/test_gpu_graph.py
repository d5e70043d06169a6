"""The entry points inside a captured HIP graph: every replay (with eager work
and synchronisations between replays) matches the eager results bit for bit.
The benchmark times its decode loop this way."""

import numpy as np
import pytest
import torch

from learned_token_pruning_tg_amd import inputs, tg

from gpu_util import dev_bf16, dev_f32, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    rng = np.random.default_rng(91)
    m, hq, hkv, d = 2304, 16, 8, 128
    r = lambda *shape: dev_bf16(np.clip(rng.standard_normal(shape), -3.5, 3.5).astype(np.float32))
    q, k, v = r(m, hq, d), r(m, hkv, d), r(m, hkv, d)
    scores = dev_f32(rng.standard_normal(30000))
    s, gain, tau = dev_f32(rng.standard_normal(m)), dev_f32(rng.uniform(0.5, 1.5, hq)), \
        dev_f32(rng.uniform(0.8, 1.2, hq))
    out = torch.empty_like(q)
    dout = torch.empty((hq, d), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(tg.kept_count(30000, 0, 29000, 3000), dtype=torch.int32, device="cuda")
    s_kept = torch.empty(idx.numel(), dtype=torch.float32, device="cuda")
    ws = tg.attn_workspace(m, hq, hkv, d)
    dws = tg.decode_workspace(m, hq, hkv, d)
    tws = tg.topk_workspace(30000)

    def work():
        tg.topk_select(scores, 0, 29000, 3000, out=idx, workspace=tws, kept_scores=s_kept)
        tg.gated_attn_fwd(q, k, v, s, gain, tau, out=out, workspace=ws)
        tg.gated_decode(q[-1], k, v, s, gain, tau, out=dout, workspace=dws)

    say("graph capture: top-K + gated attention + decode")
    work()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), dout.clone(), s_kept.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(4):
        idx.zero_(); out.zero_(); dout.zero_(); s_kept.zero_()   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(out, ref[1]) and torch.equal(dout, ref[2]), rep
        assert torch.equal(s_kept, ref[3]) and torch.equal(s_kept, scores[idx.long()]), rep


def test_graph_replays_of_the_backward_match_eager():
    """Forward with lse, then the backward (seven launches, split walks at
    this size), captured together; every replay matches the eager gradients."""
    rng = np.random.default_rng(92)
    m, hq, hkv, d = 2304, 16, 8, 128
    r = lambda *shape: dev_bf16(np.clip(rng.standard_normal(shape), -3.5, 3.5).astype(np.float32))
    q, k, v, do = r(m, hq, d), r(m, hkv, d), r(m, hkv, d), r(m, hq, d)
    s, gain, tau = dev_f32(rng.standard_normal(m)), dev_f32(rng.uniform(0.5, 1.5, hq)), \
        dev_f32(rng.uniform(0.8, 1.2, hq))
    ws = tg.attn_workspace(m, hq, hkv, d)
    bws = tg.attn_bwd_workspace(m, hq, hkv, d)
    out, lse, out32 = tg.gated_attn_fwd_train(q, k, v, s, gain, tau, workspace=ws)
    grads = tg.gated_attn_bwd(q, k, v, s, gain, tau, out32, lse, do, workspace=bws)

    def work():
        tg.gated_attn_fwd_train(q, k, v, s, gain, tau, out=out, lse=lse, out_f32=out32,
                                workspace=ws)
        tg.gated_attn_bwd(q, k, v, s, gain, tau, out32, lse, do, grads=grads, workspace=bws)

    say("graph capture: gated attention forward + backward")
    work()
    torch.cuda.synchronize()
    ref = {nm: t.clone() for nm, t in grads.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(4):
        for t in grads.values():                              # eager work between replays
            t.zero_()
        bws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for nm, t in grads.items():
            assert torch.equal(t, ref[nm]), (rep, nm)
