"""Host-side checks of bench.py that need no GPU: the CPU oracle leg's JSON
shape on the tiny workload, the flop count the roofline uses, and the
one-GPU guard."""

import os
import subprocess
import sys

import numpy as np

import bench
from learned_token_pruning_tg_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_tiny_shape():
    w = inputs.WORKLOADS["tiny"]
    r = bench.cpu_baseline(w, bench.HostInputs(w), 5.0)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert f"{w.n_layers} of {w.n_layers} gated-attention layers measured" in r["sample"]
    f = r["full_n_sample"]
    assert f["rows_per_layer"] == 256 and f["layers"] == 2 and len(f["seconds"]) == 2
    assert all(s >= 0 for s in f["seconds"])


def test_attention_flops_count_causal_pairs():
    # 4 d flop per visible (i >= j) pair and query head: QK and PV, 2 flop each
    m, hq, d = 5, 3, 8
    pairs = sum(i + 1 for i in range(m))
    assert bench.attn_flops(m, hq, d) == 4.0 * d * hq * pairs


def test_host_inputs_are_the_generators_arrays():
    w = inputs.WORKLOADS["tiny"]
    host = bench.HostInputs(w)
    g = inputs.gate_inputs(w)
    assert np.array_equal(host.gate["h"], g["h"]) and np.array_equal(host.gate["w1"], g["w1"])
    for t in range(host.n_t):
        for a, b in zip(host.templates[t], inputs.qkv_template(w, t)):
            assert np.array_equal(a, b)


def test_default_workload_is_the_long_context_target():
    w = inputs.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (w.n, w.k_doc, w.kept) == (131072, 8192, 8448)
    for name in bench.OTHER_WORKLOADS:
        assert name in inputs.WORKLOADS


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert p.returncode == 2
    assert "only one GPU" in p.stderr
    assert p.stdout.strip() == ""
