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


def test_summarize_trace_names_and_averages(tmp_path):
    # a two-kernel trace in rocprofv3's CSV form, one name left mangled as the
    # profiler leaves this library's bf16-parameter kernels
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    hdr = ('"Kind","Kernel_Name","Start_Timestamp","End_Timestamp","Workgroup_Size_X",'
           '"Workgroup_Size_Y","Workgroup_Size_Z","Grid_Size_X","Grid_Size_Y","Grid_Size_Z"\n')
    rows = [
        ("_ZN2tg12_GLOBAL__N_113v_pack_kernelILi128ELb1EEEvPKDF16bPKfS5_S5_iiiPcS6_", 0, 9000, 256, 4224),
        ("_ZN2tg12_GLOBAL__N_113v_pack_kernelILi128ELb1EEEvPKDF16bPKfS5_S5_iiiPcS6_", 0, 11000, 256, 4224),
        ("void tg::(anonymous namespace)::topk_clear_kernel(unsigned int*, int)", 5, 4005, 64, 64),
    ]
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write(hdr)
        for name, t0, t1, wg, grid in rows:
            f.write(f'"KERNEL_DISPATCH","{name}","{t0}","{t1}","{wg}","1","1","{grid}","1","1"\n')
    log = tmp_path / "bench.log"
    log.write_text('noise\n{"roofline": {"avg_launch_ms": 0.3, "achieved": 974.5, "frac": 0.3898}}\n')
    out = tmp_path / "trace.md"
    bench.summarize_trace(str(tmp_path / "trace"), str(log), "tiny", "cmd", str(out))
    text = out.read_text()
    assert "| v_pack_kernel<128, true> | 16 | 2 | 10.00 | 9.00 | 11.00 | 83.33% |" in text
    assert "| topk_clear_kernel | 1 | 1 | 4.00 | 4.00 | 4.00 | 16.67% |" in text
    assert "300.00 us per launch (974.50 TFLOP/s, frac 0.3898)" in text
