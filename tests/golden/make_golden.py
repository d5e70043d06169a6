"""Write the regression fixtures of tests/golden/ from the CPU oracle only.

The fixture pins the oracle against silent drift: a later change to its
arithmetic must come with a regenerated fixture and a commit message naming
the passage (or the reading of it) that justifies the change.

Run: python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from learned_token_pruning_tg_amd import inputs  # noqa: E402  (seeded inputs only)
from oracle import tokengate as O  # noqa: E402


def tiny_fixture():
    w = inputs.WORKLOADS["tiny"]
    g = inputs.gate_inputs(w, random_bias=True)
    gain, tau = inputs.layer_params(w)
    layers = []
    for li in range(w.n_layers):
        q, k, v = inputs.qkv_template(w, inputs.template_of_layer(w, li))
        layers.append((q, k, v, gain[li], tau[li]))
    r = O.gated_prefill(g["h"], g["w1"], g["b1"], g["w2"], g["b2"], w.doc_begin, w.doc_end,
                        w.k_doc, layers)
    rows = [0, 1, 2, w.kept // 2, w.kept - 2, w.kept - 1]
    return {
        "what": "tiny workload (512 tokens: 448 document + 64 question; K=128), random gate "
                "biases; oracle regression values",
        "cites": "three-stage forward of the lucasainews.com TokenGate article, section "
                 "'작동 방식'; token-gated attention as read in the oracle module docstring",
        "score_rows": list(range(16)),
        "scores": [float(x) for x in r["scores"][:16]],
        "idx": [int(x) for x in r["idx"]],
        "out_rows": rows,
        "out_layer0": [[float(x) for x in r["outs"][0][i].ravel()[:32]] for i in rows],
        "out_layer1": [[float(x) for x in r["outs"][1][i].ravel()[:32]] for i in rows],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_gated_prefill.json"), "w") as f:
        json.dump(tiny_fixture(), f, indent=1)
    print("wrote tiny_gated_prefill.json")
