"""CPU oracle for the TokenGate gated-prefill path (test infrastructure only).

This package is the slow, plain reference that the HIP kernels are checked
against. Only the test-suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path never does, and it imports nothing from the
product package.

Sources cited in this package (the method's coverage pages; there is no code):

  [KO]  lucasainews.com, Korean news article on TokenGate (Stanford/Berkeley
        prefill speed-up); sections "작동 방식" (how it works),
        "성능 결과" (results), "사용법과 비용" (usage and cost).
  [FR]  lefilia.fr, "Des chercheurs de Stanford et UC Berkeley présentent
        TokenGate : une attention à portes par token accélère le prefill en
        contexte long jusqu'à 11,3 fois"; lede and body.
  [PT]  miraibroadcast.com, "TokenGate acelera LLMs em até 11x cortando tokens
        irrelevantes"; section "TokenGate “ensina” o modelo a folhear o texto".
  [ABS] fugumt.com, "論文の概要: TokenGate: Adapting LLMs for Fast and
        Memory-Efficient Prefill with Learned Token Pruning"; the English
        abstract.
  [IT]  heraldofai.com, "TokenGate fa leggere ai modelli di intelligenza
        artificiale documenti lunghi fino a 11 volte più velocemente…";
        section "Come funziona".

Pin status of every function is listed in the module docstrings of
``oracle.tokengate`` and ``oracle.gated_deltanet``.
"""

from .tokengate import (  # noqa: F401
    gelu_erf,
    gate_scores,
    score_keys,
    kept_count,
    topk_select,
    compact_rows,
    gated_attention,
    gated_attention_bwd,
    full_attention,
    gated_decode,
    qk_norm_rope,
    gated_prefill,
)
from .gated_deltanet import gated_delta_rule  # noqa: F401
