"""Seeded synthetic workloads for the gated prefill (shared by tests and bench).

This module only draws and lays out inputs: it contains none of the method's
arithmetic (no scoring, selection, compaction or attention).  Both the HIP path
and the CPU oracle receive the exact arrays produced here.

The coverage pages time TokenGate on long-context tasks (RepoBench-P,
2WikiMultihopQA, MultiNews, BioDEX and needle-in-a-haystack, 16k-128k tokens,
Qwen3-1.7B; [KO] "성능 결과").  None of those datasets or weights is available,
so each workload is a stand-in of the same shape: a long document containing a
few short planted "relevant" spans, followed by a short question, with
Qwen3-1.7B-sized tensors (hidden 2048, 16 query / 8 KV heads, head dim 128).

Recipe (numpy, one ``SeedSequence`` child per tensor, seed = 1000 + config
index):
  * residual h ~ N(0, 1) [N, H]; planted spans get h_i += 3 u for a random unit
    vector u;
  * gate weights ~ N(0, 0.02) with b1 = 0, b2 = 0, plus one detector unit
    (W1[0] = u, w2[0] = 1) so that a random gate actually prefers the spans;
  * per upper layer and query head: gain ~ U(0.5, 1.5), temperature
    ~ U(0.8, 1.2);
  * per-layer q/k/v "templates" over all N rows ~ N(0, 1) clipped to +-3.5,
    rotary position encoding (rotate-half, base 1e6) applied to q and k at the
    original positions 0..N-1; three templates are cycled over the layers;
  * bf16 workloads are rounded to bf16 (round-to-nearest-even) here, so that
    both sides see identical values.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int            # total tokens
    n_doc: int        # document tokens, rows [0, n_doc)
    hidden: int       # residual width H
    gate_hidden: int  # gate MLP width H_g
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    k_doc: int        # document budget K
    n_layers: int     # gated layers above the gate
    n_spans: int
    span_len: int
    bf16: bool
    seed: int
    n_templates: int = 3

    @property
    def doc_begin(self) -> int:
        return 0

    @property
    def doc_end(self) -> int:
        return self.n_doc

    @property
    def kept(self) -> int:
        return min(self.k_doc, self.n_doc) + (self.n - self.n_doc)

    def with_budget(self, k_doc: int) -> "Workload":
        return dataclasses.replace(self, k_doc=k_doc, name=f"{self.name}-k{k_doc}")

    def with_n(self, n: int, n_doc: int, k_doc: int) -> "Workload":
        return dataclasses.replace(self, n=n, n_doc=n_doc, k_doc=k_doc,
                                   name=f"{self.name}-n{n}")


_QWEN = dict(hidden=2048, gate_hidden=512, n_q_heads=16, n_kv_heads=8, head_dim=128,
             n_layers=27, n_spans=8, span_len=64, bf16=True)

WORKLOADS = {
    # Tiny: 448 document + 64 question tokens, 256-wide, 4/2 heads of 64.
    "tiny": Workload("tiny", n=512, n_doc=448, hidden=256, gate_hidden=64, n_q_heads=4,
                     n_kv_heads=2, head_dim=64, k_doc=128, n_layers=2, n_spans=2,
                     span_len=16, bf16=False, seed=1000),
    "qwen3-1.7b-16k": Workload("qwen3-1.7b-16k", n=16384, n_doc=16128, k_doc=2048, seed=1001,
                               **_QWEN),
    "qwen3-1.7b-32k": Workload("qwen3-1.7b-32k", n=32768, n_doc=32512, k_doc=4096, seed=1002,
                               **_QWEN),
    "qwen3-1.7b-128k": Workload("qwen3-1.7b-128k", n=131072, n_doc=130816, k_doc=8192,
                                seed=1003, **_QWEN),
    "qwen3-1.7b-64k-sweep": Workload("qwen3-1.7b-64k-sweep", n=65536, n_doc=65280,
                                     k_doc=4096, seed=1004, **_QWEN),
}
SWEEP_BUDGETS = (1024, 4096, 16384, 65536)

# Child-stream slots of the per-workload SeedSequence.
_S_H, _S_SPANS, _S_U, _S_W1, _S_W2, _S_BIAS, _S_LAYER = range(7)
_S_TEMPLATE0 = 8


def _rng(seed: int, slot: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(slot + 1)[slot]))


# ---------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    # uint32 arithmetic wraps only for bit patterns >= 0xFFFF8001, which are
    # NaNs; every NaN is restored from x below.
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = x[nan]
    return out.reshape(x.shape)


def bf16_bits(x_rounded) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(np.asarray(x_rounded, dtype=np.float32))
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _maybe_round(x: np.ndarray, bf16: bool) -> np.ndarray:
    return round_bf16(x) if bf16 else x.astype(np.float32)


# ---------------------------------------------------------------------------
# Rotary position encoding (input preparation: q/k of an upper layer carry the
# tokens' original positions before they reach attention).
# ---------------------------------------------------------------------------

def apply_rope(x: np.ndarray, positions: np.ndarray, base: float = 1.0e6) -> np.ndarray:
    """Rotate-half RoPE on the last dim of x [n, heads, d] at the given positions."""
    n, _, d = x.shape
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang).astype(np.float32)[:, None, :]
    sin = np.sin(ang).astype(np.float32)[:, None, :]
    x = np.asarray(x, dtype=np.float32)
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.empty(x.shape, dtype=np.float32)
    lo, hi = out[..., :half], out[..., half:]
    tmp = np.empty(x1.shape, dtype=np.float32)
    # float32 products, each rounded, then one rounded add (no fused ops)
    np.multiply(x1, cos, out=lo)
    np.multiply(x2, sin, out=tmp)
    lo -= tmp
    np.multiply(x2, cos, out=hi)
    np.multiply(x1, sin, out=tmp)
    hi += tmp
    return out


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

def span_starts(w: Workload) -> np.ndarray:
    """Non-overlapping planted-span starts: one random start per equal slice of
    the document."""
    rng = _rng(w.seed, _S_SPANS)
    seg = w.n_doc // w.n_spans
    assert seg >= w.span_len
    offs = rng.integers(0, seg - w.span_len + 1, size=w.n_spans)
    return (np.arange(w.n_spans) * seg + offs).astype(np.int64)


def gate_inputs(w: Workload, random_bias: bool = False) -> dict:
    """Residual and gate weights.  ``random_bias`` draws nonzero b1/b2 (used by
    unit tests so that the bias terms are exercised)."""
    u = _rng(w.seed, _S_U).standard_normal(w.hidden)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    h = _rng(w.seed, _S_H).standard_normal((w.n, w.hidden), dtype=np.float32)
    starts = span_starts(w)
    for s0 in starts:
        h[s0:s0 + w.span_len] += 3.0 * u[None, :]
    w1 = (0.02 * _rng(w.seed, _S_W1).standard_normal((w.gate_hidden, w.hidden))).astype(np.float32)
    w1[0] = u
    w2 = (0.02 * _rng(w.seed, _S_W2).standard_normal(w.gate_hidden)).astype(np.float32)
    w2[0] = 1.0
    if random_bias:
        rb = _rng(w.seed, _S_BIAS)
        b1 = (0.5 * rb.standard_normal(w.gate_hidden)).astype(np.float32)
        b2 = float(np.float32(rb.standard_normal()))
    else:
        b1 = np.zeros(w.gate_hidden, dtype=np.float32)
        b2 = 0.0
    return dict(h=_maybe_round(h, w.bf16), w1=_maybe_round(w1, w.bf16), b1=b1, w2=w2,
                b2=b2, span_starts=starts, u=u)


def layer_params(w: Workload):
    """Per-upper-layer, per-query-head gain [L, Hq] and temperature [L, Hq]."""
    rng = _rng(w.seed, _S_LAYER)
    gain = rng.uniform(0.5, 1.5, size=(w.n_layers, w.n_q_heads)).astype(np.float32)
    tau = rng.uniform(0.8, 1.2, size=(w.n_layers, w.n_q_heads)).astype(np.float32)
    return gain, tau


def qkv_template(w: Workload, t: int, n: Optional[int] = None):
    """q [N, Hq, d], k/v [N, Hkv, d] for template t, RoPE at positions 0..N-1."""
    n = w.n if n is None else n
    out = []
    for j, heads in enumerate((w.n_q_heads, w.n_kv_heads, w.n_kv_heads)):
        rng = _rng(w.seed, _S_TEMPLATE0 + 3 * t + j)
        x = rng.standard_normal((n, heads, w.head_dim), dtype=np.float32)
        np.clip(x, -3.5, 3.5, out=x)
        if j < 2:
            x = apply_rope(x, np.arange(n))
        out.append(_maybe_round(x, w.bf16))
    return tuple(out)


def template_of_layer(w: Workload, layer: int) -> int:
    return layer % min(w.n_templates, w.n_layers)


# ---------------------------------------------------------------------------
# Hybrid-model (Gated DeltaNet) layer inputs
# ---------------------------------------------------------------------------

# The pages run TokenGate on a hybrid Qwen3.5-2B (Gated DeltaNet layers between
# full-attention layers) but give none of its shapes.  Stand-in: the
# linear-attention layout of the Qwen3-Next family, 16 q/k heads and 32 value
# heads of 128 (value head h reads q/k head h // 2).
GDN_QK_HEADS = 16
GDN_V_HEADS = 32
GDN_HEAD_DIM = 128
_S_GDN0 = 40


def gdn_inputs(seed: int, n: int, n_qk_heads: int = GDN_QK_HEADS, n_v_heads: int = GDN_V_HEADS,
               head_dim: int = GDN_HEAD_DIM, layer: int = 0) -> dict:
    """One Gated DeltaNet layer's inputs over n rows (positions 0..n-1):
    q, k ~ N(0, 1) L2-normalised per head (the layer's own normalisation) and
    rounded to bf16; v ~ N(0, 1) clipped to +-3.5, bf16; per row and value
    head a log decay g = log(a) with a ~ U(0.82, 0.999) and a write strength
    beta = sigmoid(N(0, 1)), both float32."""
    out = {}
    for j, (name, heads) in enumerate((("q", n_qk_heads), ("k", n_qk_heads), ("v", n_v_heads))):
        rng = _rng(seed, _S_GDN0 + 8 * layer + j)
        x = rng.standard_normal((n, heads, head_dim), dtype=np.float32)
        if name == "v":
            np.clip(x, -3.5, 3.5, out=x)
        else:
            x /= np.linalg.norm(x, axis=-1, keepdims=True)
        out[name] = round_bf16(x)
    rng = _rng(seed, _S_GDN0 + 8 * layer + 3)
    out["g"] = np.log(rng.uniform(0.82, 0.999, size=(n, n_v_heads))).astype(np.float32)
    rng = _rng(seed, _S_GDN0 + 8 * layer + 4)
    out["beta"] = (1.0 / (1.0 + np.exp(-rng.standard_normal((n, n_v_heads))))).astype(np.float32)
    return out
