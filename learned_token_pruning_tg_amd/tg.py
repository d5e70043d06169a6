"""Thin Python binding of libtg (the C ABI declared in include/tg.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch is used for device
memory and the current stream); outputs are allocated with torch when not
given.  A missing library raises at first use -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtg.so")
_lib = None

TG_OK = 0
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

_SIGNATURES = {
    "tg_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "tg_last_error": (ctypes.c_char_p, []),
    "tg_kept_count": (_I64, [_I64, _I64, _I64, _I64]),
    "tg_gate_score": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, ctypes.c_float, _I32, _P, _P]),
    "tg_topk_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "tg_topk_select": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "tg_topk_select_noalloc": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _P, _P]),
    "tg_topk_select_scores": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "tg_compact": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "tg_attn_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I32, _I32]),
    "tg_gated_attn_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                         _P, ctypes.c_size_t, _P]),
    "tg_gated_attn_fwd_train": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P,
                                               _P, _P, _P, ctypes.c_size_t, _P]),
    "tg_full_attn_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "tg_attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I32, _I32]),
    "tg_gated_attn_bwd": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "tg_decode_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I32, _I32]),
    "tg_gdn_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I32, _I32]),
    "tg_gdn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, ctypes.c_float, _P,
                                  _P, _P, _P, ctypes.c_size_t, _P]),
    "tg_qk_norm_rope": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I32, _I32, _P, ctypes.c_float,
                                       ctypes.c_double, _P, _P]),
    "tg_gated_decode_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P,
                                           _P, _P, ctypes.c_size_t, _P]),
}


class TGError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_str(status)} ({status}): {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libtg.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m learned_token_pruning_tg_amd.build`")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def lib_path() -> str:
    return _LIB_PATH


def status_str(status: int) -> str:
    return lib().tg_status_str(status).decode()


def last_error() -> str:
    return lib().tg_last_error().decode()


def _check(status: int) -> None:
    if status != TG_OK:
        raise TGError(status, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, contiguous: bool = True) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------

def kept_count(n: int, doc_begin: int, doc_end: int, k_doc: int) -> int:
    m = lib().tg_kept_count(n, doc_begin, doc_end, k_doc)
    if m < 0:
        raise ValueError(f"invalid segment/budget: n={n} doc=[{doc_begin},{doc_end}) k={k_doc}")
    return m


def k_doc_for_budget(n: int, doc_begin: int, doc_end: int, max_kept_prefill_tokens: int) -> int:
    """Document budget for a budget on all kept prefill tokens (lucasainews.com
    article, "사용법과 비용": the caller marks the prunable document and passes a
    kept-token budget).  Rows outside the document are always kept, so the
    document gets what is left of the budget: max(0, B - (n - N_doc)); the
    kept count is then B, clamped to [n - N_doc, n]."""
    if not 0 <= doc_begin <= doc_end <= n or max_kept_prefill_tokens < 0:
        raise ValueError(f"invalid segment/budget: n={n} doc=[{doc_begin},{doc_end}) "
                         f"B={max_kept_prefill_tokens}")
    return max(0, max_kept_prefill_tokens - (n - (doc_end - doc_begin)))


def gate_score(h: torch.Tensor, w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: float,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """scores[i] = w2 . GELU(W1 h[i] + b1) + b2.  h [n, H] bf16 (row stride may
    exceed H), w1 [Hg, H] bf16, b1/w2 [Hg] fp32 -> [n] fp32."""
    _need(h, "h", torch.bfloat16, contiguous=False)
    if h.dim() != 2 or h.stride(1) != 1:
        raise ValueError("h must be [n, H] with unit column stride")
    _need(w1, "w1", torch.bfloat16); _need(b1, "b1", torch.float32); _need(w2, "w2", torch.float32)
    n, hidden = h.shape
    hg = w1.shape[0]
    if w1.shape != (hg, hidden) or b1.shape != (hg,) or w2.shape != (hg,):
        raise ValueError("gate weight shapes do not match h")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=h.device)
    _need(out, "out", torch.float32)
    _check(lib().tg_gate_score(_ptr(h), n, h.stride(0), hidden, _ptr(w1), _ptr(b1), _ptr(w2),
                               float(b2), hg, _ptr(out), _stream(stream)))
    return out


def topk_workspace_bytes(n: int) -> int:
    return int(lib().tg_topk_workspace_bytes(n))


def topk_workspace(n: int, device="cuda") -> torch.Tensor:
    """A device buffer large enough for one top-K call over n scores."""
    return torch.empty(max(topk_workspace_bytes(n), 16), dtype=torch.uint8, device=device)


def topk_select(scores: torch.Tensor, doc_begin: int, doc_end: int, k_doc: int,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None, kept_scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Kept row indices (ascending int32) of a top-K over the document rows
    [doc_begin, doc_end) with every other row kept.
    ``workspace``: scratch from topk_workspace() (allocated per call if None).
    ``kept_scores``: if given ([M] fp32), also filled with scores[idx] in the
    same pass (tg_topk_select_scores)."""
    _need(scores, "scores", torch.float32)
    n = scores.numel()
    m = kept_count(n, doc_begin, doc_end, k_doc)
    if out is None:
        out = torch.empty(m, dtype=torch.int32, device=scores.device)
    _need(out, "out", torch.int32)
    if out.numel() < m:
        raise ValueError(f"out holds {out.numel()} < {m} indices")
    if workspace is None:
        workspace = topk_workspace(n, scores.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if kept_scores is None:
        _check(lib().tg_topk_select(_ptr(scores), n, doc_begin, doc_end, k_doc, _ptr(out),
                                    _ptr(workspace), ws_bytes, _stream(stream)))
    else:
        _need(kept_scores, "kept_scores", torch.float32)
        if kept_scores.numel() < m:
            raise ValueError(f"kept_scores holds {kept_scores.numel()} < {m} scores")
        _check(lib().tg_topk_select_scores(_ptr(scores), n, doc_begin, doc_end, k_doc, _ptr(out),
                                           _ptr(kept_scores), _ptr(workspace), ws_bytes,
                                           _stream(stream)))
    return out


def topk_select_noalloc(scores: torch.Tensor, doc_begin: int, doc_end: int, k_doc: int,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """topk_select with the library's static per-GPU scratch instead of a
    workspace (no device allocation inside the call; calls that overlap on
    one GPU race).  Returns the kept indices [M] int32, ascending."""
    _need(scores, "scores", torch.float32)
    n = scores.shape[0]
    m = kept_count(n, doc_begin, doc_end, k_doc)
    if m < 0:
        raise ValueError("invalid document range or budget")
    if out is None:
        out = torch.empty(m, dtype=torch.int32, device=scores.device)
    _need(out, "out", torch.int32)
    if out.shape != (m,):
        raise ValueError(f"out must hold {m} indices")
    _check(lib().tg_topk_select_noalloc(_ptr(scores), n, doc_begin, doc_end, k_doc, _ptr(out),
                                        _stream(stream)))
    return out


def compact(idx: torch.Tensor, src: torch.Tensor, out: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """out[i] = src[idx[i]] over the leading dimension (rows of any dtype)."""
    _need(idx, "idx", torch.int32)
    if not src.is_cuda:
        raise ValueError("src must be a GPU tensor")
    rows = src.shape[0]
    row_shape = tuple(src.shape[1:])
    row_elems = 1
    for s in row_shape:
        row_elems *= s
    es = src.element_size()
    if src.dim() > 1 and not src[0].is_contiguous():
        raise ValueError("src rows must be contiguous")
    n_kept = idx.numel()
    if out is None:
        out = torch.empty((n_kept,) + row_shape, dtype=src.dtype, device=src.device)
    if out.dtype != src.dtype or tuple(out.shape[1:]) != row_shape or out.shape[0] < n_kept:
        raise ValueError("out does not match src rows")
    src_stride = src.stride(0) * es if src.dim() > 0 and rows > 0 else row_elems * es
    dst_stride = out.stride(0) * es if n_kept > 0 else row_elems * es
    _check(lib().tg_compact(_ptr(idx), n_kept, _ptr(src), rows, src_stride, row_elems * es,
                            _ptr(out), dst_stride, _stream(stream)))
    return out


def attn_workspace_bytes(n: int, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    return int(lib().tg_attn_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim))


def attn_workspace(n: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                   device="cuda") -> torch.Tensor:
    """A device buffer large enough for one attention call over n rows."""
    return torch.empty(max(attn_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim), 16),
                       dtype=torch.uint8, device=device)


def _workspace(ws, n, hq, hkv, d, device):
    if ws is None:
        ws = attn_workspace(n, hq, hkv, d, device)
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws, ws.numel() * ws.element_size()


def _attn_out(q, out, lse, want_lse):
    n, hq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16)
    if want_lse and lse is None:
        lse = torch.empty((hq, n), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    return out, lse


def gated_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: torch.Tensor,
                   gain: torch.Tensor, tau: torch.Tensor, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Token-gated causal GQA attention over the kept rows.
    q [M, Hq, d], k/v [M, Hkv, d] bf16; key_score [M], gain/tau [Hq] fp32.
    ``workspace``: scratch from attn_workspace() (allocated per call if None).
    Returns out (and lse [Hq, M] if requested or given)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _need(key_score, "key_score", torch.float32); _need(gain, "gain", torch.float32)
    _need(tau, "tau", torch.float32)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (n, hkv, d) or v.shape != k.shape or key_score.shape != (n,) \
            or gain.shape != (hq,) or tau.shape != (hq,):
        raise ValueError("attention operand shapes do not match")
    out, lse = _attn_out(q, out, lse, want_lse)
    ws, ws_bytes = _workspace(workspace, n, hq, hkv, d, q.device)
    _check(lib().tg_gated_attn_fwd(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, _ptr(key_score),
                                   _ptr(gain), _ptr(tau), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                   _stream(stream)))
    return (out, lse) if lse is not None else out


def gated_attn_fwd_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         key_score: torch.Tensor, gain: torch.Tensor, tau: torch.Tensor,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         out_f32: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """gated_attn_fwd for a training step: also returns lse [Hq, M] and the
    fp32 output before rounding (what gated_attn_bwd takes).
    Returns (out, lse, out_f32)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _need(key_score, "key_score", torch.float32); _need(gain, "gain", torch.float32)
    _need(tau, "tau", torch.float32)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (n, hkv, d) or v.shape != k.shape or key_score.shape != (n,) \
            or gain.shape != (hq,) or tau.shape != (hq,):
        raise ValueError("attention operand shapes do not match")
    out, lse = _attn_out(q, out, lse, True)
    if out_f32 is None:
        out_f32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _need(out_f32, "out_f32", torch.float32)
    if out_f32.shape != q.shape:
        raise ValueError("out_f32 must be shaped like q")
    ws, ws_bytes = _workspace(workspace, n, hq, hkv, d, q.device)
    _check(lib().tg_gated_attn_fwd_train(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d,
                                         _ptr(key_score), _ptr(gain), _ptr(tau), _ptr(out),
                                         _ptr(lse), _ptr(out_f32), _ptr(ws), ws_bytes,
                                         _stream(stream)))
    return out, lse, out_f32


def full_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  want_lse: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Unpruned causal GQA attention softmax(q.k / sqrt(d)) v over all rows."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (n, hkv, d) or v.shape != k.shape:
        raise ValueError("attention operand shapes do not match")
    out, lse = _attn_out(q, out, lse, want_lse)
    ws, ws_bytes = _workspace(workspace, n, hq, hkv, d, q.device)
    _check(lib().tg_full_attn_fwd(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, _ptr(out), _ptr(lse),
                                  _ptr(ws), ws_bytes, _stream(stream)))
    return (out, lse) if lse is not None else out


def attn_bwd_workspace_bytes(n: int, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    return int(lib().tg_attn_bwd_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim))


def attn_bwd_workspace(n: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                       device="cuda") -> torch.Tensor:
    """A device buffer large enough for one attention backward over n rows."""
    return torch.empty(max(attn_bwd_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim), 16),
                       dtype=torch.uint8, device=device)


def gated_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: torch.Tensor,
                   gain: torch.Tensor, tau: torch.Tensor, out_f32: torch.Tensor,
                   lse: torch.Tensor, dout: torch.Tensor, grads: Optional[dict] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of the gated attention given gated_attn_fwd_train's fp32
    output, its lse [Hq, M] and dout.
    Returns dict(dq, dk, dv (bf16, shaped like q, k, v), dscore [M], dgain [Hq],
    dtau [Hq] (fp32)); ``grads`` may hold preallocated tensors under those names."""
    out = out_f32
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, nm, torch.bfloat16)
    for t, nm in ((key_score, "key_score"), (gain, "gain"), (tau, "tau"), (lse, "lse"),
                  (out, "out_f32")):
        _need(t, nm, torch.float32)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (n, hkv, d) or v.shape != k.shape or out.shape != q.shape \
            or dout.shape != q.shape or lse.shape != (hq, n) or key_score.shape != (n,) \
            or gain.shape != (hq,) or tau.shape != (hq,):
        raise ValueError("attention backward operand shapes do not match")
    g = dict(grads or {})
    g.setdefault("dq", torch.empty_like(q))
    g.setdefault("dk", torch.empty_like(k))
    g.setdefault("dv", torch.empty_like(v))
    g.setdefault("dscore", torch.empty(n, dtype=torch.float32, device=q.device))
    g.setdefault("dgain", torch.empty(hq, dtype=torch.float32, device=q.device))
    g.setdefault("dtau", torch.empty(hq, dtype=torch.float32, device=q.device))
    for nm in ("dq", "dk", "dv"):
        _need(g[nm], nm, torch.bfloat16)
    for nm in ("dscore", "dgain", "dtau"):
        _need(g[nm], nm, torch.float32)
    if workspace is None:
        workspace = attn_bwd_workspace(n, hq, hkv, d, q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check(lib().tg_gated_attn_bwd(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, _ptr(key_score),
                                   _ptr(gain), _ptr(tau), _ptr(out), _ptr(lse), _ptr(dout),
                                   _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dscore"]),
                                   _ptr(g["dgain"]), _ptr(g["dtau"]), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return g


def gdn_workspace_bytes(n: int, n_qk_heads: int, n_v_heads: int, head_dim: int = 128) -> int:
    return int(lib().tg_gdn_workspace_bytes(n, n_qk_heads, n_v_heads, head_dim))


def gdn_workspace(n: int, n_qk_heads: int, n_v_heads: int, head_dim: int = 128,
                  device="cuda") -> torch.Tensor:
    """A device buffer large enough for one Gated DeltaNet call over n rows."""
    return torch.empty(max(gdn_workspace_bytes(n, n_qk_heads, n_v_heads, head_dim), 16),
                       dtype=torch.uint8, device=device)


def gdn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
            beta: torch.Tensor, scale: Optional[float] = None,
            initial_state: Optional[torch.Tensor] = None, want_state: bool = False,
            out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, stream=None):
    """Gated delta rule over the rows of q/k [n, Hk, d], v [n, Hv, d] (bf16),
    g/beta [n, Hv] (fp32).  Returns out [n, Hv, d] bf16 (and the final state
    [Hv, d, d] fp32 if asked or given)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _need(g, "g", torch.float32); _need(beta, "beta", torch.float32)
    n, hk, d = q.shape
    hv = v.shape[1]
    if k.shape != q.shape or v.shape != (n, hv, d) or g.shape != (n, hv) or beta.shape != (n, hv):
        raise ValueError("gated delta rule operand shapes do not match")
    if out is None:
        out = torch.empty((n, hv, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if want_state and final_state is None:
        final_state = torch.empty((hv, d, d), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32)
    if workspace is None:
        workspace = gdn_workspace(n, hk, hv, d, q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    sc = 1.0 / (d ** 0.5) if scale is None else float(scale)
    _check(lib().tg_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), n, hk, hv, d, sc,
                            _ptr(initial_state), _ptr(final_state), _ptr(out), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))
    return (out, final_state) if final_state is not None else out


def decode_workspace_bytes(n: int, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    return int(lib().tg_decode_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim))


def decode_workspace(n: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                     device="cuda") -> torch.Tensor:
    """A device buffer large enough for one decode call over n cached rows."""
    return torch.empty(max(decode_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim), 16),
                       dtype=torch.uint8, device=device)


def gated_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 key_score: Optional[torch.Tensor] = None, gain: Optional[torch.Tensor] = None,
                 tau: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """One decode step: q [Hq, d] against the cache k/v [n, Hkv, d] (bf16).
    key_score [n], gain/tau [Hq] (fp32) add the score bias; all None gives
    plain attention.  Returns out [Hq, d] (and lse [Hq] if requested or given)."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.bfloat16)
    hq, d = q.shape
    n, hkv, _ = k_cache.shape
    if k_cache.shape != (n, hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("decode operand shapes do not match")
    given = [x is not None for x in (key_score, gain, tau)]
    if any(given) and not all(given):
        raise ValueError("key_score, gain and tau go together")
    if all(given):
        _need(key_score, "key_score", torch.float32); _need(gain, "gain", torch.float32)
        _need(tau, "tau", torch.float32)
        if key_score.shape != (n,) or gain.shape != (hq,) or tau.shape != (hq,):
            raise ValueError("key_score / gain / tau shapes do not match")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16)
    if want_lse and lse is None:
        lse = torch.empty(hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    if workspace is None:
        workspace = decode_workspace(n, hq, hkv, d, q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check(lib().tg_gated_decode_fwd(_ptr(q), _ptr(k_cache), _ptr(v_cache), n, hq, hkv, d,
                                     _ptr(key_score), _ptr(gain), _ptr(tau), _ptr(out), _ptr(lse),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
    return (out, lse) if lse is not None else out


def qk_norm_rope(src: torch.Tensor, positions: torch.Tensor, rows: Optional[torch.Tensor] = None,
                 norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                 theta: float = 1.0e6, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """out[i] = RoPE(RMSNorm(src[rows[i]]) * norm_weight) at positions[i].
    src [rows, heads, d] bf16; positions / rows [n] int32 (rows None: src[i]);
    norm_weight [d] fp32 or None (no normalisation)."""
    _need(src, "src", torch.bfloat16)
    _need(positions, "positions", torch.int32)
    src_rows, heads, d = src.shape
    n = positions.numel()
    if rows is not None:
        _need(rows, "rows", torch.int32)
        if rows.numel() != n:
            raise ValueError("rows and positions differ in length")
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", torch.float32)
        if norm_weight.numel() != d:
            raise ValueError("norm_weight must have head_dim entries")
    if out is None:
        out = torch.empty((n, heads, d), dtype=torch.bfloat16, device=src.device)
    _need(out, "out", torch.bfloat16)
    if tuple(out.shape) != (n, heads, d):
        raise ValueError("out shape does not match")
    _check(lib().tg_qk_norm_rope(_ptr(src), src_rows, _ptr(rows), _ptr(positions), n, heads, d,
                                 _ptr(norm_weight), eps, theta, _ptr(out), _stream(stream)))
    return out
