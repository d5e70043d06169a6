"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every entry point that include/tg.h declares, and
rejects invalid arguments on the host before any HIP call.  No call here
reaches a kernel launch.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from learned_token_pruning_tg_amd import tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tg.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
A = 4096  # a fake, 16-byte-aligned "device" address: never dereferenced by these calls


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tg.lib_path()):
        pytest.skip("libtg.so not built")
    return tg.lib()


def test_header_declares_the_five_entry_points():
    names = _declared()
    for fn in ("tg_gate_score", "tg_topk_select", "tg_topk_select_scores",
               "tg_topk_workspace_bytes", "tg_compact",
               "tg_gated_attn_fwd", "tg_full_attn_fwd", "tg_attn_workspace_bytes",
               "tg_gated_decode_fwd", "tg_decode_workspace_bytes", "tg_qk_norm_rope",
               "tg_gated_attn_bwd", "tg_attn_bwd_workspace_bytes", "tg_gated_attn_fwd_train",
               "tg_gdn_fwd", "tg_gdn_workspace_bytes",
               "tg_kept_count", "tg_status_str", "tg_last_error"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", tg.lib_path()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (tg_\w+)", out))
    assert set(_declared()) <= exported


def test_status_strings(L):
    assert tg.status_str(OK) == "ok"
    assert "invalid" in tg.status_str(INVALID)
    assert "unsupported" in tg.status_str(UNSUPPORTED)
    assert tg.status_str(99) == "unknown status"


@pytest.mark.parametrize("args,expect", [
    ((512, 0, 448, 128), 192), ((512, 0, 448, 0), 64), ((512, 0, 448, 10**6), 512),
    ((16384, 0, 16128, 2048), 2304), ((131072, 0, 130816, 8192), 8448),
    ((10, 3, 3, 5), 10), ((10, 2, 8, 4), 8), ((0, 0, 0, 0), 0),
    ((10, 5, 4, 1), -1), ((10, 0, 11, 1), -1), ((10, -1, 5, 1), -1), ((10, 0, 5, -1), -1),
])
def test_kept_count(L, args, expect):
    assert L.tg_kept_count(*args) == expect


@pytest.mark.parametrize("n,db,de", [(512, 0, 448), (16384, 0, 16128), (1000, 100, 900),
                                     (10, 3, 3), (64, 0, 64)])
def test_total_budget_maps_to_a_document_budget(L, n, db, de):
    """A budget B on all kept prefill tokens: the rows outside the document
    are always kept, so B is met exactly when it lies between that count and
    n, and clamped to those ends otherwise."""
    outside = n - (de - db)
    for b in (0, 1, outside - 1, outside, outside + 1, (outside + n) // 2, n - 1, n, n + 7):
        if b < 0:
            continue
        k = tg.k_doc_for_budget(n, db, de, b)
        assert k >= 0
        assert L.tg_kept_count(n, db, de, k) == min(max(b, outside), n)
    with pytest.raises(ValueError):
        tg.k_doc_for_budget(n, db, de, -1)


def test_gate_validation(L):
    s = 0
    f = L.tg_gate_score
    assert f(A, -1, 256, 256, A, A, A, 0.0, 64, A, s) == INVALID
    assert f(A, 10, 200, 256, A, A, A, 0.0, 64, A, s) == INVALID         # ld_h < hidden
    assert f(A, 10, 260, 256, A, A, A, 0.0, 64, A, s) == INVALID         # ld_h % 8
    assert f(A, 10, 256, 250, A, A, A, 0.0, 64, A, s) == UNSUPPORTED     # hidden % 64
    assert f(A, 10, 256, 224, A, A, A, 0.0, 64, A, s) == UNSUPPORTED
    assert f(A, 10, 256, 256, A, A, A, 0.0, 544, A, s) == UNSUPPORTED    # gate_hidden > 512
    assert f(None, 10, 256, 256, A, A, A, 0.0, 64, A, s) == INVALID
    assert f(A + 2, 10, 256, 256, A, A, A, 0.0, 64, A, s) == INVALID     # alignment
    assert "aligned" in tg.last_error()
    assert f(None, 0, 256, 256, None, None, None, 0.0, 64, None, s) == OK  # n == 0: no-op


def test_topk_validation(L):
    f = L.tg_topk_select
    W = 1 << 20  # a (fake) workspace size that is always large enough
    assert f(A, 10, 0, 11, 3, A, A, W, 0) == INVALID
    assert f(A, 10, 6, 5, 3, A, A, W, 0) == INVALID
    assert f(A, 10, 0, 5, -1, A, A, W, 0) == INVALID
    assert f(None, 10, 0, 5, 3, A, A, W, 0) == INVALID
    assert f(A, 1 << 31, 0, 5, 3, A, A, W, 0) == INVALID
    assert f(A, 1 << 30, 0, 5, 3, A, A, W, 0) == INVALID                 # n < 2^30
    need = L.tg_topk_workspace_bytes(10)
    assert f(A, 10, 0, 5, 3, A, None, W, 0) == WORKSPACE
    assert f(A, 10, 0, 5, 3, A, A, need - 1, 0) == WORKSPACE
    assert f(A, 10, 0, 5, 3, A, A + 4, need, 0) == WORKSPACE             # alignment
    assert "workspace" in tg.last_error()
    assert f(None, 0, 0, 0, 3, None, None, 0, 0) == OK
    assert f(A, 10, 0, 10, 0, None, A, W, 0) == OK                       # nothing kept


def test_topk_scores_validation(L):
    # the same checks as tg_topk_select, plus kept_scores: required when rows
    # are kept, may be NULL when none are
    f = L.tg_topk_select_scores
    W = 1 << 20
    assert f(A, 10, 0, 11, 3, A, A, A, W, 0) == INVALID
    assert f(A, 10, 0, 5, 3, A, None, A, W, 0) == INVALID                # kept_scores NULL
    assert "kept_scores" in tg.last_error()
    assert f(None, 10, 0, 5, 3, A, A, A, W, 0) == INVALID
    assert f(A, 10, 0, 5, 3, A, A, None, W, 0) == WORKSPACE
    assert f(None, 0, 0, 0, 3, None, None, None, 0, 0) == OK
    assert f(A, 10, 0, 5, 0, A, None, A, W, 0) == INVALID                # 5 kept (non-document rows)
    assert f(A, 10, 0, 10, 0, None, None, A, W, 0) == OK                 # nothing kept


def _topk_ws(n):
    """The top-K workspace size restated: 5136 words (three histograms of
    2048, 2048 and 1024 bins, 16 words of selection state) plus two words per
    range of rows; ranges are whole multiples of 2048 rows, at most 1024."""
    subs = -(-n // 2048)
    rows = 2048 * -(-subs // 1024)
    groups = -(-n // rows)
    return (5136 + 2 * groups) * 4


@pytest.mark.parametrize("n", [1, 2047, 2048, 2049, 16384, 131072, 2048 * 1024,
                               2048 * 1024 + 1, (1 << 30) - 1])
def test_topk_workspace_bytes(L, n):
    assert L.tg_topk_workspace_bytes(n) == _topk_ws(n)
    assert L.tg_topk_workspace_bytes(n) < 29 * 1024 + 1
    assert L.tg_topk_workspace_bytes(0) == 0
    assert L.tg_topk_workspace_bytes(1 << 30) == 0


def test_compact_validation(L):
    f = L.tg_compact
    assert f(A, -1, A, 10, 16, 16, A * 4, 16, 0) == INVALID
    assert f(A, 4, A, 10, 8, 16, A * 4, 16, 0) == INVALID               # src stride < row
    assert f(A, 4, A, 10, 16, 16, A + 64, 16, 0) == INVALID             # overlap
    assert "overlap" in tg.last_error()
    assert f(None, 4, A, 10, 16, 16, A * 4, 16, 0) == INVALID
    assert f(None, 0, None, 0, 16, 16, None, 16, 0) == OK


def test_attention_validation(L):
    g = L.tg_gated_attn_fwd
    full = L.tg_full_attn_fwd
    W = 1 << 30  # a (fake) workspace size that is always large enough
    assert g(A, A, A, 10, 16, 8, 96, A, A, A, A, None, A, W, 0) == UNSUPPORTED
    assert "head_dim" in tg.last_error()
    assert g(A, A, A, 10, 16, 6, 128, A, A, A, A, None, A, W, 0) == INVALID
    assert g(A, A, A, 10, 0, 8, 128, A, A, A, A, None, A, W, 0) == INVALID
    assert g(A, A, A, -3, 16, 8, 128, A, A, A, A, None, A, W, 0) == INVALID
    assert g(A, A, A, 10, 16, 8, 128, None, A, A, A, None, A, W, 0) == INVALID  # key_score
    assert g(A + 8, A, A, 10, 16, 8, 128, A, A, A, A, None, A, W, 0) == INVALID
    assert full(A, A, None, 10, 16, 8, 128, A, None, A, W, 0) == INVALID
    assert full(A, A, A, 10, 16, 8, 64 + 1, A, None, A, W, 0) == UNSUPPORTED
    assert full(A, A, A, 1 << 20, 16, 8, 128, A, None, A, W, 0) == UNSUPPORTED  # 2^31-byte offsets
    need = L.tg_attn_workspace_bytes(100, 16, 8, 128)
    assert need == 2 * 8 * 128 * 128 + 16 * 2 * 256  # V^T images (2 tiles x 8 heads) + fp32 biases
    assert g(A, A, A, 100, 16, 8, 128, A, A, A, A, None, A, need - 1, 0) == WORKSPACE
    assert full(A, A, A, 100, 16, 8, 128, A, None, A, 1000, 0) == WORKSPACE
    assert full(A, A, A, 100, 16, 8, 128, A, None, None, need, 0) == WORKSPACE
    assert g(A, A, A, 100, 16, 8, 128, A, A, A, A, None, A + 4, need, 0) == WORKSPACE
    assert "workspace" in tg.last_error()
    assert g(None, None, None, 0, 16, 8, 128, None, None, None, None, None, None, 0, 0) == OK
    assert full(None, None, None, 0, 16, 8, 128, None, None, None, 0, 0) == OK
    assert L.tg_attn_workspace_bytes(0, 16, 8, 128) == 0
    assert L.tg_attn_workspace_bytes(100, 16, 6, 128) == 0
    assert L.tg_attn_workspace_bytes(100, 16, 8, 96) == 0


def test_gdn_workspace_bytes(L):
    # per 64-row chunk and value head 72.25 KiB: -W, U', P, Kt^T, scaled q, Gam_last;
    # plus the fp32 state handed between the pieces of the recurrence
    rec = 16384 + 16384 + 8192 + 16384 + 16384 + 256
    for n, hk, hv in ((1, 1, 1), (64, 16, 32), (65, 16, 32), (8448, 16, 32)):
        assert L.tg_gdn_workspace_bytes(n, hk, hv, 128) == -(-n // 64) * hv * rec + hv * 128 * 128 * 4
    assert L.tg_gdn_workspace_bytes(0, 16, 32, 128) == 0
    assert L.tg_gdn_workspace_bytes(100, 16, 24, 128) == 0      # 24 % 16
    assert L.tg_gdn_workspace_bytes(100, 16, 32, 64) == 0


def test_gdn_validation(L):
    f = L.tg_gdn_fwd
    W = 1 << 34
    #        q  k  v  g  b  n   hk hv d    scale s0 s1 out ws wsb
    def call(n=10, hk=2, hv=4, d=128, scale=0.1, q=A, g=A, s0=None, s1=None, out=A, ws=A, wsb=W):
        return f(q, A, A, g, A, n, hk, hv, d, ctypes.c_float(scale), s0, s1, out, ws, wsb, 0)
    assert call(n=-1) == INVALID
    assert call(hk=3, hv=4) == INVALID
    assert call(hk=0) == INVALID
    assert call(d=64) == UNSUPPORTED
    assert call(n=1 << 20, hk=16, hv=32) == UNSUPPORTED               # 2^31-byte offsets
    assert call(scale=float("nan")) == INVALID
    assert call(scale=float("inf")) == INVALID
    assert call(q=None) == INVALID
    assert call(out=None) == INVALID
    assert call(q=A + 8) == INVALID                                  # alignment
    assert call(g=A + 2) == INVALID
    assert call(s0=A + 4) == INVALID
    need = L.tg_gdn_workspace_bytes(10, 2, 4, 128)
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(n=0, q=None, g=None, out=None, ws=None, wsb=0) == OK   # no-op


def test_training_forward_validation(L):
    t = L.tg_gated_attn_fwd_train
    W = 1 << 30
    #        q  k  v  n   hq hkv d    s  g  tau out lse out32 ws wsb
    assert t(A, A, A, 10, 16, 8, 96, A, A, A, A, A, A, A, W, 0) == UNSUPPORTED
    assert t(A, A, A, 10, 16, 8, 128, A, A, A, A, None, A, A, W, 0) == INVALID    # lse required
    assert "lse" in tg.last_error()
    assert t(A, A, A, 10, 16, 8, 128, A, A, A, A, A, None, A, W, 0) == INVALID    # out_f32 required
    assert t(A, A, A, 10, 16, 8, 128, A, A, A, A, A, A + 4, A, W, 0) == INVALID   # alignment
    assert t(A, A, A, 10, 16, 8, 128, None, A, A, A, A, A, A, W, 0) == INVALID    # key_score
    need = L.tg_attn_workspace_bytes(100, 16, 8, 128)
    assert t(A, A, A, 100, 16, 8, 128, A, A, A, A, A, A, A, need - 1, 0) == WORKSPACE
    assert t(None, None, None, 0, 16, 8, 128, None, None, None, None, None, None, None, 0, 0) == OK


def _simulated_makespan(n, n_qt, h, hq):
    """Work-groups in launch order (longest query tiles first, last chunk
    first, heads interleaved) onto 512 resident slots; each takes its key
    tiles plus 2 (plus 1 more when it writes a split partial)."""
    import heapq
    slots = [0.0] * 512
    end = 0.0
    for qt in range(n_qt - 1, -1, -1):
        walk = -(-min(128 * (qt + 1), n) // 64)
        nch = (qt + h) // h
        for c in range(nch - 1, -1, -1):
            dur = min(2 * h, walk - 2 * h * c) + 2.0 + (1.0 if nch > 1 else 0.0)
            for _ in range(hq):
                t = heapq.heappop(slots) + dur
                end = max(end, t)
                heapq.heappush(slots, t)
    return end


def _split_layout(n, hq, hkv, d, gated=True):
    """Workspace bytes restated from the split-key rule: 128-row query
    blocks, 64-key tiles, 512 resident work-groups; block qt is cut into
    ceil((qt + 1) / h) chunks of 2h tiles (1.3x the average walk per
    work-group) when its 2 n_qt-tile walk exceeds that average, one tile
    shorter when the dispatch simulation finishes more than 6 % sooner."""
    import math
    n_qt, n_tiles = -(-n // 128), -(-n // 64)
    part = 4 * (64 * d + 512)
    avg = hq * n_qt * (n_qt + 1) / 512
    h = n_qt
    if 2 * n_qt > avg:
        h = max(4, math.ceil(1.3 * avg / 2))
    h = max(min(h, n_qt), 1)
    if 4 < h < n_qt and _simulated_makespan(n, n_qt, h - 1, hq) < 0.94 * _simulated_makespan(n, n_qt, h, hq):
        h -= 1
    units = sum(-(-(qt + 1) // h) for qt in range(n_qt))
    img = d * 128                              # V^T image of one tile (fp16, 128-byte rows)
    sc = hq * n_tiles * 64 * 4                 # per query head and key: the fp32 bias
    n_part = units - min(h, n_qt)
    return n_tiles * hkv * img + -(-sc // 256) * 256 + hq * n_part * part, h, units


@pytest.mark.parametrize("n,hq,hkv,d", [(2304, 16, 8, 128), (1000, 2, 1, 128), (1280, 16, 8, 64),
                                         (8448, 16, 8, 128), (700, 4, 2, 64), (64, 1, 1, 128),
                                         (4352, 16, 8, 128), (5000, 2, 1, 128), (3000, 1, 1, 64),
                                         (2300, 16, 8, 128)])
def test_attention_workspace_split_layout(L, n, hq, hkv, d):
    want, h, units = _split_layout(n, hq, hkv, d)
    assert L.tg_attn_workspace_bytes(n, hq, hkv, d) == want
    if (n, hq) == (2304, 16):
        assert (h, units) == (6, 36)          # the 16k-context kept prefix splits three ways
    if (n, hq) == (4352, 16):
        assert h == 25                        # 32k: the simulation keeps the base choice
    if (n, hq) == (8448, 16):
        assert h == -(-8448 // 128)           # long prefixes: no split


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(tg, "_lib", None)
    monkeypatch.setattr(tg, "_LIB_PATH", "/nonexistent/libtg.so")
    with pytest.raises(RuntimeError, match="missing"):
        tg.lib()


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "learned_token_pruning_tg_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), fn
                assert "oracle/" not in text, fn


def _decode_ws(n, hq, hkv, d):
    """The decode workspace restated: chunks of 256 keys when that gives >= 512
    work-groups over the KV heads, else 128 when that gives >= 128, else 64
    (at most 128 for groups of 4 query heads, 64 for 8); per (KV head, chunk,
    query head of its group) a (max, sum, d outputs) fp32 state."""
    g = hq // hkv
    c = 256 if g <= 2 else 128 if g == 4 else 64
    while c > 64 and -(-n // c) * hkv < (512 if c == 256 else 128):
        c //= 2
    return hkv * -(-n // c) * (hq // hkv) * (d + 2) * 4


@pytest.mark.parametrize("n,hq,hkv,d", [(1, 16, 8, 128), (2304, 16, 8, 128), (8448, 16, 8, 128),
                                        (131072, 16, 8, 128), (300, 8, 1, 64), (5000, 32, 4, 128),
                                        (64, 4, 4, 64)])
def test_decode_workspace_bytes(L, n, hq, hkv, d):
    assert L.tg_decode_workspace_bytes(n, hq, hkv, d) == _decode_ws(n, hq, hkv, d)


def test_decode_validation(L):
    f = L.tg_gated_decode_fwd
    W = 1 << 30
    assert f(A, A, A, 0, 16, 8, 128, A, A, A, A, None, A, W, 0) == INVALID       # no cached row
    assert f(A, A, A, 10, 16, 6, 128, A, A, A, A, None, A, W, 0) == INVALID      # Hq % Hkv
    assert f(A, A, A, 10, 16, 8, 96, A, A, A, A, None, A, W, 0) == UNSUPPORTED   # head_dim
    assert f(A, A, A, 10, 48, 3, 128, A, A, A, A, None, A, W, 0) == UNSUPPORTED  # group 16
    assert f(A, A, A, 1 << 20, 16, 8, 128, A, A, A, A, None, A, W, 0) == UNSUPPORTED  # 2^31 bytes
    assert f(A, A, None, 10, 16, 8, 128, A, A, A, A, None, A, W, 0) == INVALID
    assert f(A, A, A, 10, 16, 8, 128, A, None, A, A, None, A, W, 0) == INVALID   # partial bias
    assert "all be given" in tg.last_error()
    assert f(A + 8, A, A, 10, 16, 8, 128, A, A, A, A, None, A, W, 0) == INVALID  # alignment
    need = L.tg_decode_workspace_bytes(10, 16, 8, 128)
    assert f(A, A, A, 10, 16, 8, 128, A, A, A, A, None, A, need - 1, 0) == WORKSPACE
    assert f(A, A, A, 10, 16, 8, 128, None, None, None, A, None, None, W, 0) == WORKSPACE
    assert L.tg_decode_workspace_bytes(0, 16, 8, 128) == 0
    assert L.tg_decode_workspace_bytes(10, 16, 8, 96) == 0


def test_qk_norm_rope_validation(L):
    f = L.tg_qk_norm_rope
    B = A * 64   # a second fake address far from A
    assert f(A, 10, None, A, -1, 4, 128, None, 1e-6, 1e6, B, 0) == INVALID
    assert f(A, 10, None, A, 5, 0, 128, None, 1e-6, 1e6, B, 0) == INVALID
    assert f(A, 10, None, A, 5, 4, 96, None, 1e-6, 1e6, B, 0) == UNSUPPORTED
    assert f(A, 10, None, A, 5, 4, 128, None, 1e-6, 0.0, B, 0) == INVALID       # theta
    assert f(A, 10, None, A, 11, 4, 128, None, 1e-6, 1e6, B, 0) == INVALID      # n > src_rows
    assert f(A, 10, None, None, 5, 4, 128, None, 1e-6, 1e6, B, 0) == INVALID    # positions
    assert f(A + 8, 10, None, A, 5, 4, 128, None, 1e-6, 1e6, B, 0) == INVALID   # alignment
    assert f(A, 10, A, A, 5, 4, 128, None, 1e-6, 1e6, A + 1024, 0) == INVALID   # overlap
    assert "overlap" in tg.last_error()
    assert f(None, 0, None, None, 0, 4, 128, None, 1e-6, 1e6, None, 0) == OK    # n == 0


def _bwd_split(longest, total):
    """Walks longer than 1.3x the average steps per resident work-group (512)
    are cut into chunks of that length (at least 8 steps)."""
    avg = total / 512.0
    ln = longest
    if longest > 1.3 * avg:
        ln = max(8, math.ceil(1.3 * avg))
    ln = max(1, min(ln, longest))
    return ln, -(-longest // ln)


def _bwd_ws(n, hq, hkv, d):
    """The backward workspace restated: rows padded to whole 128-row blocks;
    (lse, D) as 64 floats per query head and 32-row tile;
    per dK/dV chunk, query head and padded row one column-sum float and d fp32
    each of the dk and dv partials; per dK/dV chunk, query head and 128-row
    block one float (gain partial); per dQ chunk the same for q.dq; fp32 dq
    partials when the dQ walks are split; every region rounded up to 256 bytes."""
    t128 = -(-n // 128)
    t32, mp = 4 * t128, 128 * t128
    t_real = -(-n // 32)
    _, nkv = _bwd_split(t_real, hq * sum(t_real - 4 * b for b in range(t128)))
    _, nq = _bwd_split(t_real, hq * sum(min(4 * b + 4, t_real) for b in range(t128)))
    o = 0
    for size in (hq * t32 * 256,
                 nkv * hq * mp * 4, nkv * hq * mp * d * 4, nkv * hq * mp * d * 4,
                 nkv * hq * t128 * 4, nq * hq * t128 * 4, nq * mp * hq * d * 4 if nq > 1 else 0):
        o = -(-(o + size) // 256) * 256
    return o


def test_attn_bwd_split_rule():
    assert _bwd_split(264, 16 * 8844) == (264, 1)       # 8448 rows: balanced, no split
    assert _bwd_split(72, 16 * 684) == (28, 3)          # 2304 rows: three chunks


@pytest.mark.parametrize("n,hq,hkv,d", [(1, 16, 8, 128), (2304, 16, 8, 128), (4352, 16, 8, 128),
                                        (8448, 16, 8, 128), (300, 8, 1, 64), (129, 4, 2, 64)])
def test_attn_bwd_workspace_bytes(L, n, hq, hkv, d):
    assert L.tg_attn_bwd_workspace_bytes(n, hq, hkv, d) == _bwd_ws(n, hq, hkv, d)


def test_attn_bwd_validation(L):
    f = L.tg_gated_attn_bwd
    W = 1 << 34
    P = [A] * 13   # key_score, gain, tau, out_f32, lse, dout, dq, dk, dv, dscore, dgain, dtau
    def call(n=10, hq=16, hkv=8, d=128, q=A, ptrs=None, ws=A, wsb=W):
        p = list(P[:12] if ptrs is None else ptrs)
        return f(q, A, A, n, hq, hkv, d, *p, ws, wsb, 0)
    assert call(n=-1) == INVALID
    assert call(hkv=6) == INVALID                                   # Hq % Hkv
    assert call(d=96) == UNSUPPORTED
    assert call(n=1 << 20) == UNSUPPORTED                           # 2^31 bytes of q
    assert call(n=0, q=None, ptrs=[None] * 12, ws=None, wsb=0) == OK   # no-op
    for i in range(12):                                             # every pointer required
        ptrs = [A] * 12
        ptrs[i] = None
        assert call(ptrs=ptrs) == INVALID, i
    assert call(q=A + 8) == INVALID                                 # alignment
    need = L.tg_attn_bwd_workspace_bytes(10, 16, 8, 128)
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=A + 8, wsb=need + 64) == WORKSPACE               # workspace alignment
    assert L.tg_attn_bwd_workspace_bytes(0, 16, 8, 128) == 0
    assert L.tg_attn_bwd_workspace_bytes(10, 16, 8, 96) == 0
