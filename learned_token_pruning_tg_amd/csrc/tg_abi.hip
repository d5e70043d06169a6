// C ABI of libtg: host-side argument validation, error reporting and dispatch
// to the HIP launchers.  Every check runs before any HIP call, so a rejected
// call touches neither the device nor the stream.
#include <stdarg.h>
#include <stdio.h>

#include "tg.h"
#include "tg_launch.h"

namespace {

thread_local char g_err[512] = "";

tg_status fail(tg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

tg_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TG_OK;
  return fail(TG_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipStream_t as_hip(tg_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

tg_status check_attn(const char* fn, const tg_bf16* q, const tg_bf16* k, const tg_bf16* v,
                     int64_t n, int32_t hq, int32_t hkv, int32_t d, const tg_bf16* out,
                     const void* ws, size_t ws_bytes, bool gated) {
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(TG_E_INVALID, "%s: n=%lld out of range", fn, (long long)n);
  if (hq <= 0 || hkv <= 0) return fail(TG_E_INVALID, "%s: head counts must be positive", fn);
  if (hq % hkv != 0)
    return fail(TG_E_INVALID, "%s: n_q_heads=%d not a multiple of n_kv_heads=%d", fn, hq, hkv);
  if (d != 64 && d != 128) return fail(TG_E_UNSUPPORTED, "%s: head_dim=%d (supported: 64, 128)", fn, d);
  if (n * hq * d * 2 >= (int64_t(1) << 31))
    return fail(TG_E_UNSUPPORTED, "%s: n=%lld rows of %d heads x %d exceed 2^31 bytes", fn,
                (long long)n, hq, d);
  if (n == 0) return TG_OK;
  if (!q || !k || !v || !out) return fail(TG_E_INVALID, "%s: null tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(TG_E_INVALID, "%s: q/k/v/out must be 16-byte aligned", fn);
  const size_t per_head = tg::attn_image_bytes_per_kv_head(n, d, gated);
  if (per_head >= (size_t(1) << 32))
    return fail(TG_E_UNSUPPORTED, "%s: n=%lld needs %zu tile-image bytes per KV head (limit 2^32)",
                fn, (long long)n, per_head);
  const size_t need = tg::attn_workspace_bytes(n, hq, hkv, d, gated);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(TG_E_WORKSPACE, "%s: workspace %p of %zu bytes (need %zu, 16-byte aligned)", fn, ws,
                ws_bytes, need);
  return TG_OK;
}

}  // namespace

extern "C" {

const char* tg_status_str(tg_status s) {
  switch (s) {
    case TG_OK: return "ok";
    case TG_E_INVALID: return "invalid argument";
    case TG_E_UNSUPPORTED: return "unsupported shape";
    case TG_E_WORKSPACE: return "workspace too small";
    case TG_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tg_last_error(void) { return g_err; }

int64_t tg_kept_count(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k_doc) {
  if (!(0 <= doc_begin && doc_begin <= doc_end && doc_end <= n) || k_doc < 0) return -1;
  const int64_t n_doc = doc_end - doc_begin;
  return (k_doc < n_doc ? k_doc : n_doc) + (n - n_doc);
}

tg_status tg_gate_score(const tg_bf16* h, int64_t n, int64_t ld_h, int32_t hidden,
                        const tg_bf16* w1, const float* b1, const float* w2, float b2,
                        int32_t gate_hidden, float* scores, tg_stream_t stream) {
  if (n < 0) return fail(TG_E_INVALID, "tg_gate_score: n=%lld < 0", (long long)n);
  if (hidden <= 0 || gate_hidden <= 0)
    return fail(TG_E_INVALID, "tg_gate_score: hidden=%d gate_hidden=%d must be positive", hidden,
                gate_hidden);
  if (ld_h < hidden) return fail(TG_E_INVALID, "tg_gate_score: ld_h=%lld < hidden=%d", (long long)ld_h, hidden);
  if (hidden % 64 != 0 || gate_hidden > 512)
    return fail(TG_E_UNSUPPORTED,
                "tg_gate_score: hidden=%d gate_hidden=%d (need hidden %% 64 == 0, gate_hidden <= 512)",
                hidden, gate_hidden);
  if (ld_h % 8 != 0) return fail(TG_E_INVALID, "tg_gate_score: ld_h=%lld not a multiple of 8", (long long)ld_h);
  if (n == 0) return TG_OK;
  if (!h || !w1 || !b1 || !w2 || !scores) return fail(TG_E_INVALID, "tg_gate_score: null pointer");
  if (!aligned16(h) || !aligned16(w1)) return fail(TG_E_INVALID, "tg_gate_score: h/w1 must be 16-byte aligned");
  return hip_status(tg::launch_gate_score(h, n, ld_h, hidden, w1, b1, w2, b2, gate_hidden, scores,
                                          as_hip(stream)),
                    "tg_gate_score launch");
}

size_t tg_topk_workspace_bytes(int64_t n) {
  if (n <= 0 || n >= (int64_t(1) << 30)) return 0;
  return tg::topk_workspace_bytes(n);
}

namespace {
tg_status topk_select_impl(const char* fn, const float* scores, int64_t n, int64_t doc_begin,
                           int64_t doc_end, int64_t k_doc, int32_t* kept_idx, float* kept_scores,
                           void* workspace, size_t workspace_bytes, tg_stream_t stream) {
  if (n < 0 || n >= (int64_t(1) << 30))
    return fail(TG_E_INVALID, "%s: n=%lld out of range (n < 2^30)", fn, (long long)n);
  if (tg_kept_count(n, doc_begin, doc_end, k_doc) < 0)
    return fail(TG_E_INVALID, "%s: need 0 <= doc_begin=%lld <= doc_end=%lld <= n=%lld, k_doc=%lld >= 0",
                fn, (long long)doc_begin, (long long)doc_end, (long long)n, (long long)k_doc);
  const size_t need = tg::topk_workspace_bytes(n);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(TG_E_WORKSPACE, "%s: workspace %p of %zu bytes (need %zu, 16-byte aligned)", fn,
                workspace, workspace_bytes, need);
  if (n == 0 || tg_kept_count(n, doc_begin, doc_end, k_doc) == 0) return TG_OK;  // nothing kept
  if (!scores || !kept_idx) return fail(TG_E_INVALID, "%s: null pointer", fn);
  return hip_status(tg::launch_topk_select(scores, n, doc_begin, doc_end, k_doc, kept_idx,
                                           kept_scores, workspace, as_hip(stream)),
                    fn);
}
}  // namespace

tg_status tg_topk_select(const float* scores, int64_t n, int64_t doc_begin, int64_t doc_end,
                         int64_t k_doc, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                         tg_stream_t stream) {
  return topk_select_impl("tg_topk_select", scores, n, doc_begin, doc_end, k_doc, kept_idx, nullptr,
                          workspace, workspace_bytes, stream);
}

tg_status tg_topk_select_scores(const float* scores, int64_t n, int64_t doc_begin,
                                int64_t doc_end, int64_t k_doc, int32_t* kept_idx,
                                float* kept_scores, void* workspace, size_t workspace_bytes,
                                tg_stream_t stream) {
  if (!kept_scores && n > 0 && tg_kept_count(n, doc_begin, doc_end, k_doc) > 0)
    return fail(TG_E_INVALID, "tg_topk_select_scores: kept_scores is null");
  return topk_select_impl("tg_topk_select_scores", scores, n, doc_begin, doc_end, k_doc, kept_idx,
                          kept_scores, workspace, workspace_bytes, stream);
}

tg_status tg_topk_select_noalloc(const float* scores, int64_t n, int64_t doc_begin, int64_t doc_end,
                                 int64_t k_doc, int32_t* kept_idx, tg_stream_t stream) {
  const char* fn = "tg_topk_select_noalloc";
  if (n < 0 || n >= (int64_t(1) << 30))
    return fail(TG_E_INVALID, "%s: n=%lld out of range (n < 2^30)", fn, (long long)n);
  if (tg_kept_count(n, doc_begin, doc_end, k_doc) < 0)
    return fail(TG_E_INVALID, "%s: need 0 <= doc_begin=%lld <= doc_end=%lld <= n=%lld, k_doc=%lld >= 0",
                fn, (long long)doc_begin, (long long)doc_end, (long long)n, (long long)k_doc);
  const size_t need = tg::topk_workspace_bytes(n);
  if (need > tg::kTopkScratchBytes)
    return fail(TG_E_UNSUPPORTED, "%s: n=%lld needs %zu scratch bytes, above the static %zu",
                fn, (long long)n, need, tg::kTopkScratchBytes);
  if (n == 0 || tg_kept_count(n, doc_begin, doc_end, k_doc) == 0) return TG_OK;  // nothing kept
  if (!scores || !kept_idx) return fail(TG_E_INVALID, "%s: null pointer", fn);
  return hip_status(tg::launch_topk_select_noalloc(scores, n, doc_begin, doc_end, k_doc, kept_idx,
                                                   as_hip(stream)),
                    "tg_topk_select_noalloc launch");
}

tg_status tg_compact(const int32_t* kept_idx, int64_t n_kept, const void* src, int64_t src_rows,
                     int64_t src_stride_bytes, int64_t row_bytes, void* dst,
                     int64_t dst_stride_bytes, tg_stream_t stream) {
  if (n_kept < 0 || src_rows < 0 || row_bytes < 0)
    return fail(TG_E_INVALID, "tg_compact: negative size");
  if (src_stride_bytes < row_bytes || dst_stride_bytes < row_bytes)
    return fail(TG_E_INVALID, "tg_compact: strides (%lld, %lld) smaller than row_bytes=%lld",
                (long long)src_stride_bytes, (long long)dst_stride_bytes, (long long)row_bytes);
  if (n_kept == 0 || row_bytes == 0) return TG_OK;
  if (!kept_idx || !src || !dst) return fail(TG_E_INVALID, "tg_compact: null pointer");
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  const char* s1 = s0 + (src_rows > 0 ? (src_rows - 1) * src_stride_bytes + row_bytes : 0);
  const char* d1 = d0 + (n_kept - 1) * dst_stride_bytes + row_bytes;
  if (s0 < d1 && d0 < s1) return fail(TG_E_INVALID, "tg_compact: src and dst overlap");
  return hip_status(tg::launch_compact(kept_idx, n_kept, src, src_rows, src_stride_bytes, row_bytes,
                                       dst, dst_stride_bytes, as_hip(stream)),
                    "tg_compact launch");
}

size_t tg_attn_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  if (n <= 0 || n >= (int64_t(1) << 31) || n_q_heads <= 0 || n_kv_heads <= 0 ||
      n_q_heads % n_kv_heads != 0 || (head_dim != 64 && head_dim != 128))
    return 0;
  return tg::attn_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim, true);
}

tg_status tg_gated_attn_fwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            const float* key_score, const float* gain, const float* tau,
                            tg_bf16* out, float* lse, void* workspace, size_t workspace_bytes,
                            tg_stream_t stream) {
  const char* fn = "tg_gated_attn_fwd";
  const tg_status st = check_attn(fn, q, k, v, n, n_q_heads, n_kv_heads, head_dim, out,
                                  workspace, workspace_bytes, true);
  if (st != TG_OK || n == 0) return st;
  if (!key_score || !gain || !tau) return fail(TG_E_INVALID, "%s: null key_score/gain/tau", fn);
  return hip_status(tg::launch_attn_fwd(q, k, v, n, n_q_heads, n_kv_heads, head_dim, key_score,
                                        gain, tau, out, lse, nullptr, workspace, as_hip(stream)),
                    "tg_gated_attn_fwd launch");
}

tg_status tg_gated_attn_fwd_train(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                                  int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                  const float* key_score, const float* gain, const float* tau,
                                  tg_bf16* out, float* lse, float* out_f32, void* workspace,
                                  size_t workspace_bytes, tg_stream_t stream) {
  const char* fn = "tg_gated_attn_fwd_train";
  const tg_status st = check_attn(fn, q, k, v, n, n_q_heads, n_kv_heads, head_dim, out,
                                  workspace, workspace_bytes, true);
  if (st != TG_OK || n == 0) return st;
  if (!key_score || !gain || !tau) return fail(TG_E_INVALID, "%s: null key_score/gain/tau", fn);
  if (!lse || !out_f32) return fail(TG_E_INVALID, "%s: null lse/out_f32", fn);
  if (!aligned16(out_f32)) return fail(TG_E_INVALID, "%s: out_f32 must be 16-byte aligned", fn);
  return hip_status(tg::launch_attn_fwd(q, k, v, n, n_q_heads, n_kv_heads, head_dim, key_score,
                                        gain, tau, out, lse, out_f32, workspace, as_hip(stream)),
                    "tg_gated_attn_fwd_train launch");
}

tg_status tg_full_attn_fwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           tg_bf16* out, float* lse, void* workspace, size_t workspace_bytes,
                           tg_stream_t stream) {
  const tg_status st = check_attn("tg_full_attn_fwd", q, k, v, n, n_q_heads, n_kv_heads, head_dim,
                                  out, workspace, workspace_bytes, false);
  if (st != TG_OK || n == 0) return st;
  return hip_status(tg::launch_attn_fwd(q, k, v, n, n_q_heads, n_kv_heads, head_dim, nullptr,
                                        nullptr, nullptr, out, lse, nullptr, workspace,
                                        as_hip(stream)),
                    "tg_full_attn_fwd launch");
}

size_t tg_attn_bwd_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim) {
  if (n <= 0 || n >= (int64_t(1) << 31) || n_q_heads <= 0 || n_kv_heads <= 0 ||
      n_q_heads % n_kv_heads != 0 || (head_dim != 64 && head_dim != 128))
    return 0;
  return tg::attn_bwd_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim);
}

tg_status tg_gated_attn_bwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            const float* key_score, const float* gain, const float* tau,
                            const float* out_f32, const float* lse, const tg_bf16* dout,
                            tg_bf16* dq, tg_bf16* dk, tg_bf16* dv, float* dscore, float* dgain,
                            float* dtau, void* workspace, size_t workspace_bytes,
                            tg_stream_t stream) {
  const char* fn = "tg_gated_attn_bwd";
  const float* out = out_f32;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(TG_E_INVALID, "%s: n=%lld out of range", fn, (long long)n);
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
    return fail(TG_E_INVALID, "%s: n_q_heads=%d, n_kv_heads=%d", fn, n_q_heads, n_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(TG_E_UNSUPPORTED, "%s: head_dim=%d (supported: 64, 128)", fn, head_dim);
  if (n * n_q_heads * head_dim * 2 >= (int64_t(1) << 31))
    return fail(TG_E_UNSUPPORTED, "%s: n=%lld rows of %d heads x %d exceed 2^31 bytes", fn,
                (long long)n, n_q_heads, head_dim);
  if (n == 0) return TG_OK;
  if (!q || !k || !v || !out || !dout || !dq || !dk || !dv)
    return fail(TG_E_INVALID, "%s: null tensor pointer", fn);
  if (!key_score || !gain || !tau || !lse || !dscore || !dgain || !dtau)
    return fail(TG_E_INVALID, "%s: null key_score/gain/tau/lse/dscore/dgain/dtau", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(TG_E_INVALID, "%s: q/k/v/out_f32/dout/dq/dk/dv must be 16-byte aligned", fn);
  const size_t need = tg::attn_bwd_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(TG_E_WORKSPACE, "%s: workspace %p of %zu bytes (need %zu, 16-byte aligned)", fn,
                workspace, workspace_bytes, need);
  return hip_status(tg::launch_attn_bwd(q, k, v, n, n_q_heads, n_kv_heads, head_dim, key_score,
                                        gain, tau, out, lse, dout, dq, dk, dv, dscore, dgain, dtau,
                                        workspace, as_hip(stream)),
                    "tg_gated_attn_bwd launch");
}

namespace {
bool gdn_shape_ok(int64_t n, int32_t hk, int32_t hv, int32_t d) {
  return n >= 0 && n < (int64_t(1) << 31) && hk > 0 && hv > 0 && hv % hk == 0 && d == 128 &&
         n * hv * d * 2 < (int64_t(1) << 31);
}
}  // namespace

size_t tg_gdn_workspace_bytes(int64_t n, int32_t n_qk_heads, int32_t n_v_heads, int32_t head_dim) {
  if (n <= 0 || !gdn_shape_ok(n, n_qk_heads, n_v_heads, head_dim)) return 0;
  return tg::gdn_workspace_bytes(n, n_qk_heads, n_v_heads);
}

tg_status tg_gdn_fwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* g,
                     const float* beta, int64_t n, int32_t n_qk_heads, int32_t n_v_heads,
                     int32_t head_dim, float scale, const float* initial_state, float* final_state,
                     tg_bf16* out, void* workspace, size_t workspace_bytes, tg_stream_t stream) {
  const char* fn = "tg_gdn_fwd";
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(TG_E_INVALID, "%s: n=%lld out of range", fn, (long long)n);
  if (n_qk_heads <= 0 || n_v_heads <= 0 || n_v_heads % n_qk_heads != 0)
    return fail(TG_E_INVALID, "%s: n_qk_heads=%d, n_v_heads=%d (need a positive multiple)", fn,
                n_qk_heads, n_v_heads);
  if (head_dim != 128) return fail(TG_E_UNSUPPORTED, "%s: head_dim=%d (supported: 128)", fn, head_dim);
  if (n * n_v_heads * head_dim * 2 >= (int64_t(1) << 31))
    return fail(TG_E_UNSUPPORTED, "%s: n=%lld rows of %d value heads x %d exceed 2^31 bytes", fn,
                (long long)n, n_v_heads, head_dim);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(TG_E_INVALID, "%s: scale must be finite", fn);
  if (n == 0) return TG_OK;
  if (!q || !k || !v || !g || !beta || !out) return fail(TG_E_INVALID, "%s: null tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return fail(TG_E_INVALID, "%s: q/k/v/out/states must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(g) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return fail(TG_E_INVALID, "%s: g/beta must be 4-byte aligned", fn);
  const size_t need = tg::gdn_workspace_bytes(n, n_qk_heads, n_v_heads);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(TG_E_WORKSPACE, "%s: workspace %p of %zu bytes (need %zu, 16-byte aligned)", fn,
                workspace, workspace_bytes, need);
  return hip_status(tg::launch_gdn_fwd(q, k, v, g, beta, n, n_qk_heads, n_v_heads, scale,
                                       initial_state, final_state, out, workspace, as_hip(stream)),
                    "tg_gdn_fwd launch");
}

namespace {
bool decode_shape_ok(int64_t n, int32_t hq, int32_t hkv, int32_t d) {
  if (n <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return false;
  const int32_t g = hq / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  if (d != 64 && d != 128) return false;
  return n * hkv * d * 2 < (int64_t(1) << 31);
}
}  // namespace

size_t tg_decode_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  if (!decode_shape_ok(n, n_q_heads, n_kv_heads, head_dim)) return 0;
  return tg::decode_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim);
}

tg_status tg_gated_decode_fwd(const tg_bf16* q, const tg_bf16* k_cache, const tg_bf16* v_cache,
                              int64_t n, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              const float* key_score, const float* gain, const float* tau,
                              tg_bf16* out, float* lse, void* workspace, size_t workspace_bytes,
                              tg_stream_t stream) {
  const char* fn = "tg_gated_decode_fwd";
  if (n <= 0 || n >= (int64_t(1) << 31))
    return fail(TG_E_INVALID, "%s: n=%lld out of range (n >= 1 cached rows)", fn, (long long)n);
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
    return fail(TG_E_INVALID, "%s: n_q_heads=%d, n_kv_heads=%d", fn, n_q_heads, n_kv_heads);
  if (!decode_shape_ok(n, n_q_heads, n_kv_heads, head_dim))
    return fail(TG_E_UNSUPPORTED,
                "%s: head_dim=%d, group %d, n=%lld (need head_dim 64/128, group 1/2/4/8, "
                "n * n_kv_heads * head_dim * 2 < 2^31)",
                fn, head_dim, n_q_heads / n_kv_heads, (long long)n);
  if (!q || !k_cache || !v_cache || !out) return fail(TG_E_INVALID, "%s: null tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(TG_E_INVALID, "%s: q/k/v/out must be 16-byte aligned", fn);
  const int nb = (key_score != nullptr) + (gain != nullptr) + (tau != nullptr);
  if (nb != 0 && nb != 3)
    return fail(TG_E_INVALID, "%s: key_score, gain and tau must all be given or all be NULL", fn);
  const size_t need = tg::decode_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(TG_E_WORKSPACE, "%s: workspace %p of %zu bytes (need %zu, 16-byte aligned)", fn,
                workspace, workspace_bytes, need);
  return hip_status(tg::launch_decode(q, k_cache, v_cache, n, n_q_heads, n_kv_heads, head_dim,
                                      key_score, gain, tau, out, lse, workspace, as_hip(stream)),
                    "tg_gated_decode_fwd launch");
}

tg_status tg_qk_norm_rope(const tg_bf16* src, int64_t src_rows, const int32_t* rows,
                          const int32_t* positions, int64_t n, int32_t n_heads, int32_t head_dim,
                          const float* norm_weight, float eps, double rope_theta, tg_bf16* dst,
                          tg_stream_t stream) {
  const char* fn = "tg_qk_norm_rope";
  if (n < 0 || n >= (int64_t(1) << 31) || src_rows < 0)
    return fail(TG_E_INVALID, "%s: n=%lld, src_rows=%lld", fn, (long long)n, (long long)src_rows);
  if (n_heads <= 0) return fail(TG_E_INVALID, "%s: n_heads=%d", fn, n_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(TG_E_UNSUPPORTED, "%s: head_dim=%d (supported: 64, 128)", fn, head_dim);
  if (!(rope_theta > 0.0) || !(eps >= 0.f))
    return fail(TG_E_INVALID, "%s: rope_theta=%g, eps=%g", fn, rope_theta, (double)eps);
  if (rows == nullptr && n > src_rows)
    return fail(TG_E_INVALID, "%s: n=%lld rows > src_rows=%lld without a row index", fn,
                (long long)n, (long long)src_rows);
  if (n == 0) return TG_OK;
  if (!src || !dst || !positions) return fail(TG_E_INVALID, "%s: null pointer", fn);
  if (!aligned16(src) || !aligned16(dst)) return fail(TG_E_INVALID, "%s: src/dst must be 16-byte aligned", fn);
  const int64_t row = int64_t(n_heads) * head_dim * 2;
  const char* s0 = reinterpret_cast<const char*>(src);
  const char* d0 = reinterpret_cast<const char*>(dst);
  const bool in_place = rows == nullptr && s0 == d0;
  if (!in_place && s0 < d0 + n * row && d0 < s0 + src_rows * row)
    return fail(TG_E_INVALID, "%s: src and dst overlap (only exact in-place without rows)", fn);
  return hip_status(tg::launch_qk_norm_rope(src, src_rows, rows, positions, n, n_heads, head_dim,
                                            norm_weight, eps, rope_theta, dst, as_hip(stream)),
                    "tg_qk_norm_rope launch");
}

}  // extern "C"
