// Internal launchers (host side).  Arguments arrive here already validated by
// the C ABI layer; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

hipError_t launch_gate_score(const uint16_t* h, int64_t n, int64_t ld_h, int hidden,
                             const uint16_t* w1, const float* b1, const float* w2, float b2,
                             int gate_hidden, float* scores, hipStream_t stream);

// Bytes of workspace the top-K launch needs for n scores.
size_t topk_workspace_bytes(int64_t n);

// kept_scores may be null; else kept_scores[i] = scores[kept_idx[i]], bit for bit
hipError_t launch_topk_select(const float* scores, int64_t n, int64_t doc_begin, int64_t doc_end,
                              int64_t k_doc, int32_t* kept_idx, float* kept_scores,
                              void* workspace, hipStream_t stream);

// The top-K with the library's own per-device static scratch (no allocation).
constexpr size_t kTopkScratchBytes = 32768;
hipError_t launch_topk_select_noalloc(const float* scores, int64_t n, int64_t doc_begin,
                                      int64_t doc_end, int64_t k_doc, int32_t* kept_idx,
                                      hipStream_t stream);

hipError_t launch_compact(const int32_t* kept_idx, int64_t n_kept, const void* src,
                          int64_t src_rows, int64_t src_stride, int64_t row_bytes, void* dst,
                          int64_t dst_stride, hipStream_t stream);

// Bytes of workspace the attention launch needs: the packed V^T tile images,
// (gated) the per-key bias fragments, and the split chunks' partial states.
size_t attn_workspace_bytes(int64_t n, int n_q_heads, int n_kv_heads, int head_dim, bool gated);

// Bytes of the tile images of one KV head (addressed with 32-bit offsets).
size_t attn_image_bytes_per_kv_head(int64_t n, int head_dim, bool gated);

// gain == nullptr selects the unbiased (full-prefill) kernel with tau = 1.
// out32 (nullable) also receives the fp32 output before its bf16 rounding.
// `workspace` holds attn_workspace_bytes(n, n_q_heads, n_kv_heads, head_dim, gated) bytes.
hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                           int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                           const float* gain, const float* tau, uint16_t* out, float* lse,
                           float* out32, void* workspace, hipStream_t stream);

// Bytes of workspace the attention backward needs: per-row (lse, D), per-head
// key column sums of dS, fp32 per-head dK and dV partials (per split chunk),
// per-work-group gain and q.dq sums, fp32 dQ partials when dQ walks split.
size_t attn_bwd_workspace_bytes(int64_t n, int n_q_heads, int n_kv_heads, int head_dim);

// Gradients of the token-gated attention given its fp32 output, its
// natural-log lse and dout.  `workspace` holds attn_bwd_workspace_bytes(...) bytes.
hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                           int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                           const float* gain, const float* tau, const float* out,
                           const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk,
                           uint16_t* dv, float* dscore, float* dgain, float* dtau,
                           void* workspace, hipStream_t stream);

// Bytes of workspace one decode call needs (the per-chunk partial states).
size_t decode_workspace_bytes(int64_t n, int n_q_heads, int n_kv_heads, int head_dim);

// gain == nullptr selects plain attention (no bias, tau = 1).
hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                         int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                         const float* gain, const float* tau, uint16_t* out, float* lse,
                         void* workspace, hipStream_t stream);

// dst[i] = RoPE(RMSNorm(src[rows ? rows[i] : i]) * w) at pos[i]; w == nullptr skips the norm.
hipError_t launch_qk_norm_rope(const uint16_t* src, int64_t src_rows, const int32_t* rows,
                               const int32_t* pos, int64_t n, int n_heads, int head_dim,
                               const float* norm_weight, float eps, double theta, uint16_t* dst,
                               hipStream_t stream);

// Bytes of workspace the Gated DeltaNet launch needs for n rows (head_dim 128):
// per 64-row chunk and value head the prep pass's fp16 operand fragments and
// cumulative decays, per chunk and q/k head the q fragments.
size_t gdn_workspace_bytes(int64_t n, int n_qk_heads, int n_v_heads);

// Gated delta rule over n rows (head_dim 128); initial_state / final_state
// [n_v_heads, 128, 128] fp32 are optional.
hipError_t launch_gdn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                          const float* beta, int64_t n, int n_qk_heads, int n_v_heads, float scale,
                          const float* initial_state, float* final_state, uint16_t* out,
                          void* workspace, hipStream_t stream);

}  // namespace tg
