/*
 * tg.h -- C ABI of the TokenGate gated-prefill kernels for MI355X (gfx950).
 *
 * The path these calls implement (coverage pages of the method, cited by
 * title and section):
 *   - lucasainews.com, Korean TokenGate article, section "작동 방식" (how it
 *     works): below the gate layer every token is processed; at the gate
 *     layer a small MLP scores each token from its post-attention residual and
 *     a top-K selector keeps only the best-scoring ones; the layers above see
 *     only the kept tokens and build no KV entries for the dropped ones; only
 *     the document part of the prompt is pruned, the question stays whole.
 *     The same section says the kept tokens' scores enter the attention
 *     logits above the gate as a bias, with a learned gain and temperature per
 *     head.  Section "사용법과 비용" (usage and cost): the document is marked
 *     in the prompt and the caller passes a budget of kept prefill tokens.
 *   - fugumt.com, "論文の概要: TokenGate: Adapting LLMs for Fast and
 *     Memory-Efficient Prefill with Learned Token Pruning", English abstract:
 *     above the gate, each kept key's gate score enters the attention
 *     logits as an additive bias.
 *
 * Readings fixed here where the pages are silent:
 *   - logit_ij = q_i.k_j / (sqrt(d) * tau_h) + gain_h * s_j (s_j raw score);
 *   - selection compares float32 scores in a total order: -0.0 == +0.0,
 *     NaN below -inf, ties to the lower index;
 *   - kept rows stay in ascending original order and keep their original
 *     rotary positions (applied to q/k by the caller).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless stated; the caller allocates and
 *     frees them.  The library never allocates, never synchronises the stream
 *     and keeps no global mutable state besides a thread-local error text.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; 0 = the
 *     null stream).  Inputs must stay valid until the work completes.
 *   - Arguments are validated on the host before any launch.  On a non-OK
 *     return nothing was launched (except TG_E_HIP, reported by the launch
 *     itself) and outputs are undefined; tg_last_error() gives the detail.
 *   - bf16 tensors are passed as tg_bf16 (the raw 16-bit pattern).
 *   - Row-major tensors must be 16-byte aligned where stated.
 */
#ifndef TG_H_
#define TG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same underlying type as hipStream_t, so a hipStream_t can be passed as is. */
typedef struct ihipStream_t* tg_stream_t;

/* bfloat16 bit pattern. */
typedef uint16_t tg_bf16;

typedef enum tg_status {
  TG_OK = 0,
  TG_E_INVALID = 1,     /* bad pointer, size, range or alignment            */
  TG_E_UNSUPPORTED = 2, /* valid request outside the shapes the kernels take */
  TG_E_WORKSPACE = 3,   /* workspace missing or smaller than required        */
  TG_E_HIP = 4          /* the HIP runtime reported an error at launch       */
} tg_status;

/* Static description of a status code. */
const char* tg_status_str(tg_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* tg_last_error(void);

/*
 * Number of rows that survive selection: min(k_doc, N_doc) + (n - N_doc),
 * N_doc = doc_end - doc_begin.  Host-only arithmetic (lucasainews.com
 * article, "작동 방식": document tokens are pruned to the budget, the rest is
 * kept).  Returns -1 if 0 <= doc_begin <= doc_end <= n and k_doc >= 0 do not
 * hold.
 */
int64_t tg_kept_count(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k_doc);

/*
 * Gate MLP score of every row (lucasainews.com article, "작동 방식"; a small
 * MLP scores each token from its post-attention residual):
 *     scores[i] = sum_u w2[u] * GELU(sum_c w1[u, c] * h[i, c] + b1[u]) + b2
 * with the exact (erf) GELU, bf16 products accumulated in fp32.
 *   h        [n, hidden] bf16, row stride ld_h elements (ld_h >= hidden,
 *            ld_h % 8 == 0, 16-byte aligned)
 *   w1       [gate_hidden, hidden] bf16, contiguous, 16-byte aligned
 *   b1, w2   [gate_hidden] fp32
 *   scores   [n] fp32 (output)
 * Supported: hidden % 64 == 0, gate_hidden <= 512.
 * n == 0 is a no-op.  Deterministic: identical inputs give identical bits.
 */
tg_status tg_gate_score(const tg_bf16* h, int64_t n, int64_t ld_h, int32_t hidden,
                        const tg_bf16* w1, const float* b1, const float* w2, float b2,
                        int32_t gate_hidden, float* scores, tg_stream_t stream);

/*
 * Bytes of device workspace tg_topk_select needs for n scores: three digit
 * histograms (20 KiB), the selection state and two counters per range of
 * rows (at most 1024 ranges): under 29 KiB for any n.  Host-only
 * arithmetic; 0 for n <= 0 or n >= 2^30.
 */
size_t tg_topk_workspace_bytes(int64_t n);

/*
 * Top-K selection over the document rows [doc_begin, doc_end) with every
 * other row kept (lucasainews.com article, "작동 방식": only the document is
 * pruned, the question stays; "사용법과 비용": the budget is a token count).
 * Document rows are ranked by score (total order above, ties to the lower
 * index) and the first min(k_doc, N_doc) are kept.
 *   scores    [n] fp32
 *   kept_idx  [tg_kept_count(n, doc_begin, doc_end, k_doc)] int32 (output),
 *             strictly ascending original row indices (they double as the
 *             rows' position ids); may be NULL when that count is 0
 *   workspace device scratch of at least tg_topk_workspace_bytes(n) bytes,
 *             16-byte aligned, owned by the caller; overwritten, carries
 *             nothing between calls; calls sharing one must be ordered on one
 *             stream.  Too small or NULL -> TG_E_WORKSPACE.
 * Exact: the result is unique and reproduced bit for bit (the global
 * histograms are integer sums, independent of the order of their atomics).
 * n < 2^30 (else TG_E_INVALID).
 */
tg_status tg_topk_select(const float* scores, int64_t n, int64_t doc_begin, int64_t doc_end,
                         int64_t k_doc, int32_t* kept_idx, void* workspace,
                         size_t workspace_bytes, tg_stream_t stream);

/*
 * tg_topk_select that also gathers the kept rows' scores in the same pass
 * (lucasainews.com article, "작동 방식": the kept tokens' scores are the
 * bias the layers above the gate take):
 *   kept_scores [tg_kept_count(...)] fp32 (output): kept_scores[i] =
 *               scores[kept_idx[i]], bit for bit; NULL when that count is
 *               positive -> TG_E_INVALID
 * Every other argument, the result in kept_idx and the errors are those of
 * tg_topk_select.  Saves the compaction of the scores (a launch and a pass
 * over the kept indices).
 */
tg_status tg_topk_select_scores(const float* scores, int64_t n, int64_t doc_begin,
                                int64_t doc_end, int64_t k_doc, int32_t* kept_idx,
                                float* kept_scores, void* workspace, size_t workspace_bytes,
                                tg_stream_t stream);

/*
 * tg_topk_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same selection, arguments and result, with no workspace argument.
 * Its scratch is a static device array of 32 KiB inside the library, one per
 * GPU, held until the process ends; it covers every n < 2^30 (a larger need
 * would return TG_E_UNSUPPORTED).  The call allocates and frees nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or threads without ordering) race and give
 * undefined results.  The calling thread's current device must be the one
 * `stream` belongs to.  Errors as tg_topk_select (no TG_E_WORKSPACE).
 */
tg_status tg_topk_select_noalloc(const float* scores, int64_t n, int64_t doc_begin,
                                 int64_t doc_end, int64_t k_doc, int32_t* kept_idx,
                                 tg_stream_t stream);

/*
 * Row compaction (lucasainews.com article, "작동 방식": only kept rows go
 * up; nothing is built for the dropped ones):
 *     dst[i, :] = src[kept_idx[i], :]   for i < n_kept, bytewise
 *   kept_idx  [n_kept] int32; entries outside [0, src_rows) are skipped (that
 *             dst row is left unwritten)
 *   src       src_rows rows of row_bytes, stride src_stride_bytes
 *   dst       n_kept rows of row_bytes, stride dst_stride_bytes
 * Strides must be >= row_bytes; src and dst must not overlap.  Rows whose
 * bytes, strides and base pointers are multiples of 16 (else 4) move with
 * 16-byte (else 4-byte, else 1-byte) accesses.
 */
tg_status tg_compact(const int32_t* kept_idx, int64_t n_kept, const void* src, int64_t src_rows,
                     int64_t src_stride_bytes, int64_t row_bytes, void* dst,
                     int64_t dst_stride_bytes, tg_stream_t stream);

/*
 * Bytes of device workspace tg_gated_attn_fwd / tg_full_attn_fwd need for n
 * rows (enough for either):
 *   - per KV head and 64-key tile, a packed copy of V (fp16, transposed,
 *     laid out as the kernel's LDS image: about 1.1x the bytes of V) and, per
 *     query head and key, the fp32 bias gain * sqrt(head_dim) * tau * score
 *     (K itself is read in place);
 *   - when n is short enough that long query blocks are split over several
 *     work-groups along the keys: one counter per split block and one
 *     partial state (fp16 output, fp32 max and sum; 34 KiB at head_dim 128)
 *     per split work-group.
 * Host-only arithmetic; 0 for n <= 0 or unsupported heads / head_dim.
 */
size_t tg_attn_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim);

/*
 * Token-gated causal GQA attention over the n kept rows (lucasainews.com
 * article, "작동 방식": each kept token's score is added to the attention
 * logits above the gate, scaled by a per-head learned gain, with a per-head
 * temperature; fugumt.com abstract: the kept keys' gate scores bias the
 * logits):
 *     logit_ij = q_i,h . k_j,g / (sqrt(head_dim) * tau[h]) + gain[h] * key_score[j]
 *     out_i,h  = sum_{j <= i} softmax_j(logit_i,h) v_j,g,   g = h / (n_q_heads / n_kv_heads)
 * Causality is by row order (kept rows are in original order).
 *   q    [n, n_q_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   k, v [n, n_kv_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   key_score [n] fp32; gain, tau [n_q_heads] fp32 (tau > 0)
 *   out  [n, n_q_heads, head_dim] bf16 (output, round-to-nearest-even)
 *   lse  [n_q_heads, n] fp32 natural-log log-sum-exp of the logits
 *        (output; may be NULL)
 *   workspace  device scratch of at least tg_attn_workspace_bytes(n, ...)
 *        bytes, 16-byte aligned, owned by the caller; its contents are
 *        overwritten and carry nothing between calls.  Calls that share one
 *        workspace must be ordered on one stream.  Too small -> TG_E_WORKSPACE.
 * Supported: head_dim in {64, 128}, n_q_heads % n_kv_heads == 0,
 * n * n_q_heads * head_dim * 2 < 2^31 (byte offsets fit 31 bits).
 * Numerics: q.k as bf16 products with fp32 accumulation, starting from the
 * fp32 bias gain * sqrt(head_dim) * tau * key_score; softmax in fp32;
 * probabilities and v rounded to fp16 for the p.v product (v magnitudes above
 * 65504 saturate), fp32 accumulation; where a query block is split along the
 * keys, each part's normalised output is rounded to fp16 before the merge.
 * n == 0 is a no-op.
 */
tg_status tg_gated_attn_fwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            const float* key_score, const float* gain, const float* tau,
                            tg_bf16* out, float* lse, void* workspace, size_t workspace_bytes,
                            tg_stream_t stream);

/*
 * tg_gated_attn_fwd for a training step (lucasainews.com article, "작동 방식":
 * the gate is trained through the score bias above it): the same
 * computation, layouts, limits and workspace, and in addition
 *   lse     [n_q_heads, n] fp32 (required here)
 *   out_f32 [n, n_q_heads, head_dim] fp32, 16-byte aligned: the output before
 *           its bf16 rounding, which tg_gated_attn_bwd takes (output)
 * NULL lse or out_f32 -> TG_E_INVALID.  n == 0 is a no-op.
 */
tg_status tg_gated_attn_fwd_train(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                                  int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                  const float* key_score, const float* gain, const float* tau,
                                  tg_bf16* out, float* lse, float* out_f32, void* workspace,
                                  size_t workspace_bytes, tg_stream_t stream);

/*
 * Unpruned causal GQA attention over all n rows, softmax(q.k / sqrt(d)) v:
 * the full prefill that the pages' speed-ups are measured against
 * (lucasainews.com article, lede and "성능 결과").  Same layouts, limits,
 * workspace and numerics as tg_gated_attn_fwd with gain = 0 and tau = 1.
 */
tg_status tg_full_attn_fwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           tg_bf16* out, float* lse, void* workspace, size_t workspace_bytes,
                           tg_stream_t stream);

/*
 * Bytes of device workspace tg_gated_attn_bwd needs for n rows: per row and
 * query head its log-sum-exp and dout.out, per query head and key the column
 * sum of the logit gradient, fp32 per-query-head dk and dv partials
 * (2 * 4 * n * n_q_heads * head_dim bytes) and a few floats per query head
 * and 128-row block.  For short n, where the causal walks are split over
 * several work-groups, the column sums and partials are held per split
 * chunk (up to ~3x at 2304 rows) and fp32 dq partials are added.
 * Host-only arithmetic; 0 for arguments tg_gated_attn_bwd would reject as
 * invalid or unsupported (n <= 0 included).
 */
size_t tg_attn_bwd_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim);

/*
 * Backward of tg_gated_attn_fwd: the gradients through which a training loss
 * reaches the gate's scores, gains and temperatures (lucasainews.com
 * article, "작동 방식": the score is a bias on the logits of the layers above
 * the gate, with a learned per-head gain and temperature; fugumt.com
 * abstract).  With c_h = 1 / (sqrt(head_dim) * tau[h]), P the causal softmax
 * of logit_ij = c_h q_i.k_j + gain[h] key_score[j] and dS_ij = P_ij (dout_i.v_j
 * - dout_i.out_i):
 *     dq_i = c_h sum_j dS_ij k_j          dk_j = sum_h c_h sum_i dS_ij q_i
 *     dv_j = sum_h sum_i P_ij dout_i      dscore_j = sum_h gain[h] sum_i dS_ij
 *     dgain[h] = sum_ij dS_ij key_score[j]
 *     dtau[h]  = -(1 / tau[h]) sum_i q_i.dq_i     (sums over i, j within head h)
 *   q, k, v, key_score, gain, tau  as given to tg_gated_attn_fwd_train
 *   out_f32 [n, n_q_heads, head_dim] fp32: that call's output before rounding
 *         (D_i = dout_i.out_i is formed from it: from the bf16 output, rows
 *         with few keys, whose dS terms nearly cancel against D, would lose
 *         most of their precision)
 *   lse   [n_q_heads, n] fp32: that call's natural-log log-sum-exp
 *   dout  [n, n_q_heads, head_dim] bf16: gradient of the loss w.r.t. out
 *   dq    [n, n_q_heads, head_dim], dk, dv [n, n_kv_heads, head_dim] bf16
 *         (outputs, round-to-nearest-even; no overlap with the inputs)
 *   dscore [n], dgain [n_q_heads], dtau [n_q_heads] fp32 (outputs, overwritten)
 *   workspace  device scratch of at least tg_attn_bwd_workspace_bytes(...)
 *         bytes, 16-byte aligned, caller-owned; overwritten.
 * Every pointer is required (TG_E_INVALID); tensors 16-byte aligned.
 * Supported: head_dim in {64, 128}, n * n_q_heads * head_dim * 2 < 2^31.
 * Numerics: bf16 MFMA products with fp32 accumulation; P and dS enter the
 * dv, dk and dq products as bf16; softmax, dS and every reduction in fp32, in
 * a fixed order (deterministic).  n == 0 is a no-op (nothing written).
 */
tg_status tg_gated_attn_bwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, int64_t n,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            const float* key_score, const float* gain, const float* tau,
                            const float* out_f32, const float* lse, const tg_bf16* dout,
                            tg_bf16* dq, tg_bf16* dk, tg_bf16* dv, float* dscore, float* dgain,
                            float* dtau, void* workspace, size_t workspace_bytes,
                            tg_stream_t stream);

/*
 * Bytes of device workspace tg_gdn_fwd needs for n rows: per 64-row chunk and
 * value head 72.25 KiB (the recurrence's operands as fp16 MFMA fragments and
 * the chunk's decay), plus 64 KiB per value head (the fp32 state handed from
 * one piece of the recurrence to the next: the layer runs in pieces of chunks,
 * each piece's recurrence beside the next piece's operand preparation).
 * Host-only arithmetic; 0 for n <= 0 or unsupported shapes.
 */
size_t tg_gdn_workspace_bytes(int64_t n, int32_t n_qk_heads, int32_t n_v_heads, int32_t head_dim);

/*
 * A Gated DeltaNet layer's recurrence over the n kept rows (lucasainews.com
 * article, "성능 결과": on a hybrid model with Gated DeltaNet layers between
 * full-attention layers, TokenGate prunes the recurrent layers too, so above
 * the gate they run over the kept tokens only, in original order; the
 * recurrence is the gated delta rule of Gated DeltaNet, Yang, Kautz and
 * Hatamizadeh, ICLR 2025).  Per value head h, with q/k head h / (n_v_heads /
 * n_qk_heads) and state S [head_dim (v), head_dim (k)]:
 *     S <- exp(g[t,h]) S
 *     S <- S + beta[t,h] (v_t,h - S k_t) k_t^T
 *     out_t,h = scale * S q_t
 *   q, k  [n, n_qk_heads, head_dim] bf16, contiguous, 16-byte aligned; the
 *         layer's L2-normalised queries and keys
 *   v     [n, n_v_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   g     [n, n_v_heads] fp32 log decay (exp(g) <= 1 expected; g <= 0)
 *   beta  [n, n_v_heads] fp32 write strength in [0, 1]
 *   scale the read-out scale (1/sqrt(head_dim) in the usual layer); finite
 *   initial_state [n_v_heads, head_dim, head_dim] fp32 or NULL (zeros)
 *   final_state   [n_v_heads, head_dim, head_dim] fp32 or NULL (output)
 *   out   [n, n_v_heads, head_dim] bf16 (output, round-to-nearest-even)
 *   workspace  device scratch of at least tg_gdn_workspace_bytes(...) bytes,
 *         16-byte aligned, caller-owned, overwritten.
 * Supported: head_dim 128, n_v_heads % n_qk_heads == 0,
 * n * n_v_heads * head_dim * 2 < 2^31 (else TG_E_UNSUPPORTED).
 * Numerics: chunks of 64 rows; the within-chunk solve, decays, state and sums
 * in fp32, the MFMA operands in fp16.  n == 0 is a no-op (final_state not
 * written).
 */
tg_status tg_gdn_fwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* g,
                     const float* beta, int64_t n, int32_t n_qk_heads, int32_t n_v_heads,
                     int32_t head_dim, float scale, const float* initial_state, float* final_state,
                     tg_bf16* out, void* workspace, size_t workspace_bytes, tg_stream_t stream);

/*
 * Bytes of device workspace tg_gated_decode_fwd needs for n cached rows:
 * per KV head and chunk of 64-256 keys, a (max, sum, head_dim outputs) fp32
 * state for each of its query heads.  Host-only arithmetic; 0 for arguments
 * tg_gated_decode_fwd would reject as invalid or unsupported.
 */
size_t tg_decode_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim);

/*
 * One decode step over the pruned KV cache (lucasainews.com article, lede:
 * the gains are in time to first token; "작동 방식": above the gate only the
 * kept tokens have KV entries, and their scores bias the logits there with a
 * per-head gain and temperature).  One new query row per head against every
 * cached row (the kept rows plus the new token's own row, appended by the
 * caller, so no key is masked):
 *     logit_j = q_h . k_j,g / (sqrt(head_dim) * tau[h]) + gain[h] * key_score[j]
 *     out_h   = sum_j softmax_j(logit) v_j,g,   g = h / (n_q_heads / n_kv_heads)
 *   q        [n_q_heads, head_dim] bf16, 16-byte aligned
 *   k_cache, v_cache [n, n_kv_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   key_score [n], gain, tau [n_q_heads] fp32: all three given (gated, the
 *            layers above the gate) or all three NULL (plain softmax(q.k/sqrt(d)),
 *            the gate layer's decode over all rows); else TG_E_INVALID
 *   out      [n_q_heads, head_dim] bf16 (output, round-to-nearest-even)
 *   lse      [n_q_heads] fp32 natural-log log-sum-exp (output; may be NULL)
 *   workspace device scratch of at least tg_decode_workspace_bytes(...) bytes,
 *            16-byte aligned, caller-owned; overwritten; calls sharing one
 *            must be ordered on one stream.  Too small -> TG_E_WORKSPACE.
 * Supported: head_dim in {64, 128}, n_q_heads / n_kv_heads in {1, 2, 4, 8},
 * n * n_kv_heads * head_dim * 2 < 2^31.  n must be >= 1 (TG_E_INVALID).
 * Numerics: bf16 inputs, fp32 dot products, softmax and P.V; deterministic.
 */
tg_status tg_gated_decode_fwd(const tg_bf16* q, const tg_bf16* k_cache, const tg_bf16* v_cache,
                              int64_t n, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              const float* key_score, const float* gain, const float* tau,
                              tg_bf16* out, float* lse, void* workspace, size_t workspace_bytes,
                              tg_stream_t stream);

/*
 * Query/key prologue of the layers above the gate, fused with the row gather
 * (lucasainews.com article, "작동 방식": the kept tokens go up as the tokens
 * they are, so their rotary positions are their original indices; the
 * normalisation and rotation themselves are Qwen3's, not the method's):
 *     y = x / sqrt(mean_f x_f^2 + eps) * norm_weight       (per head vector)
 *     a_f = positions[i] * rope_theta^(-2 f / head_dim),   f < head_dim / 2
 *     dst[i, h, f]     = y_f cos a_f - y_{f+d/2} sin a_f
 *     dst[i, h, f+d/2] = y_{f+d/2} cos a_f + y_f sin a_f
 * with x = src[rows[i], h, :] (rows may be NULL: x = src[i, h, :]).
 *   src        [src_rows, n_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   rows       [n] int32 or NULL; entries outside [0, src_rows) skip the
 *              row (dst row left unwritten)
 *   positions  [n] int32 rotary positions
 *   norm_weight [head_dim] fp32, or NULL for no normalisation
 *   dst        [n, n_heads, head_dim] bf16 (output); may equal src only when
 *              rows is NULL (in place); any other overlap -> TG_E_INVALID
 * Supported: head_dim in {64, 128}.  Angles are formed in fp64 (positions up
 * to 2^31 keep their phase); the rest is fp32, output rounded to nearest even.
 * n == 0 is a no-op.
 */
tg_status tg_qk_norm_rope(const tg_bf16* src, int64_t src_rows, const int32_t* rows,
                          const int32_t* positions, int64_t n, int32_t n_heads, int32_t head_dim,
                          const float* norm_weight, float eps, double rope_theta, tg_bf16* dst,
                          tg_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TG_H_ */
