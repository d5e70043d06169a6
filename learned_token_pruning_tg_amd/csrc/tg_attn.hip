// Token-gated causal GQA attention (forward) for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"; fugumt.com
// abstract): above the gate layer each kept key's gate score is added to the
// attention logits, scaled by a per-head gain, and a per-head temperature
// rescales q.k.  Read here as
//     logit_ij = q_i.k_j / (sqrt(d) * tau_h) + gain_h * s_j ,   j <= i.
// With gain = 0 and tau = 1 the same kernel is plain causal attention, the
// unpruned baseline.
//
// Design (flash-style; one work-group = 128 query rows of one query head,
// four waves of 32 rows each):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K tile from LDS, B = Q held
//    in registers): each lane owns one query column and 16 keys of each
//    32-key block, so the online-softmax statistics are lane-local plus one
//    exchange between lane halves.
//  * O^T = V^T P^T on v_mfma_f32_32x32x16_f16 takes the probabilities straight
//    from registers as the B operand.  P and V are fp16 for this product:
//    bf16 P (8-bit mantissa) costs up to ~3e-3 of output error on peaked
//    rows, on top of the bf16 output rounding; fp16 P is 4x finer.  V is
//    converted bf16 -> fp16 (exact in fp16's normal range) while it is
//    transposed into LDS; the key order inside each 16-key group is permuted
//    so each lane's eight keys are one 16-byte LDS read.
//  * Scores are pre-multiplied by gain_h * log2(e) when staged into LDS; the
//    temperature and 1/sqrt(d) are folded with log2(e) into one scale, so a
//    logit costs one FMA before the exp2-based online softmax.  The running
//    max is only moved when a tile raises it by more than 2^8 (lazy
//    rescaling): probabilities stay <= 256, exact in fp16's range.
//  * Software pipeline, one barrier per 64-key tile: while tile j's softmax
//    and P.V run, S for tile j+1 is issued from the other LDS buffer and the
//    global loads of tile j+2 are in flight.  Loads are raw buffer loads whose
//    hardware range check returns zeros past the last row, so the loop has no
//    per-row guards.
//  * Causal masking is applied only on the (at most two) diagonal tiles of a
//    wave, and tiles entirely above a wave's rows are skipped.
//  * Work-groups: heads of one KV group are pinned to one XCD (work-groups are
//    dealt round-robin over the 8 XCDs) so that group's K/V stays in that
//    XCD's L2; within an XCD the longest (last) query tiles go first.
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kBM = 128;     // query rows per work-group
constexpr int kBN = 64;      // keys per tile
constexpr int kThreads = 512;    // two groups of four waves
constexpr float kRescaleThreshold = 8.f;  // log2 units

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

__device__ __forceinline__ floatx16 mfma_f16(f16x8 a, f16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two bf16 (one dword) -> two fp16 (one dword), round toward zero.  Exact for
// bf16 values in fp16's normal range; larger magnitudes saturate at 65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __uint_as_float(x << 16);
  const float hi = __uint_as_float(x & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

template <int D, bool kBias>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const _Float16* __restrict__ vt_pack,
    int M, int Hq, int Hkv, const float* __restrict__ key_score, const float* __restrict__ gain,
    const float* __restrict__ tau, bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int KSTEPS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;            // 32-row tiles of O^T
  constexpr int K_LD = D + 8;           // K row in LDS (bf16), padded by 16 B
  constexpr int VT_LD = kBN + 8;        // V^T row in LDS (fp16), padded by 16 B
  constexpr int CPR = D / 8;            // 16-byte chunks per K row
  constexpr int K_PER_T = 2 * kBN * CPR / kThreads;   // K chunks per thread per tile pair
  constexpr int V_PER_T = 2 * D * (kBN / 8) / kThreads;  // V^T chunks per thread per pair
  static_assert((2 * kBN * CPR) % kThreads == 0, "K tile split");
  static_assert((2 * D * (kBN / 8)) % kThreads == 0, "V tile split");

  // [step parity][wave group] tiles; the group-1 half of k_lds is reused for
  // the final merge of the two groups' partial results.
  __shared__ __align__(16) bf16 k_lds[2][2][kBN * K_LD];
  __shared__ __align__(16) _Float16 vt_lds[2][2][D * VT_LD];
  __shared__ __align__(16) float b_lds[2][2][kBN];

  // ---- work-group -> (query tile, head)
  const int n_qt = (M + kBM - 1) / kBM;
  int head, qt;
  {
    const int b = blockIdx.x;
    if ((Hq & 7) == 0) {
      const int hpx = Hq >> 3;            // heads per XCD
      const int xcd = b & 7, slot = b >> 3;
      head = xcd * hpx + slot % hpx;
      qt = n_qt - 1 - slot / hpx;
    } else {
      head = b % Hq;
      qt = n_qt - 1 - b / Hq;
    }
  }
  const int kvh = head / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int grp = wave >> 2;            // 0: even key tiles, 1: odd key tiles
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBM + (wave & 3) * 32;
  const int my_q = q0 + l32;

  const float t_h = kBias ? tau[head] : 1.f;
  const float alpha = kLog2e / (sqrtf(static_cast<float>(D)) * t_h);
  const float beta = kBias ? gain[head] * kLog2e : 0.f;

  const uint32_t q_row_bytes = static_cast<uint32_t>(Hq) * D * 2;
  const uint32_t kv_row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
  const uint32_t kv_tile_bytes = kv_row_bytes * kBN;
  const uint32_t kv_bytes = kv_row_bytes * static_cast<uint32_t>(M);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + static_cast<size_t>(head) * D, q_row_bytes * M);
  const char* k_base = reinterpret_cast<const char*>(k + static_cast<size_t>(kvh) * D);
  // Packed V^T of this KV head: n_tiles blocks of [D][kBN] fp16.
  const int n_tiles_all = (M + kBN - 1) / kBN;
  const uint32_t vt_tile_bytes = D * kBN * 2;
  const uint32_t vt_bytes = vt_tile_bytes * static_cast<uint32_t>(n_tiles_all);
  const char* v_base = reinterpret_cast<const char*>(vt_pack) +
                       static_cast<size_t>(kvh) * n_tiles_all * vt_tile_bytes;
  // Per-tile-pair descriptors: base moved to the pair's first row (scalar
  // work only), so the per-thread offsets are loop-invariant and the range
  // check still zero-fills rows >= M.
  auto pair_rsrc = [&](const char* base, int t0) __attribute__((always_inline)) {
    const uint32_t off = static_cast<uint32_t>(t0) * kv_tile_bytes;
    return make_rsrc(base + off, off < kv_bytes ? kv_bytes - off : 0u);
  };
  auto vt_rsrc = [&](int t0) __attribute__((always_inline)) {
    const uint32_t off = static_cast<uint32_t>(t0) * vt_tile_bytes;
    return make_rsrc(v_base + off, off < vt_bytes ? vt_bytes - off : 0u);
  };
  auto score_rsrc = [&](int t0) __attribute__((always_inline)) {
    const uint32_t off = static_cast<uint32_t>(t0) * kBN;
    return make_rsrc(key_score + off, off < static_cast<uint32_t>(M) ? 4u * (M - off) : 0u);
  };

  // Q fragments (B operand): lane holds Q[my_q][16 s + 8 hh .. + 7].
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = as_bf16x8(bload16(rq, static_cast<uint32_t>(my_q) * q_row_bytes + (16 * s + 8 * hh) * 2));

  floatx16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int q_last = min(qt * kBM + kBM, M) - 1;
  const int n_kt = q_last / kBN + 1;                  // key tiles of the work-group
  const int n_steps = (n_kt + 1) / 2;                 // tile pairs
  const int w_last = min(q0 + 31, q_last);            // last row this wave owns
  const int n_vis = q0 <= q_last ? w_last / kBN + 1 : 0;  // tiles this wave sees

  // ---- register staging of one tile pair
  u32x4 kreg[K_PER_T];
  u32x4 vreg[V_PER_T];
  float breg = 0.f;

  uint32_t k_off[K_PER_T];
#pragma unroll
  for (int p = 0; p < K_PER_T; ++p) {
    const int f = tid + p * kThreads;   // chunk index within the pair
    k_off[p] = static_cast<uint32_t>(f / CPR) * kv_row_bytes + 16 * (f % CPR);
  }

  auto load_k = [&](int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = pair_rsrc(k_base, t0);
#pragma unroll
    for (int p = 0; p < K_PER_T; ++p) kreg[p] = bload16(r, k_off[p]);
  };
  auto load_v = [&](int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = vt_rsrc(t0);
#pragma unroll
    for (int p = 0; p < V_PER_T; ++p) vreg[p] = bload16(r, 16u * (tid + p * kThreads));
    if (kBias && tid < 2 * kBN) breg = beta * bload4f(score_rsrc(t0), 4 * tid);
  };
  auto store_k = [&](int par) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < K_PER_T; ++p) {
      const int f = tid + p * kThreads;
      const int row = f / CPR;          // 0 .. 2 kBN - 1
      st16(&k_lds[par][row / kBN][(row % kBN) * K_LD + 8 * (f % CPR)], kreg[p]);
    }
  };
  auto store_v = [&](int par) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < V_PER_T; ++p) {
      const int f = tid + p * kThreads;          // 16-byte chunk within the pair
      const int tp = f / (D * kBN / 8), rem = f % (D * kBN / 8);
      st16(&vt_lds[par][tp][(rem / (kBN / 8)) * VT_LD + 8 * (rem % (kBN / 8))], vreg[p]);
    }
    if (kBias && tid < 2 * kBN) b_lds[par][tid / kBN][tid % kBN] = breg;
  };

  auto qk = [&](const bf16* kt_lds, floatx16* s) __attribute__((always_inline)) {
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 a = lds_bf16x8(&kt_lds[(32 * t + l32) * K_LD + 16 * ks + 8 * hh]);
        s[t] = mfma_32x32x16(a, qf[ks], s[t]);
      }
    }
  };

  // softmax of the tile held in s (in place -> probabilities), then O += P V
  auto soft_pv = [&](const _Float16* vt, const float* bt, int kb, floatx16* s, bool mask)
      __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        if (kBias) {
          const float4 b4 = *reinterpret_cast<const float4*>(&bt[32 * t + 8 * j4 + 4 * hh]);
          bias[0] = b4.x; bias[1] = b4.y; bias[2] = b4.z; bias[3] = b4.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 4 * j4 + r;
          float x = kBias ? fmaf(s[t][j], alpha, bias[r]) : s[t][j] * alpha;
          if (mask && kb + 32 * t + 8 * j4 + 4 * hh + r > my_q) x = -INFINITY;
          s[t][j] = x;
          mx = fmaxf(mx, x);
        }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Wave-uniform and rare after the first tiles: a real branch, not a select.
    if (__builtin_expect(__builtin_amdgcn_readfirstlane(__any(mx > m_run + kRescaleThreshold)), 0)) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < DT; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) o[i][j] *= corr;
      }
    }
    float rs = 0.f;
    uint32_t pk[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float p0 = fast_exp2(s[t][j] - m_run);
        const float p1 = fast_exp2(s[t][j + 1] - m_run);
        rs += p0 + p1;
        pk[t][j >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      }
    }
    l_run += rs;
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint32_t* src = &pk[ps >> 1][4 * (ps & 1)];
      const u32x4 pv = {src[0], src[1], src[2], src[3]};
      const f16x8 b = __builtin_bit_cast(f16x8, pv);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&vt[(32 * dt + l32) * VT_LD + 16 * ps + 8 * hh]);
        o[dt] = mfma_f16(a, b, o[dt]);
      }
    }
  };

  // ---- prologue: K of tiles 0, 1 in LDS and S of this group's first tile;
  // K of tiles 2, 3 and V of tiles 0, 1 in registers.
  load_k(0);
  store_k(0);
  load_k(2);
  load_v(0);
  __syncthreads();
  floatx16 s_cur[2];
  if (grp < n_vis) qk(k_lds[0][grp], s_cur);

  // One pipeline stage per tile pair: group g consumes tile 2 st + g while
  // S of tile 2 st + 2 + g is formed from the other LDS buffer and the loads
  // of the following pair are in flight.  One barrier per stage: a buffer
  // written at stage st was last read at stage st - 1.
  auto stage = [&](auto par_c, int st) __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value, npar = par ^ 1;
    store_k(npar);   // K of tiles 2 st + 2, 2 st + 3
    store_v(par);    // V (and scores) of tiles 2 st, 2 st + 1
    __syncthreads();
    load_k(2 * st + 4);
    load_v(2 * st + 2);
    const int t = 2 * st + grp;
    if (t < n_vis) {
      const int kb = t * kBN;
      const bool diag = kb + kBN - 1 > q0;
      const _Float16* vt = vt_lds[par][grp];
      const float* bt = b_lds[par][grp];
      if (t + 2 < n_vis) {
        floatx16 s_nxt[2];
        qk(k_lds[npar][grp], s_nxt);
        if (diag) soft_pv(vt, bt, kb, s_cur, true);
        else soft_pv(vt, bt, kb, s_cur, false);
        s_cur[0] = s_nxt[0];
        s_cur[1] = s_nxt[1];
      } else {
        if (diag) soft_pv(vt, bt, kb, s_cur, true);
        else soft_pv(vt, bt, kb, s_cur, false);
      }
    }
  };
  for (int st = 0; st < n_steps; st += 2) {
    stage(std::integral_constant<int, 0>{}, st);
    if (st + 1 < n_steps) stage(std::integral_constant<int, 1>{}, st + 1);
  }

  // ---- merge the two groups' partial softmax states (same query rows)
  __syncthreads();
  float* xch = reinterpret_cast<float*>(&k_lds[0][0][0]) + ((wave & 3) * 64 + lane) * (16 * DT + 2);
  if (grp == 1) {
#pragma unroll
    for (int i = 0; i < DT; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) xch[16 * i + j] = o[i][j];
    }
    xch[16 * DT] = m_run;
    xch[16 * DT + 1] = l_run;
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float m1 = xch[16 * DT], l1 = xch[16 * DT + 1];
    const float m = fmaxf(m_run, m1);
    const float c0 = fast_exp2(m_run - m), c1 = fast_exp2(m1 - m);
#pragma unroll
    for (int i = 0; i < DT; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) o[i][j] = o[i][j] * c0 + xch[16 * i + j] * c1;
    }
    l_run = l_run * c0 + l1 * c1;
    m_run = m;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < M) {
    const float inv = 1.f / l_tot;
    bf16* orow = out + static_cast<size_t>(my_q) * Hq * D + static_cast<size_t>(head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16 pk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pk[r] = static_cast<bf16>(o[dt][4 * jj + r] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = __builtin_bit_cast(uint2, pk);
      }
    }
    if (lse != nullptr && hh == 0)
      lse[static_cast<size_t>(head) * M + my_q] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// V -> packed V^T: for each KV head and each 64-key tile, a [D][64] fp16 block
// whose key order inside each 16-key group is permuted so that every lane's
// eight keys of a P.V step are one contiguous 16-byte run.  Keys >= M are
// zero.  One work-group per (tile, KV head); each thread moves 4 keys x 8 dims.
template <int D>
__global__ __launch_bounds__(256) void v_pack_kernel(const bf16* __restrict__ v, int M, int Hkv,
                                                     _Float16* __restrict__ vt_pack) {
  constexpr int CPR = D / 8;
  constexpr int TASKS = (kBN / 4) * CPR;
  const int n_tiles = (M + kBN - 1) / kBN;
  const int tile = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int tid = threadIdx.x;
  if (tid >= TASKS) return;
  const int kg = tid % 16, dc = tid / 16;
  const uint32_t kv_row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
  const uint32_t kv_bytes = kv_row_bytes * static_cast<uint32_t>(M);
  const uint32_t off0 = static_cast<uint32_t>(tile) * kBN * kv_row_bytes;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(
      reinterpret_cast<const char*>(v + static_cast<size_t>(kvh) * D) + off0,
      off0 < kv_bytes ? kv_bytes - off0 : 0u);
  u32x4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = bload16(r, (4 * kg + i) * kv_row_bytes + 16 * dc);
  // keys 4 kg + i sit at positions 16 s + 8 h' + 4 b + i, with
  // s = kg / 4, h' = (kg % 4) & 1, b = (kg % 4) >> 1.
  const int s = kg >> 2, j = kg & 3;
  const int phys = 16 * s + 8 * (j & 1) + 4 * (j >> 1);
  _Float16* dst = vt_pack + (static_cast<size_t>(kvh) * n_tiles + tile) * D * kBN;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x0 = bf16x2_to_f16x2(x[0][w]), x1 = bf16x2_to_f16x2(x[1][w]);
    const uint32_t x2 = bf16x2_to_f16x2(x[2][w]), x3 = bf16x2_to_f16x2(x[3][w]);
    uint2 lo, hi;  // dim 2w: low halves; dim 2w+1: high halves
    lo.x = (x0 & 0xFFFFu) | (x1 << 16);
    lo.y = (x2 & 0xFFFFu) | (x3 << 16);
    hi.x = (x0 >> 16) | (x1 & 0xFFFF0000u);
    hi.y = (x2 >> 16) | (x3 & 0xFFFF0000u);
    const int d0 = 8 * dc + 2 * w;
    *reinterpret_cast<uint2*>(&dst[d0 * kBN + phys]) = lo;
    *reinterpret_cast<uint2*>(&dst[(d0 + 1) * kBN + phys]) = hi;
  }
}

template <int D, bool kBias>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int M, int Hq, int Hkv,
                  const float* s, const float* g, const float* t, uint16_t* out, float* lse,
                  void* ws, hipStream_t stream) {
  const int n_tiles = (M + kBN - 1) / kBN;
  _Float16* vt = static_cast<_Float16*>(ws);
  hipLaunchKernelGGL((v_pack_kernel<D>), dim3(static_cast<unsigned>(n_tiles * Hkv)), dim3(256), 0,
                     stream, reinterpret_cast<const bf16*>(v), M, Hkv, vt);
  const int n_qt = (M + kBM - 1) / kBM;
  const dim3 grid(static_cast<unsigned>(n_qt) * static_cast<unsigned>(Hq));
  hipLaunchKernelGGL((attn_fwd_kernel<D, kBias>), grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k), vt, M, Hq,
                     Hkv, s, g, t, reinterpret_cast<bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int64_t n, int n_kv_heads, int head_dim) {
  const int64_t n_tiles = (n + kBN - 1) / kBN;
  return static_cast<size_t>(n_tiles) * kBN * n_kv_heads * head_dim * 2;
}

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                           int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                           const float* gain, const float* tau, uint16_t* out, float* lse,
                           void* workspace, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int M = static_cast<int>(n);
  const bool bias = gain != nullptr;
  if (head_dim == 128)
    return bias ? launch<128, true>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out,
                                    lse, workspace, stream)
                : launch<128, false>(q, k, v, M, n_q_heads, n_kv_heads, nullptr, nullptr,
                                     nullptr, out, lse, workspace, stream);
  return bias ? launch<64, true>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out,
                                 lse, workspace, stream)
              : launch<64, false>(q, k, v, M, n_q_heads, n_kv_heads, nullptr, nullptr, nullptr,
                                  out, lse, workspace, stream);
}

}  // namespace tg
