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
// Design (flash-style, one work-group = 128 query rows of one query head):
//  * 4 waves, each owning 32 query rows.  S^T = K Q^T is formed with
//    v_mfma_f32_32x32x16_bf16 (A = K tile from LDS, B = Q kept in registers),
//    so every lane owns one query column and 16 keys of each 32-key block:
//    the online-softmax row statistics are lane-local plus one exchange with
//    the other lane half.
//  * O^T = V^T P^T reuses the softmax output straight from registers as the B
//    operand; V is stored transposed in LDS (key order permuted within each
//    16-key group so that each lane's eight keys are one 16-byte read).
//  * Scores are pre-multiplied by gain_h * log2(e) when staged into LDS; the
//    temperature and 1/sqrt(d) are folded with log2(e) into one scale, so each
//    logit costs one FMA before the exp2-based online softmax.
//  * The next K/V tile is loaded into registers while the current one is
//    consumed; fully masked causal tiles are skipped per wave; work-groups
//    are issued longest-first (last query tile first).
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kBM = 128;     // query rows per work-group
constexpr int kBN = 64;      // keys per tile
constexpr int kThreads = 256;

template <int D, bool kBias>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, int M,
    int Hq, int Hkv, const float* __restrict__ key_score, const float* __restrict__ gain,
    const float* __restrict__ tau, bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int KSTEPS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;            // 32-row tiles of O^T
  constexpr int K_LD = D + 8;           // K row in LDS, padded by 16 B
  constexpr int VT_LD = kBN + 8;        // V^T row in LDS, padded by 16 B
  constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  constexpr int K_TASKS = kBN * CPR;    // 16-byte K chunks per tile
  constexpr int K_PER_T = K_TASKS / kThreads;
  constexpr int V_TASKS = (kBN / 4) * CPR;  // (4 keys x 8 dims) V blocks per tile
  static_assert(K_TASKS % kThreads == 0, "K tile split");
  static_assert(V_TASKS <= kThreads, "V tile split");

  __shared__ __align__(16) bf16 k_lds[kBN * K_LD];
  __shared__ __align__(16) bf16 vt_lds[D * VT_LD];
  __shared__ __align__(16) float b_lds[kBN];

  const int n_qt = (M + kBM - 1) / kBM;
  const int head = blockIdx.x % Hq;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.x / Hq);
  const int kvh = head / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBM + wave * 32;
  const int my_q = q0 + l32;

  const float t_h = kBias ? tau[head] : 1.f;
  const float alpha = kLog2e / (sqrtf(static_cast<float>(D)) * t_h);
  const float beta = kBias ? gain[head] * kLog2e : 0.f;

  const size_t q_stride = static_cast<size_t>(Hq) * D;
  const size_t kv_stride = static_cast<size_t>(Hkv) * D;

  // Q fragments: lane holds Q[my_q][16 s + 8 hh .. + 7].
  bf16x8 qf[KSTEPS];
  {
    const bf16* qrow = q + static_cast<size_t>(my_q) * q_stride + static_cast<size_t>(head) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = as_bf16x8(my_q < M ? ld16(qrow + 16 * s + 8 * hh) : zero_u32x4());
  }

  floatx16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int q_last = min(qt * kBM + kBM, M) - 1;
  const int n_kt = q_last / kBN + 1;

  // ---- register staging of one K/V tile
  u32x4 kreg[K_PER_T];
  u32x4 vreg[4];
  float breg = 0.f;
  const int v_kg = tid % 16;  // group of 4 consecutive keys
  const int v_dc = tid / 16;  // 8-dim chunk

  auto load_tile = [&](int kt) {
    const int kb = kt * kBN;
#pragma unroll
    for (int p = 0; p < K_PER_T; ++p) {
      const int f = tid + p * kThreads;
      const int row = f / CPR, c = f % CPR;
      const int key = kb + row;
      kreg[p] = key < M ? ld16(k + static_cast<size_t>(key) * kv_stride +
                               static_cast<size_t>(kvh) * D + 8 * c)
                        : zero_u32x4();
    }
    if (tid < V_TASKS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 4 * v_kg + r;
        vreg[r] = key < M ? ld16(v + static_cast<size_t>(key) * kv_stride +
                                 static_cast<size_t>(kvh) * D + 8 * v_dc)
                          : zero_u32x4();
      }
    }
    if (kBias && tid < kBN) {
      const int key = kb + tid;
      breg = key < M ? beta * key_score[key] : 0.f;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < K_PER_T; ++p) {
      const int f = tid + p * kThreads;
      const int row = f / CPR, c = f % CPR;
      st16(&k_lds[row * K_LD + 8 * c], kreg[p]);
    }
    if (tid < V_TASKS) {
      // keys 4 kg + r sit at positions 16 s + 8 h' + 4 b + r, with
      // s = kg / 4, h' = (kg % 4) & 1, b = (kg % 4) >> 1.
      const int s = v_kg >> 2, j = v_kg & 3;
      const int phys = 16 * s + 8 * (j & 1) + 4 * (j >> 1);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = vreg[0][w], x1 = vreg[1][w], x2 = vreg[2][w], x3 = vreg[3][w];
        // dim 2w: low halves; dim 2w+1: high halves
        uint2 lo, hi;
        lo.x = (x0 & 0xFFFFu) | (x1 << 16);
        lo.y = (x2 & 0xFFFFu) | (x3 << 16);
        hi.x = (x0 >> 16) | (x1 & 0xFFFF0000u);
        hi.y = (x2 >> 16) | (x3 & 0xFFFF0000u);
        const int d0 = 8 * v_dc + 2 * w;
        *reinterpret_cast<uint2*>(&vt_lds[d0 * VT_LD + phys]) = lo;
        *reinterpret_cast<uint2*>(&vt_lds[(d0 + 1) * VT_LD + phys]) = hi;
      }
    }
    if (kBias && tid < kBN) b_lds[tid] = breg;
  };

  load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);

    const int kb = kt * kBN;
    if (kb <= q0 + 31) {  // some key of this tile is visible to this wave
      floatx16 s[2];
      s[0] = zero16();
      s[1] = zero16();
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 a = lds_bf16x8(&k_lds[(32 * t + l32) * K_LD + 16 * ks + 8 * hh]);
          s[t] = mfma_32x32x16(a, qf[ks], s[t]);
        }
      }
      const bool diag = kb + kBN - 1 > q0;
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kl = 32 * t + 8 * (j >> 2) + 4 * hh + (j & 3);
          float x = kBias ? fmaf(s[t][j], alpha, b_lds[kl]) : s[t][j] * alpha;
          if (diag && kb + kl > my_q) x = -INFINITY;
          s[t][j] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = fast_exp2(s[t][j] - m_new);
          s[t][j] = p;
          rs += p;
        }
      }
      l_run = l_run * corr + rs;
#pragma unroll
      for (int i = 0; i < DT; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) o[i][j] *= corr;
      }
      bf16x8 pf[4];
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[ps][i] = static_cast<bf16>(s[ps >> 1][8 * (ps & 1) + i]);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
          const bf16x8 a = lds_bf16x8(&vt_lds[(32 * dt + l32) * VT_LD + 16 * ps + 8 * hh]);
          o[dt] = mfma_32x32x16(a, pf[ps], o[dt]);
        }
      }
    }
    __syncthreads();
  }

  if (my_q < M) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    bf16* orow = out + static_cast<size_t>(my_q) * q_stride + static_cast<size_t>(head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16 pk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pk[r] = static_cast<bf16>(o[dt][4 * jj + r] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) =
            __builtin_bit_cast(uint2, pk);
      }
    }
    if (lse != nullptr && hh == 0)
      lse[static_cast<size_t>(head) * M + my_q] = (m_run + __log2f(l_tot)) * kLn2;
  } else {
    (void)__shfl_xor(l_run, 32);
  }
}

template <int D, bool kBias>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int M, int Hq, int Hkv,
                  const float* s, const float* g, const float* t, uint16_t* out, float* lse,
                  hipStream_t stream) {
  const int n_qt = (M + kBM - 1) / kBM;
  const dim3 grid(static_cast<unsigned>(n_qt) * static_cast<unsigned>(Hq));
  hipLaunchKernelGGL((attn_fwd_kernel<D, kBias>), grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),
                     reinterpret_cast<const bf16*>(v), M, Hq, Hkv, s, g, t,
                     reinterpret_cast<bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                           int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                           const float* gain, const float* tau, uint16_t* out, float* lse,
                           hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int M = static_cast<int>(n);
  const bool bias = gain != nullptr;
  if (head_dim == 128)
    return bias ? launch<128, true>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out,
                                    lse, stream)
                : launch<128, false>(q, k, v, M, n_q_heads, n_kv_heads, nullptr, nullptr,
                                     nullptr, out, lse, stream);
  return bias ? launch<64, true>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out,
                                 lse, stream)
              : launch<64, false>(q, k, v, M, n_q_heads, n_kv_heads, nullptr, nullptr, nullptr,
                                  out, lse, stream);
}

}  // namespace tg
