// Token-gated causal GQA attention (forward) for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"; fugumt.com
// abstract): above the gate layer each kept key's gate score is added to the
// attention logits, scaled by a per-head gain, and a per-head temperature
// rescales q.k.  Read here as
//     logit_ij = q_i.k_j / (sqrt(d) * tau_h) + gain_h * s_j ,   j <= i.
// With gain = 0 and tau = 1 the same kernels give plain causal attention, the
// unpruned baseline.
//
// Two launches per call:
//
// 1. kv_pack: per KV head and 64-key tile, build the exact LDS image the main
//    kernel consumes, in the caller's workspace:
//      * K~ rows [k_j | s_hi, s_lo, s_hi, 0...] in bf16 (the extra 16-column
//        k-step exists only in the gated kernel; s_hi/s_lo split the score
//        into two bf16 parts), rows padded to avoid LDS bank conflicts;
//      * V^T in fp16 ([d][key], key order permuted inside each 16-key group
//        so that every lane's eight keys of a P.V step are one 16-byte run).
//    Rows past n are zero.
// 2. attn_fwd: one work-group = 128 query rows of one query head, eight
//    waves: two groups of four waves of 32 rows; the groups take the even and
//    the odd key tiles (halving the serial chain of the longest rows, two
//    waves per SIMD so one's softmax overlaps the other's MFMAs) and merge
//    their softmax states in LDS at the end.
//      * S^T = K~ Q~^T on v_mfma_f32_32x32x16_bf16 (A = K~ from LDS, B = Q~
//        held in registers for the whole key loop).  The bias rides in the
//        extra k-step: Q~ carries c = gain * sqrt(d) * tau split as (c_hi,
//        c_hi, c_lo), so S~ = q.k + c s_j and one multiply by
//        alpha = log2(e) / (sqrt(d) tau) gives the logit in log2 units.
//      * Each lane owns one query column, so the online-softmax statistics are
//        lane-local plus one exchange between lane halves; the running max
//        only moves when a tile raises it by more than 2^8 (lazy rescaling).
//      * O^T = V^T P^T on v_mfma_f32_32x32x16_f16 with P taken straight from
//        registers.  P and V are fp16 for this product: bf16 P (8-bit
//        mantissa) costs up to ~3e-3 of output error on peaked rows on top of
//        the bf16 output rounding.  O accumulates in fp32.
//      * Tiles arrive by buffer-to-LDS DMA (buffer_load_dwordx4 ... lds) one
//        tile pair ahead into double-buffered LDS: no staging registers, no
//        LDS store instructions, one barrier per tile pair.
//      * Causal masking only on diagonal tiles; tiles above a wave's rows are
//        skipped.  Heads of one KV group are pinned to one XCD (work-groups
//        are dealt round-robin over the 8 XCDs) so its K/V stays in that L2;
//        within an XCD the longest query tiles go first.
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kBM = 128;       // query rows per work-group
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 512;  // two groups of four waves (32 rows each)
constexpr float kRescaleThreshold = 8.f;  // log2 units

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

template <int D, bool kBias>
struct Tile {
  static constexpr int KD = D + (kBias ? 16 : 0);        // K~ columns
  static constexpr int KS = KD / 16;                      // k-steps of S^T
  static constexpr int K_ROW = KD * 2 + 16;               // bytes, padded
  static constexpr int K_IMG = kBN * K_ROW;
  static constexpr int V_ROW = kBN * 2 + 16;              // bytes, padded
  static constexpr int V_IMG = D * V_ROW;
  static constexpr int IMG = K_IMG + V_IMG;               // one tile in LDS / workspace
  static_assert(IMG % 1024 == 0, "tile image must be whole 1 KiB DMA chunks");
};


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

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<bf16>(x));  // round to nearest even
}

// ---------------------------------------------------------------------------
// kv_pack: one work-group per (tile, KV head).
// ---------------------------------------------------------------------------
template <int D, bool kBias>
__global__ __launch_bounds__(256) void kv_pack_kernel(const bf16* __restrict__ k,
                                                      const bf16* __restrict__ v,
                                                      const float* __restrict__ key_score, int M,
                                                      int Hkv, char* __restrict__ ws) {
  using T = Tile<D, kBias>;
  const int n_tiles = (M + kBN - 1) / kBN;
  const int tile = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int tid = threadIdx.x;
  char* img = ws + (static_cast<size_t>(kvh) * n_tiles + tile) * T::IMG;
  const uint32_t kv_row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
  const uint32_t kv_bytes = kv_row_bytes * static_cast<uint32_t>(M);
  const uint32_t off0 = static_cast<uint32_t>(tile) * kBN * kv_row_bytes;
  const uint32_t left = off0 < kv_bytes ? kv_bytes - off0 : 0u;

  // K~ rows: D/8 data chunks, then (gated) the score chunk and a zero chunk,
  // then the pad chunk.
  {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(reinterpret_cast<const char*>(k + static_cast<size_t>(kvh) * D) + off0, left);
    constexpr int CHUNKS = T::K_ROW / 16;
    for (int f = tid; f < kBN * CHUNKS; f += 256) {
      const int row = f / CHUNKS, c = f % CHUNKS;
      u32x4 val = zero_u32x4();
      if (c < D / 8) {
        val = bload16(rk, row * kv_row_bytes + 16 * c);
      } else if (kBias && c == D / 8) {
        const int key = tile * kBN + row;
        const float s = key < M ? key_score[key] : 0.f;
        const uint16_t hi = bf16_bits(s);
        const uint16_t lo = bf16_bits(s - __uint_as_float(static_cast<uint32_t>(hi) << 16));
        val[0] = hi | (static_cast<uint32_t>(lo) << 16);
        val[1] = hi;
      }
      st16(img + row * T::K_ROW + 16 * c, val);
    }
  }
  // V^T: 4 keys x 8 dims per task; keys 4 kg + i sit at positions
  // 16 s + 8 h' + 4 b + i with s = kg / 4, h' = (kg % 4) & 1, b = (kg % 4) >> 1.
  {
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(reinterpret_cast<const char*>(v + static_cast<size_t>(kvh) * D) + off0, left);
    char* vimg = img + T::K_IMG;
    constexpr int TASKS = (kBN / 4) * (D / 8);
    for (int f = tid; f < TASKS; f += 256) {
      const int kg = f % 16, dc = f / 16;
      u32x4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = bload16(rv, (4 * kg + i) * kv_row_bytes + 16 * dc);
      const int s = kg >> 2, j = kg & 3;
      const int phys = 16 * s + 8 * (j & 1) + 4 * (j >> 1);
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
        *reinterpret_cast<uint2*>(vimg + d0 * T::V_ROW + 2 * phys) = lo;
        *reinterpret_cast<uint2*>(vimg + (d0 + 1) * T::V_ROW + 2 * phys) = hi;
      }
    }
    for (int d = tid; d < D; d += 256) st16(vimg + d * T::V_ROW + kBN * 2, zero_u32x4());
  }
}

// ---------------------------------------------------------------------------
// attn_fwd
// ---------------------------------------------------------------------------
template <int D, bool kBias>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(
    const bf16* __restrict__ q, const char* __restrict__ ws, int M, int Hq, int Hkv,
    const float* __restrict__ gain, const float* __restrict__ tau, bf16* __restrict__ out,
    float* __restrict__ lse) {
  using T = Tile<D, kBias>;
  constexpr int KS = T::KS;
  constexpr int DT = D / 32;                 // 32-row tiles of O^T
  constexpr int N_DMA = 2 * T::IMG / 1024;   // 1 KiB DMA chunks per tile pair
  constexpr int NW = kThreads / 64;

  __shared__ __align__(16) char lds[2][2][T::IMG];   // [parity][tile of the pair]

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
  const int grp = wave >> 2;             // 0: even key tiles, 1: odd key tiles
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBM + (wave & 3) * 32;   // first of this wave's 32 rows
  const int my_q = q0 + l32;

  const float t_h = kBias ? tau[head] : 1.f;
  const float alpha = kLog2e / (sqrtf(static_cast<float>(D)) * t_h);

  // ---- Q~ fragments (B operand): lane holds Q[my_q][16 s + 8 hh .. + 7]
  bf16x8 qf[KS];
  {
    const uint32_t q_row_bytes = static_cast<uint32_t>(Hq) * D * 2;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(q + static_cast<size_t>(head) * D, q_row_bytes * static_cast<uint32_t>(M));
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = as_bf16x8(bload16(rq, static_cast<uint32_t>(my_q) * q_row_bytes + (16 * s + 8 * hh) * 2));
    if (kBias) {
      const float c = gain[head] * sqrtf(static_cast<float>(D)) * t_h;   // gain / alpha * log2(e)
      const uint16_t c_hi = bf16_bits(c);
      const uint16_t c_lo = bf16_bits(c - __uint_as_float(static_cast<uint32_t>(c_hi) << 16));
      u32x4 e = zero_u32x4();
      if (hh == 0) {
        e[0] = c_hi | (static_cast<uint32_t>(c_hi) << 16);
        e[1] = c_lo;
      }
      qf[KS - 1] = as_bf16x8(e);
    }
  }

  floatx16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int q_last = min(qt * kBM + kBM, M) - 1;
  const int n_kt = q_last / kBN + 1;                  // key tiles of the work-group
  const int n_steps = (n_kt + 1) / 2;                 // tile pairs
  const int n_vis = q0 <= q_last ? min(q0 + 31, q_last) / kBN + 1 : 0;  // tiles this wave sees

  // ---- DMA of one tile pair (2 * IMG bytes) into lds[par]
  const int n_tiles = (M + kBN - 1) / kBN;
  const __amdgpu_buffer_rsrc_t rws =
      make_rsrc(ws + static_cast<size_t>(kvh) * n_tiles * T::IMG,
                static_cast<uint32_t>(n_tiles) * T::IMG);
  auto dma_pair = [&](int par, int t0) __attribute__((always_inline)) {
    const uint32_t base = static_cast<uint32_t>(t0) * T::IMG + 16u * lane;
    for (int i = wave; i < N_DMA; i += NW) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rws, (__attribute__((address_space(3))) void*)(&lds[par][0][0] + 1024 * i), 16,
          static_cast<int>(base + 1024u * i), 0, 0, 0);
    }
  };

  // ---- one 64-key tile for this wave's 32 rows; MASK (compile time) applies
  // the causal mask, needed only on diagonal tiles.
  auto tile = [&](auto mask_c, const char* img, int kb) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    floatx16 s[2];   // 32-key halves
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            img + (32 * t2 + l32) * T::K_ROW + (16 * ks + 8 * hh) * 2);
        s[t2] = mfma_32x32x16(a, qf[ks], s[t2]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = s[t2][j] * alpha;
        if (MASK && kb + 32 * t2 + 8 * (j >> 2) + 4 * hh + (j & 3) > my_q) x = -INFINITY;
        s[t2][j] = x;
        mx = fmaxf(mx, x);
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
    uint32_t pk[2][8];   // fp16 pairs of P: [32-key half][pair]
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float p0 = fast_exp2(s[t2][j] - m_run);
        const float p1 = fast_exp2(s[t2][j + 1] - m_run);
        rs += p0 + p1;
        pk[t2][j >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      }
    }
    l_run += rs;
    const char* vimg = img + T::K_IMG;
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint32_t* src = &pk[ps >> 1][4 * (ps & 1)];
      const u32x4 pv = {src[0], src[1], src[2], src[3]};
      const f16x8 b = __builtin_bit_cast(f16x8, pv);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(
            vimg + (32 * dt + l32) * T::V_ROW + (16 * ps + 8 * hh) * 2);
        o[dt] = mfma_f16(a, b, o[dt]);
      }
    }
  };

  // ---- main loop: one tile pair per step, one barrier per step.  The DMA
  // issued at step st fills the parity read at step st + 1; that buffer was
  // last read at step st - 1, which every wave finished before barrier st.
  // The two waves sharing a SIMD (one per group) leave each barrier in the
  // same phase; raising one group's priority (alternating per step) lets its
  // MFMAs run first while the other wave's softmax fills the VALU slots.
  dma_pair(0, 0);
  for (int st = 0; st < n_steps; ++st) {
    const int par = st & 1;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA into lds[par] has landed
    __syncthreads();                 // ... and every other wave's
    if (grp == par) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    if (st + 1 < n_steps) dma_pair(par ^ 1, 2 * st + 2);
    const int t = 2 * st + grp;
    if (t < n_vis) {
      if (t * kBN + kBN - 1 > q0) tile(std::true_type{}, &lds[par][grp][0], t * kBN);
      else tile(std::false_type{}, &lds[par][grp][0], t * kBN);
    }
  }

  // ---- merge the two groups' partial softmax states (same query rows)
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();
  constexpr int XU = 16 * DT + 2;         // floats per lane
  float* xch = reinterpret_cast<float*>(&lds[0][0][0]) + ((wave & 3) * 64 + lane) * XU;
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
  const float m1 = xch[16 * DT], l1 = xch[16 * DT + 1];
  const float m = fmaxf(m_run, m1);
  const float c0 = fast_exp2(m_run - m), c1 = fast_exp2(m1 - m);
#pragma unroll
  for (int i = 0; i < DT; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) o[i][j] = o[i][j] * c0 + xch[16 * i + j] * c1;
  }
  const float l = l_run * c0 + l1 * c1;
  const float l_tot = l + __shfl_xor(l, 32);
  if (my_q < M) {
    const float inv = 1.f / l_tot;
    bf16* orow = out + static_cast<size_t>(my_q) * Hq * D + static_cast<size_t>(head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16 pkk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pkk[r] = static_cast<bf16>(o[dt][4 * jj + r] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = __builtin_bit_cast(uint2, pkk);
      }
    }
    if (lse != nullptr && hh == 0)
      lse[static_cast<size_t>(head) * M + my_q] = (m + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool kBias>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int M, int Hq, int Hkv,
                  const float* s, const float* g, const float* t, uint16_t* out, float* lse,
                  void* ws, hipStream_t stream) {
  const int n_tiles = (M + kBN - 1) / kBN;
  char* img = static_cast<char*>(ws);
  hipLaunchKernelGGL((kv_pack_kernel<D, kBias>), dim3(static_cast<unsigned>(n_tiles * Hkv)),
                     dim3(256), 0, stream, reinterpret_cast<const bf16*>(k),
                     reinterpret_cast<const bf16*>(v), s, M, Hkv, img);
  const int n_qt = (M + kBM - 1) / kBM;
  const dim3 grid(static_cast<unsigned>(n_qt) * static_cast<unsigned>(Hq));
  hipLaunchKernelGGL((attn_fwd_kernel<D, kBias>), grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const bf16*>(q), img, M, Hq, Hkv, g, t,
                     reinterpret_cast<bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int64_t n, int n_kv_heads, int head_dim, bool gated) {
  const int64_t n_tiles = (n + kBN - 1) / kBN;
  int64_t img;
  if (head_dim == 128) img = gated ? Tile<128, true>::IMG : Tile<128, false>::IMG;
  else img = gated ? Tile<64, true>::IMG : Tile<64, false>::IMG;
  return static_cast<size_t>(n_tiles * n_kv_heads * img);
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
