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
// Two or three launches per call:
//
// 1. kv_pack: per KV head and 64-key tile, build the exact LDS image the main
//    kernel consumes, in the caller's workspace:
//      * K~ rows [k_j | s_hi, s_lo, s_hi, 0...] in bf16 (the extra 16-column
//        k-step exists only in the gated kernel; s_hi/s_lo split the score
//        into two bf16 parts), rows padded to avoid LDS bank conflicts;
//      * V^T in fp16 ([d][key], key order permuted inside each 16-key group
//        so that every lane's eight keys of a P.V step are one 16-byte run).
//    Rows past n are zero.
// 2. attn_fwd: one work-group = 128 query rows of one query head over a run
//    of their key tiles; four waves of 32 rows; two work-groups per CU (they
//    drift out of phase, so one's softmax and DMA waits overlap the other's
//    MFMAs).
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
//        tile ahead into double-buffered LDS: no staging registers, no LDS
//        store instructions, one barrier per tile.
//      * Causal masking only on diagonal tiles; tiles above a wave's rows are
//        skipped.
//      * Split keys.  When few query tiles exist (short kept prefixes), the
//        longest query tile's key loop would outlast the average work of a
//        resident work-group many times over.  Then the key tiles of query
//        tile qt are cut into ceil((qt + 1) / h) chunks of 2h tiles, each a
//        work-group of its own.  Every chunk stores its normalised partial
//        output (fp16) and its running max and sum in the workspace.
// 3. attn_merge (only when some query tile is split): one work-group per
//    split query tile combines its chunks' partials in chunk order and writes
//    the output.  A third launch rather than a last-arriver merge inside
//    attn_fwd: the agent-scope fences such a merge needs (L2 write-back and
//    invalidate on every chunk) cost more than the whole split saves.
//      * Heads of one KV group are pinned to one XCD (work-groups are dealt
//        round-robin over the 8 XCDs) so its K/V stays in that L2; within an
//        XCD the units of the longest query tiles go first.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kBM = 128;       // query rows per work-group
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // four waves of 32 rows
constexpr int kSlots = 512;    // resident work-groups: 256 CUs x 2
constexpr int kMinHalf = 4;    // chunks are at least 8 key tiles
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
  // One split chunk's partial state: per wave, the lane-major fp16 output
  // (D bytes per lane in 16-byte vectors) and a (max, sum) pair per lane.
  static constexpr int PART_O = D * 64;
  static constexpr int PART_WAVE = PART_O + 8 * 64;
  static constexpr int PART = 4 * PART_WAVE;
};

// Work-groups of one head before query tile q when query tile i has
// ceil((i + 1) / h) chunks: sum_{j=1..q} ceil(j / h).
__host__ __device__ __forceinline__ int64_t units_before(int64_t q, int64_t h) {
  const int64_t a = q / h, r = q % h;
  return h * a * (a + 1) / 2 + r * (a + 1);
}

// Chunk half-length h (chunks are 2h key tiles): no split (h = n_qt) unless
// the longest query tile (2 n_qt key tiles) exceeds the average number of
// tile steps per resident work-group; then chunks of about that average, but
// no shorter than 2 kMinHalf tiles (each split chunk pays a partial-state
// round trip).
struct Plan {
  int n_qt, n_tiles, h;
  int64_t units;       // work-groups per head
  int64_t n_split;     // query tiles per head with more than one chunk
  int64_t n_part;      // split chunks per head
  size_t img_bytes, part_off, total;
};

template <int D, bool kBias>
Plan make_plan(int64_t M, int Hq, int Hkv) {
  using T = Tile<D, kBias>;
  Plan p{};
  p.n_qt = static_cast<int>((M + kBM - 1) / kBM);
  p.n_tiles = static_cast<int>((M + kBN - 1) / kBN);
  const double avg = static_cast<double>(Hq) * p.n_qt * (p.n_qt + 1) / kSlots;
  int64_t h = p.n_qt;
  if (2.0 * p.n_qt > avg) h = std::max<int64_t>(kMinHalf, static_cast<int64_t>(std::ceil(avg / 2.0)));
  if (h >= p.n_qt) h = std::max(p.n_qt, 1);
  p.h = static_cast<int>(h);
  p.units = units_before(p.n_qt, h);
  p.n_split = std::max<int64_t>(p.n_qt - h, 0);
  p.n_part = p.units - std::min<int64_t>(h, p.n_qt);
  p.img_bytes = static_cast<size_t>(p.n_tiles) * Hkv * T::IMG;
  p.part_off = p.img_bytes;
  p.total = p.part_off + static_cast<size_t>(Hq) * p.n_part * T::PART;
  return p;
}
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

  // Every load of the tile is issued before the first store (one memory
  // round trip per work-group).
  constexpr int DC = D / 8;                        // 16-byte data chunks per row
  constexpr int KL = kBN * DC / 256;               // K chunks per thread
  constexpr int XC = T::K_ROW / 16 - DC;           // extra chunks per K~ row
  static_assert(kBN * DC % 256 == 0 && kBN * XC <= 256 && 16 * DC <= 256, "kv_pack tiling");
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(reinterpret_cast<const char*>(k + static_cast<size_t>(kvh) * D) + off0, left);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(reinterpret_cast<const char*>(v + static_cast<size_t>(kvh) * D) + off0, left);
  u32x4 kx[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const int f = tid + 256 * i;
    kx[i] = bload16(rk, (f / DC) * kv_row_bytes + 16 * (f % DC));
  }
  // V^T task of this thread: 4 keys x 8 dims; keys 4 kg + i sit at positions
  // 16 s + 8 h' + 4 b + i with s = kg / 4, h' = (kg % 4) & 1, b = (kg % 4) >> 1.
  const int kg = tid % 16, dc = tid / 16;
  const bool v_task = dc < DC;
  u32x4 vx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    vx[i] = v_task ? bload16(rv, (4 * kg + i) * kv_row_bytes + 16 * dc) : zero_u32x4();
  // Extra K~ chunk of this thread: (gated) the score chunk, a zero chunk,
  // then the pad chunk.
  const int x_row = tid / XC, x_c = tid % XC;
  const int x_key = tile * kBN + x_row;
  const float x_s = (kBias && tid < kBN * XC && x_c == 0 && x_key < M) ? key_score[x_key] : 0.f;

#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const int f = tid + 256 * i;
    st16(img + (f / DC) * T::K_ROW + 16 * (f % DC), kx[i]);
  }
  if (tid < kBN * XC) {
    u32x4 val = zero_u32x4();
    if (kBias && x_c == 0) {
      const uint16_t hi = bf16_bits(x_s);
      const uint16_t lo = bf16_bits(x_s - __uint_as_float(static_cast<uint32_t>(hi) << 16));
      val[0] = hi | (static_cast<uint32_t>(lo) << 16);
      val[1] = hi;
    }
    st16(img + x_row * T::K_ROW + 16 * (DC + x_c), val);
  }
  char* vimg = img + T::K_IMG;
  if (v_task) {
    const int sg = kg >> 2, j = kg & 3;
    const int phys = 16 * sg + 8 * (j & 1) + 4 * (j >> 1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x0 = bf16x2_to_f16x2(vx[0][w]), x1 = bf16x2_to_f16x2(vx[1][w]);
      const uint32_t x2 = bf16x2_to_f16x2(vx[2][w]), x3 = bf16x2_to_f16x2(vx[3][w]);
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
  if (tid < D) st16(vimg + tid * T::V_ROW + kBN * 2, zero_u32x4());
}

// First partial slot of split query tile qt of `head` (split chunks of a head
// are its units from query tile h on, in order).
__device__ __forceinline__ int64_t split_slot0(int head, int qt, int h, int units, int n_qt) {
  return static_cast<int64_t>(head) * (units - min(h, n_qt)) + units_before(qt, h) - h;
}

// Normalise O^T (lane = query column my_q, registers = its D/2 dims of this
// lane half) and write the bf16 output row slice and the natural-log LSE.
template <int D>
__device__ __forceinline__ void store_out(const floatx16 (&o)[D / 32], float m, float l, int my_q,
                                          int M, int Hq, int head, int hh, bf16* __restrict__ out,
                                          float* __restrict__ lse) {
  if (my_q >= M) return;
  const float inv = 1.f / l;
  bf16* orow = out + static_cast<size_t>(my_q) * Hq * D + static_cast<size_t>(head) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16 pkk[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pkk[r] = static_cast<bf16>(o[dt][4 * jj + r] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = __builtin_bit_cast(uint2, pkk);
    }
  }
  if (lse != nullptr && hh == 0)
    lse[static_cast<size_t>(head) * M + my_q] = (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// attn_fwd
// ---------------------------------------------------------------------------
template <int D, bool kBias>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const bf16* __restrict__ q, const char* __restrict__ ws, int M, int Hq, int Hkv,
    const float* __restrict__ gain, const float* __restrict__ tau, bf16* __restrict__ out,
    float* __restrict__ lse, int h, int units, char* __restrict__ part) {
  using T = Tile<D, kBias>;
  constexpr int KS = T::KS;
  constexpr int DT = D / 32;             // 32-row tiles of O^T
  constexpr int N_DMA = T::IMG / 1024;   // 1 KiB DMA chunks per tile
  constexpr int NW = kThreads / 64;
  constexpr int NV = DT * 2;             // 16-byte fp16 vectors of partial output per lane

  __shared__ __align__(16) char lds[2][T::IMG];

  // ---- work-group -> (head, unit); unit -> (query tile, chunk)
  const int n_qt = (M + kBM - 1) / kBM;
  int head, u;
  {
    const int b = blockIdx.x;
    int v;
    if ((Hq & 7) == 0) {
      const int hpx = Hq >> 3;            // heads per XCD
      const int xcd = b & 7, slot = b >> 3;
      head = xcd * hpx + slot % hpx;
      v = slot / hpx;
    } else {
      head = b % Hq;
      v = b / Hq;
    }
    u = units - 1 - v;                    // largest query tiles first
  }
  int qt = 0;
  {
    int hi = n_qt;                        // units_before(qt) <= u < units_before(hi)
    while (hi - qt > 1) {
      const int mid = (qt + hi) >> 1;
      if (units_before(mid, h) <= u) qt = mid;
      else hi = mid;
    }
  }
  const int chunk = u - static_cast<int>(units_before(qt, h));
  const int n_chunks = (qt + h) / h;

  const int kvh = head / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBM + wave * 32;   // first of this wave's 32 rows
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
  const int n_kt = q_last / kBN + 1;                  // key tiles of the query tile
  const int t_begin = chunk * 2 * h;
  const int t_end = min(t_begin + 2 * h, n_kt);       // this work-group's key tiles
  const int n_vis = q0 <= q_last ? min(q0 + 31, q_last) / kBN + 1 : 0;  // tiles this wave sees

  // ---- DMA of one tile (IMG bytes) into lds[par]
  const int n_tiles = (M + kBN - 1) / kBN;
  const __amdgpu_buffer_rsrc_t rws =
      make_rsrc(ws + static_cast<size_t>(kvh) * n_tiles * T::IMG,
                static_cast<uint32_t>(n_tiles) * T::IMG);
  // Lane i of a wave instruction moves 16 bytes to M0 + 16 i; the per-lane
  // part of the source offset is one VGPR, the rest a scalar offset.
  const int lane16 = 16 * lane;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // provably wave-uniform
  auto dma_tile = [&](int par, int t) __attribute__((always_inline)) {
    const int tile_off = t * T::IMG;
#pragma unroll
    for (int j = 0; j < (N_DMA + NW - 1) / NW; ++j) {
      const int i = wave_s + NW * j;
      if (i < N_DMA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rws, (__attribute__((address_space(3))) void*)(&lds[par][0] + 1024 * i), 16, lane16,
            tile_off + 1024 * i, 0, 0);
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

  // ---- main loop: one tile per step, one barrier per step.  The DMA issued
  // at step t fills the buffer read at step t + 1; that buffer was last read
  // at step t - 1, which every wave finished before barrier t.
  dma_tile(0, t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    const int par = (t - t_begin) & 1;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA into lds[par] has landed
    __syncthreads();                 // ... and every other wave's
    if (t + 1 < t_end) dma_tile(par ^ 1, t + 1);
    if (t < n_vis) {
      if (t * kBN + kBN - 1 > q0) tile(std::true_type{}, &lds[par][0], t * kBN);
      else tile(std::false_type{}, &lds[par][0], t * kBN);
    }
  }

  float m = m_run;
  float l = l_run + __shfl_xor(l_run, 32);

  if (n_chunks > 1) {
    // ---- split: store this chunk's normalised partial for attn_merge
    char* pw = part + (split_slot0(head, qt, h, units, n_qt) + chunk) * T::PART +
               wave * T::PART_WAVE;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      f16x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = static_cast<_Float16>(o[i >> 1][8 * (i & 1) + e] * inv);
      *reinterpret_cast<f16x8*>(pw + i * 1024 + lane * 16) = x;
    }
    *reinterpret_cast<float2*>(pw + T::PART_O + lane * 8) = make_float2(m, l);
    return;
  }
  store_out<D>(o, m, l, my_q, M, Hq, head, hh, out, lse);
}

// ---------------------------------------------------------------------------
// attn_merge: one work-group (four waves, the rows of attn_fwd's waves) per
// split query tile; lanes read their own partial vectors, so every load is a
// contiguous 1 KiB per wave.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(const char* __restrict__ part, int M,
                                                              int Hq, int h, int units,
                                                              int n_split, bf16* __restrict__ out,
                                                              float* __restrict__ lse) {
  using T = Tile<D, false>;   // partial layout does not depend on the bias
  constexpr int DT = D / 32;
  constexpr int NV = DT * 2;
  const int n_qt = (M + kBM - 1) / kBM;
  const int head = blockIdx.x / n_split;
  const int qt = h + blockIdx.x % n_split;
  const int n_chunks = (qt + h) / h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5;
  const int my_q = qt * kBM + wave * 32 + (lane & 31);
  const char* p0 = part + split_slot0(head, qt, h, units, n_qt) * T::PART + wave * T::PART_WAVE;

  floatx16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = zero16();
  float m = -INFINITY, l = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const char* pr = p0 + static_cast<int64_t>(c) * T::PART;
    const float2 st = *reinterpret_cast<const float2*>(pr + T::PART_O + lane * 8);
    const float m_new = fmaxf(m, st.x);
    const float a = m == m_new ? 1.f : fast_exp2(m - m_new);
    const float b = st.y > 0.f ? st.y * fast_exp2(st.x - m_new) : 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const f16x8 x = *reinterpret_cast<const f16x8*>(pr + i * 1024 + lane * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[i >> 1][8 * (i & 1) + e] = o[i >> 1][8 * (i & 1) + e] * a + static_cast<float>(x[e]) * b;
    }
    l = l * a + b;
    m = m_new;
  }
  store_out<D>(o, m, l, my_q, M, Hq, head, hh, out, lse);
}

template <int D, bool kBias>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int M, int Hq, int Hkv,
                  const float* s, const float* g, const float* t, uint16_t* out, float* lse,
                  void* ws, hipStream_t stream) {
  const Plan p = make_plan<D, kBias>(M, Hq, Hkv);
  char* img = static_cast<char*>(ws);
  char* part = img + p.part_off;
  hipLaunchKernelGGL((kv_pack_kernel<D, kBias>), dim3(static_cast<unsigned>(p.n_tiles * Hkv)),
                     dim3(256), 0, stream, reinterpret_cast<const bf16*>(k),
                     reinterpret_cast<const bf16*>(v), s, M, Hkv, img);
  const dim3 grid(static_cast<unsigned>(p.units * Hq));
  hipLaunchKernelGGL((attn_fwd_kernel<D, kBias>), grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const bf16*>(q), img, M, Hq, Hkv, g, t,
                     reinterpret_cast<bf16*>(out), lse, p.h, static_cast<int>(p.units), part);
  if (p.n_split > 0)
    hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(static_cast<unsigned>(Hq * p.n_split)),
                       dim3(kThreads), 0, stream, part, M, Hq, p.h, static_cast<int>(p.units),
                       static_cast<int>(p.n_split), reinterpret_cast<bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int64_t n, int n_q_heads, int n_kv_heads, int head_dim, bool gated) {
  if (n <= 0) return 0;
  Plan p;
  if (head_dim == 128) p = gated ? make_plan<128, true>(n, n_q_heads, n_kv_heads)
                                 : make_plan<128, false>(n, n_q_heads, n_kv_heads);
  else p = gated ? make_plan<64, true>(n, n_q_heads, n_kv_heads)
                 : make_plan<64, false>(n, n_q_heads, n_kv_heads);
  return p.total;
}

size_t attn_image_bytes_per_kv_head(int64_t n, int head_dim, bool gated) {
  const int64_t n_tiles = (n + kBN - 1) / kBN;
  int64_t img;
  if (head_dim == 128) img = gated ? Tile<128, true>::IMG : Tile<128, false>::IMG;
  else img = gated ? Tile<64, true>::IMG : Tile<64, false>::IMG;
  return static_cast<size_t>(n_tiles * img);
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
