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
// 1. v_pack: per KV head and 64-key tile, the V^T image the main kernel
//    DMAs into LDS, in the caller's workspace: fp16 [d][key], key order
//    permuted inside each 16-key group so that every lane's eight keys of a
//    P.V step are one 16-byte run, the runs of a row XOR-swizzled (unpadded
//    128-byte rows, conflict-free fragment reads); plus (gated) per query head
//    and key the bias in units of q.k, c_h s_j with c_h = gain_h sqrt(d)
//    tau_h, in fp32.  Keys past n are zero.  K is not copied: the main kernel
//    DMAs K tiles straight from k.
// 2. attn_fwd: one work-group = 128 query rows of one query head over a run
//    of their key tiles; four waves of 32 rows; two work-groups per CU (they
//    drift out of phase, so one's softmax and DMA waits overlap the other's
//    MFMAs).  Where a KV group has two query heads and no query tile is
//    split, one eight-wave work-group takes the same 128 rows of both heads
//    instead, so each K and V^T tile is DMAed and read once for the two.
//      * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held
//        in registers for the whole key loop), with the accumulators starting
//        from the tile's bias values c_h s_j (register j holds a fixed key,
//        so the 64 values of a tile are four 16-byte LDS reads per 32-key
//        half), so S~ = q.k + c_h s_j exactly in fp32 and one multiply by
//        alpha = log2(e) / (sqrt(d) tau) gives the logit in log2 units.  K
//        tiles sit in LDS unpadded, 16-byte chunk c of key r at slot
//        c ^ swz(r) (see Tile::swz).
//      * Each lane owns one query column, so the online-softmax statistics are
//        lane-local plus one exchange between lane halves; the running max
//        only moves when a tile raises it by more than 2^8 (lazy rescaling).
//      * O^T = V^T P^T on v_mfma_f32_32x32x16_f16 with P taken straight from
//        registers.  P and V are fp16 for this product: bf16 P (8-bit
//        mantissa) costs up to ~3e-3 of output error on peaked rows on top of
//        the bf16 output rounding.  O accumulates in fp32.
//      * The softmax runs on fp32 logits in log2 units: the logit scale is
//        folded into the exponent's FMA, and the row sum adds the fp16 P
//        values that the P.V product uses (v_dot2_f32_f16 against (1, 1)).
//      * Software-pipelined steps: step t runs the QK MFMAs of tile t + 1
//        with the exponentials of tile t placed between them, half after
//        the k-steps of the QK product and half after the first P.V
//        MFMAs, in an order fixed in the source (independent work for the
//        MFMA pipe while the VALU runs the softmax, within one wave as well
//        as across the two work-groups of a CU).
//      * Tiles arrive by buffer-to-LDS DMA (buffer_load_dwordx4 ... lds): K
//        straight from k (and the tile's bias values), two tiles ahead, V^T
//        images one tile ahead, each in its own double-buffered LDS ring; no
//        staging registers, no LDS store instructions, one barrier per tile.
//      * Causal masking only on diagonal tiles; tiles above a wave's rows are
//        skipped.
//      * Heads of one KV group are pinned to one XCD (work-groups are dealt
//        round-robin over the 8 XCDs) so its K/V stays in that L2; within an
//        XCD the units of the longest query tiles go first.
//      * Split keys.  When few query tiles exist (short kept prefixes), the
//        longest query tile's key loop would outlast the average work of a
//        resident work-group many times over.  Then the key tiles of query
//        tile qt are cut into ceil((qt + 1) / h) chunks of 2h tiles, each a
//        work-group of its own.  Every chunk stores its normalised partial
//        output (fp16) and its running max and sum in the workspace.
// 3. attn_merge (only when some query tile is split): one single-wave
//    work-group per (head, split query tile, wave) combines the chunks'
//    partials in chunk order and writes the output.  A third launch rather
//    than a last-arriver merge inside attn_fwd: the agent-scope fences such a
//    merge needs (L2 write-back and invalidate on every chunk) cost more than
//    the whole split saves.
#include <algorithm>
#include <cmath>
#include <type_traits>
#include <vector>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kSets = 1;                  // 32-row query sets per wave (2 spills at d = 128)
constexpr int kBM = 128 * kSets;          // query rows per work-group
constexpr int kBN = 64;                   // keys per tile
constexpr int kThreads = 256;             // four waves of 32 * kSets rows
constexpr int kSlots = 512 / kSets;       // resident work-groups: 2 / kSets per CU
constexpr int kTilesPerQt = kBM / kBN;
constexpr int kMinChunk = 8 / kTilesPerQt;   // chunks are at least 8 key tiles
constexpr double kChunkScale = 1.3;           // chunk length / average tile steps per slot
constexpr float kRescaleThreshold = 8.f;  // log2 units

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __fp16 f16x2 __attribute__((ext_vector_type(2)));   // cvt_pkrtz / fdot2 operand type

template <int D, bool kBias>
struct Tile {
  static constexpr int KS = D / 16;                       // k-steps of S^T
  static constexpr int K_ROW = D * 2;                     // LDS bytes per key: 16-byte chunks,
                                                          //   chunk c of key r at slot c ^ swz(r)
  static constexpr int K_IMG = kBN * K_ROW;               // one K tile in LDS
  static constexpr int V_ROW = kBN * 2;                   // bytes: 16-byte piece c of dim row r at
                                                          //   slot c ^ vswz(r)
  static constexpr int V_IMG = D * V_ROW;                 // one V^T tile (workspace and LDS)
  static constexpr int S_TILE = kBN * 4;                  // one head's bias values of a tile (fp32)
  // XOR key of K row r: 16 consecutive rows hit 16 different 16-byte slots
  // modulo 256 bytes (rows are 256 bytes at d = 128, 128 bytes at d = 64), so
  // the fragment reads are free of bank conflicts.
  static __host__ __device__ constexpr int swz(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
  }
  // XOR key of V^T row r (128-byte rows): the 16 rows one pass of a fragment
  // read serves, eight of each parity, hit 16 different 16-byte bank slots.
  static __host__ __device__ constexpr int vswz(int r) { return (r >> 1) & 7; }
  static_assert(K_IMG % 1024 == 0 && V_IMG % 1024 == 0, "tiles must be whole 1 KiB DMA chunks");
  // One split chunk's partial state: per 32-row set (kSets per wave), the
  // lane-major fp16 output (D bytes per lane in 16-byte vectors) and a
  // (max, sum) pair per lane.
  static constexpr int PART_O = D * 64;
  static constexpr int PART_SET = PART_O + 8 * 64;
  static constexpr int PART = 4 * kSets * PART_SET;
};

// Work-groups of one head before query tile q when query tile i has
// ceil((i + 1) / h) chunks: sum_{j=1..q} ceil(j / h).
__host__ __device__ __forceinline__ int64_t units_before(int64_t q, int64_t h) {
  const int64_t a = q / h, r = q % h;
  return h * a * (a + 1) / 2 + r * (a + 1);
}

// Query tile qt walks kTilesPerQt * (qt + 1) key tiles (fewer on a ragged
// last tile).  Split chunks are kTilesPerQt * h key tiles, h query tiles'
// worth, so query tile qt has ceil((qt + 1) / h) chunks (also on a ragged last
// tile) and h = n_qt means no split.
struct Plan {
  int n_qt, n_tiles, h;
  int64_t units;       // work-groups per head
  int64_t n_split;     // query tiles per head with more than one chunk
  int64_t n_part;      // split chunks per head
  size_t img_bytes, sc_off, part_off, total;
};

// Chunk parameter h: no split unless the longest query tile's walk exceeds
// the average number of tile steps per resident work-group; then chunks of
// 1.3x that average, never shorter than 8 key tiles (each split chunk pays a
// partial-state round trip).  Measured at 16 heads: 1.0x-1.3x is best for
// 2304 kept rows, 1.3x-1.5x for 4352 (25% faster than 1.0x).
int base_h(int n_qt, int Hq) {
  const double steps = static_cast<double>(kTilesPerQt) * n_qt * (n_qt + 1) / 2;
  const double avg = static_cast<double>(Hq) * steps / kSlots;
  int64_t h = n_qt;
  if (static_cast<double>(kTilesPerQt) * n_qt > avg)
    h = std::max<int64_t>(kMinChunk, static_cast<int64_t>(std::ceil(kChunkScale * avg / kTilesPerQt)));
  return static_cast<int>(std::max<int64_t>(std::min<int64_t>(h, n_qt), 1));
}

// Makespan of the launch in key-tile steps: work-groups in launch order (the
// kernel's: longest query tiles first, last chunk first, heads interleaved)
// onto kSlots resident slots, each busy for its key tiles plus two (three
// when it writes a split partial).  Durations are whole steps and a greedy
// list schedule never starts a work-group earlier than the one before it, so
// the slots are counted per free time and a pointer walks forward.
int simulate_split(int64_t M, int n_qt, int h, int Hq) {
  auto walk = [&](int qt) {
    return static_cast<int>((std::min<int64_t>(static_cast<int64_t>(kBM) * (qt + 1), M) + kBN - 1) / kBN);
  };
  int64_t total = 0;
  int longest = 0;
  for (int qt = 0; qt < n_qt; ++qt) {
    const int nch = (qt + h) / h;
    total += static_cast<int64_t>(walk(qt) + (2 + (nch > 1 ? 1 : 0)) * nch) * Hq;
    longest = std::max(longest, std::min(kTilesPerQt * h, walk(qt)) + 3);
  }
  // list scheduling ends by total / slots + the longest work-group
  std::vector<int> free_at(static_cast<size_t>(total / kSlots + longest + 2), 0);
  free_at[0] = kSlots;
  int t = 0, end = 0;
  for (int qt = n_qt - 1; qt >= 0; --qt) {
    const int nch = (qt + h) / h;
    for (int c = nch - 1; c >= 0; --c) {
      const int d = std::min(kTilesPerQt * h, walk(qt) - kTilesPerQt * h * c) + 2 + (nch > 1 ? 1 : 0);
      for (int head = 0; head < Hq; ++head) {
        while (free_at[t] == 0) ++t;
        --free_at[t];
        ++free_at[t + d];
        end = std::max(end, t + d);
      }
    }
  }
  return end;
}

// Short prefixes: the chunk one step shorter than base_h's when the dispatch
// simulation finishes more than 6 % sooner with it.  The simulation ignores
// the merge and partial traffic that more chunks add and that a lone
// work-group runs faster on its CU, so only clear wins are taken.  Measured
// at 16 heads (base -> chosen h): 2000 rows 43.4 -> 38.5 us, 2304 rows 45.1 ->
// 43.5 us, 2600 rows 52.9 -> 51.6 us, 3000 rows 63.0 -> 61.1 us; at 1800 and
// 3500-7000 rows, where the simulation keeps base_h, the shorter chunk
// measured 0-12 % slower.
int choose_h(int64_t M, int n_qt, int Hq) {
  int h = base_h(n_qt, Hq);
  if (h > kMinChunk && h < n_qt &&
      simulate_split(M, n_qt, h - 1, Hq) < 0.94 * simulate_split(M, n_qt, h, Hq))
    h -= 1;
  return h;
}

template <int D, bool kBias>
Plan make_plan(int64_t M, int Hq, int Hkv) {
  using T = Tile<D, kBias>;
  Plan p{};
  p.n_qt = static_cast<int>((M + kBM - 1) / kBM);
  p.n_tiles = static_cast<int>((M + kBN - 1) / kBN);
  const int64_t h = choose_h(M, p.n_qt, Hq);
  p.h = static_cast<int>(h);
  p.units = units_before(p.n_qt, h);
  p.n_split = std::max<int64_t>(p.n_qt - h, 0);
  p.n_part = p.units - std::min<int64_t>(h, p.n_qt);
  p.img_bytes = static_cast<size_t>(p.n_tiles) * Hkv * T::V_IMG;
  p.sc_off = p.img_bytes;
  p.part_off = p.sc_off + ((static_cast<size_t>(Hq) * p.n_tiles * T::S_TILE + 255) & ~size_t(255));
  p.total = p.part_off + static_cast<size_t>(Hq) * p.n_part * T::PART;
  return p;
}

__device__ __forceinline__ floatx16 mfma_f16(f16x8 a, f16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two bf16 (one dword) -> two fp16 (one dword), round toward zero.  Exact for
// bf16 values in fp16's normal range; larger magnitudes saturate at 65504,
// smaller ones lose low bits as fp16 subnormals (absolute error < 6e-8).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __uint_as_float(x << 16);
  const float hi = __uint_as_float(x & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<bf16>(x));  // round to nearest even
}

// ---------------------------------------------------------------------------
// v_pack: one work-group per (tile, KV head) builds the tile's V^T image in
// the workspace (fp16, [d][key] with the key order permuted inside each
// 16-key group so that every lane's eight keys of a P.V step are one 16-byte
// run; the runs of row r at slot run ^ vswz(r); keys past n zero).  In a
// gated call each work-group also
// stores, for the query heads of its KV group and the tile's keys, the bias
// c_h s_j (fp32, [head][key]).  K needs no pass of its own: the attention
// kernel DMAs its tiles straight from k.
// ---------------------------------------------------------------------------
template <int D, bool kBias>
__global__ __launch_bounds__(256) void v_pack_kernel(const bf16* __restrict__ v,
                                                     const float* __restrict__ key_score,
                                                     const float* __restrict__ gain,
                                                     const float* __restrict__ tau, int M, int Hq,
                                                     int Hkv, char* __restrict__ ws,
                                                     char* __restrict__ sc) {
  using T = Tile<D, kBias>;
  const int n_tiles = (M + kBN - 1) / kBN;
  const int tile = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int tid = threadIdx.x;
  char* vimg = ws + (static_cast<size_t>(kvh) * n_tiles + tile) * T::V_IMG;
  const uint32_t kv_row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
  const uint32_t kv_bytes = kv_row_bytes * static_cast<uint32_t>(M);
  const uint32_t off0 = static_cast<uint32_t>(tile) * kBN * kv_row_bytes;
  const uint32_t left = off0 < kv_bytes ? kv_bytes - off0 : 0u;
  constexpr int DC = D / 8;                        // 16-byte data chunks per row
  static_assert(16 * DC <= 256, "v_pack tiling");
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(reinterpret_cast<const char*>(v + static_cast<size_t>(kvh) * D) + off0, left);
  // This thread's task: 4 keys x 8 dims; keys 4 kg + i sit at positions
  // 16 s + 8 h' + 4 b + i with s = kg / 4, h' = (kg % 4) & 1, b = (kg % 4) >> 1.
  // Every load is issued before the first store.
  const int kg = tid % 16, dc = tid / 16;
  const int key = tile * kBN + tid;
  const bool score_task = kBias && tid < kBN;
  const float x_s = (score_task && key < M) ? key_score[key] : 0.f;
  if (dc < DC) {
    u32x4 vx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vx[i] = bload16(rv, (4 * kg + i) * kv_row_bytes + 16 * dc);
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
      const int pc = phys >> 3, pb = (2 * phys) & 15;   // 16-byte piece, byte within it
      *reinterpret_cast<uint2*>(vimg + d0 * T::V_ROW + ((pc ^ T::vswz(d0)) << 4) + pb) = lo;
      *reinterpret_cast<uint2*>(vimg + (d0 + 1) * T::V_ROW + ((pc ^ T::vswz(d0 + 1)) << 4) + pb) = hi;
    }
  }
  if (score_task) {
    // the key's bias in units of q.k for each head of this group:
    // c_h s_j with c_h = gain_h sqrt(d) tau_h
    const int G = Hq / Hkv;
    for (int g = 0; g < G; ++g) {
      const int h = kvh * G + g;
      const float c = gain[h] * sqrtf(static_cast<float>(D)) * tau[h];
      reinterpret_cast<float*>(sc)[(static_cast<size_t>(h) * n_tiles + tile) * kBN + tid] = c * x_s;
    }
  }
}

// First partial slot of split query tile qt of `head` (split chunks of a head
// are its units from query tile h on, in order).
__device__ __forceinline__ int64_t split_slot0(int head, int qt, int h, int units, int n_qt) {
  return static_cast<int64_t>(head) * (units - min(h, n_qt)) + units_before(qt, h) - h;
}

// Normalise O^T (lane = query column my_q, registers = its D/2 dims of this
// lane half) and write the bf16 output row slice, the natural-log LSE and,
// for a training forward, the fp32 output before rounding (out32).
template <int D>
__device__ __forceinline__ void store_out(const floatx16 (&o)[D / 32], float m, float l, int my_q,
                                          int M, int Hq, int head, int hh, bf16* __restrict__ out,
                                          float* __restrict__ lse, float* __restrict__ out32) {
  if (my_q >= M) return;
  const float inv = 1.f / l;
  const size_t row = static_cast<size_t>(my_q) * Hq * D + static_cast<size_t>(head) * D;
  bf16* orow = out + row;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16 pkk[4];
      float4 f;
      f.x = o[dt][4 * jj] * inv; f.y = o[dt][4 * jj + 1] * inv;
      f.z = o[dt][4 * jj + 2] * inv; f.w = o[dt][4 * jj + 3] * inv;
      pkk[0] = static_cast<bf16>(f.x); pkk[1] = static_cast<bf16>(f.y);
      pkk[2] = static_cast<bf16>(f.z); pkk[3] = static_cast<bf16>(f.w);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = __builtin_bit_cast(uint2, pkk);
      if (out32 != nullptr)
        *reinterpret_cast<float4*>(out32 + row + 32 * dt + 8 * jj + 4 * hh) = f;
    }
  }
  if (lse != nullptr && hh == 0)
    lse[static_cast<size_t>(head) * M + my_q] = (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// attn_fwd
// ---------------------------------------------------------------------------
// HG query heads per work-group: 1, or 2 when a KV group has two query heads
// and no query tile is split (then the work-group's eight waves, four per
// head, share one K and one V^T ring: half the DMA and LDS traffic per MFMA;
// measured 2-4 % faster at 8448 kept rows, slower where query tiles split).
template <int D, bool kBias, int HG>
__global__ __launch_bounds__(kThreads * HG, 2 / (kSets * HG)) void attn_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const char* __restrict__ ws,
    const char* __restrict__ bias_frag, int M, int Hq, int Hkv, const float* __restrict__ gain,
    const float* __restrict__ tau, bf16* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ out32, int h, int units, char* __restrict__ part) {
  using T = Tile<D, kBias>;
  constexpr int KS = T::KS;
  constexpr int DT = D / 32;                 // 32-row tiles of O^T
  static_assert(HG == 1 || HG == 2, "query heads per work-group");
  constexpr int NW = kThreads * HG / 64;     // waves of the work-group (DMA pieces go over all)
  constexpr int NV = DT * 2;                 // 16-byte fp16 vectors of partial output per lane
  constexpr int N_DMA_K = T::K_IMG / 1024;   // 1 KiB DMA chunks per K tile
  constexpr int N_DMA_V = T::V_IMG / 1024;   // ... per V^T image
  constexpr int NKJ = (N_DMA_K + NW - 1) / NW;

  // K ring (with the tile's packed scores) runs one tile ahead of the V^T
  // ring: step t reads K(t+1) and V^T(t) while K(t+2) and V^T(t+1) land.
  // Each ring stage is an LDS object of its own, always named at compile
  // time: the compiler tracks DMA into LDS per object and makes a read of an
  // object wait for every DMA in flight into it, so two stages of one array
  // would serialize each tile's reads behind the next tiles' DMA.
  __shared__ __align__(16) char lds_k0[T::K_IMG];
  __shared__ __align__(16) char lds_k1[T::K_IMG];
  __shared__ __align__(16) char lds_s0[kBias ? HG * T::S_TILE : 16];   // a bias tile per head
  __shared__ __align__(16) char lds_s1[kBias ? HG * T::S_TILE : 16];
  __shared__ __align__(16) char lds_v0[T::V_IMG];
  __shared__ __align__(16) char lds_v1[T::V_IMG];
  auto ring_k = [&](auto b_c) __attribute__((always_inline)) -> char* {
    if constexpr (decltype(b_c)::value) return lds_k1; else return lds_k0;
  };
  auto ring_s = [&](auto b_c) __attribute__((always_inline)) -> char* {
    if constexpr (decltype(b_c)::value) return lds_s1; else return lds_s0;
  };
  auto ring_v = [&](auto b_c) __attribute__((always_inline)) -> char* {
    if constexpr (decltype(b_c)::value) return lds_v1; else return lds_v0;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  // ---- work-group -> (head group, unit); unit -> (query tile, chunk).  A
  // head group is HG consecutive query heads (with HG = 2, a KV group); wave
  // w serves head HG-group head + w / 4 (the same head -> XCD rule either way).
  const int n_qt = (M + kBM - 1) / kBM;
  const int n_hg = Hq / HG;
  const int wave_g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // provably wave-uniform
  int head, u;
  {
    const int b = blockIdx.x;
    int v, hg;
    if ((n_hg & 7) == 0) {
      const int hpx = n_hg >> 3;          // head groups per XCD
      const int xcd = b & 7, slot = b >> 3;
      hg = xcd * hpx + slot % hpx;
      v = slot / hpx;
    } else {
      hg = b % n_hg;
      v = b / n_hg;
    }
    head = hg * HG + (wave_g >> 2);
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
  const int wave = (tid >> 6) & 3;           // wave within its head
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBM + wave * 32 * kSets;   // first of this wave's rows
  int my_q[kSets];   // this lane's query in each set
#pragma unroll
  for (int r = 0; r < kSets; ++r) my_q[r] = q0 + 32 * r + l32;

  const float t_h = kBias ? tau[head] : 1.f;
  const float alpha = kLog2e / (sqrtf(static_cast<float>(D)) * t_h);

  // ---- Q~ fragments (B operand): lane holds Q[my_q][16 s + 8 hh .. + 7]
  bf16x8 qf[kSets][KS];
  {
    const uint32_t q_row_bytes = static_cast<uint32_t>(Hq) * D * 2;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(q + static_cast<size_t>(head) * D, q_row_bytes * static_cast<uint32_t>(M));
#pragma unroll
    for (int r = 0; r < kSets; ++r) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        qf[r][s] = as_bf16x8(
            bload16(rq, static_cast<uint32_t>(my_q[r]) * q_row_bytes + (16 * s + 8 * hh) * 2));
    }

  }

  floatx16 o[kSets][DT];
#pragma unroll
  for (int r = 0; r < kSets; ++r) {
#pragma unroll
    for (int i = 0; i < DT; ++i) o[r][i] = zero16();
  }
  float m_run[kSets], l_run[kSets];
#pragma unroll
  for (int r = 0; r < kSets; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  const int q_last = min(qt * kBM + kBM, M) - 1;
  const int n_kt = q_last / kBN + 1;                  // key tiles of the query tile
  const int t_begin = chunk * kTilesPerQt * h;
  const int t_end = min(t_begin + kTilesPerQt * h, n_kt);   // this work-group's key tiles
  // tiles this wave sees (its rows end at or before the tile holding q0 + 31 * kSets + 31)
  const int n_vis = min(q0 <= q_last ? min(q0 + 32 * kSets - 1, q_last) / kBN + 1 : 0, t_end);

  // ---- DMA into LDS.  Lane i of a wave instruction moves 16 bytes to
  // M0 + 16 i.  K tiles come straight from k: the lane that fills LDS slot s
  // of key r fetches chunk s ^ swz(r) of that key's row (the XOR swizzle
  // keeps the fragment reads free of bank conflicts without padding); keys
  // past n read as zeros (buffer range check on the full per-lane offset).
  // V^T images and packed scores come from the workspace.
  const int n_tiles = (M + kBN - 1) / kBN;
  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k, kv_row * static_cast<uint32_t>(M));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(ws + static_cast<size_t>(kvh) * n_tiles * T::V_IMG,
                static_cast<uint32_t>(n_tiles) * T::V_IMG);
  const __amdgpu_buffer_rsrc_t rsc =
      make_rsrc(bias_frag + static_cast<size_t>(head) * n_tiles * T::S_TILE,
                static_cast<uint32_t>(n_tiles) * T::S_TILE);
  const int lane16 = 16 * lane;
  const int wave_s = wave_g;
  uint32_t koff[NKJ];   // this lane's source offset (within a tile) per K DMA instruction
#pragma unroll
  for (int jj = 0; jj < NKJ; ++jj) {
    const int byte = 1024 * (wave_s + NW * jj) + lane16;
    const int r = byte / T::K_ROW, slot = (byte % T::K_ROW) / 16;
    koff[jj] = static_cast<uint32_t>(r) * kv_row + static_cast<uint32_t>(kvh) * D * 2 +
               static_cast<uint32_t>((slot ^ T::swz(r)) * 16);
  }
  auto dma_k = [&](auto buf, int t) __attribute__((always_inline)) {
    const uint32_t tile_off = static_cast<uint32_t>(t) * kBN * kv_row;
#pragma unroll
    for (int jj = 0; jj < NKJ; ++jj) {
      const int j = wave_s + NW * jj;
      if (j < N_DMA_K)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(ring_k(buf) + 1024 * j), 16,
            static_cast<int>(tile_off + koff[jj]), 0, 0, 0);
    }
    if (kBias && (wave_s & 3) == 3 && lane < T::S_TILE / 16) {   // a wave per head
      const int s_off = t * T::S_TILE;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsc, (__attribute__((address_space(3))) void*)(ring_s(buf) + (wave_s >> 2) * T::S_TILE), 16,
          lane16, s_off, 0, 0);
    }
  };
  auto dma_v = [&](auto buf, int t) __attribute__((always_inline)) {
    // (the tile offset is formed outside the loop: written inline in the
    // builtin's offset argument, the host pass drops this kernel's stub)
    const int tile_off = t * T::V_IMG;
#pragma unroll
    for (int jj = 0; jj < (N_DMA_V + NW - 1) / NW; ++jj) {
      const int j = wave_s + NW * jj;
      if (j < N_DMA_V)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(ring_v(buf) + 1024 * j), 16, lane16,
            tile_off + 1024 * j, 0, 0);
    }
  };

  // ---- S^T of one tile for every set: each K fragment read feeds kSets
  // MFMAs.  Lane (l32, hh) reads chunk 2 ks + hh of key 32 t2 + l32, stored at
  // slot (2 ks + hh) ^ swz(l32): the per-k-step address is one XOR.
  const uint32_t k_base = static_cast<uint32_t>(l32) * T::K_ROW + ((hh ^ T::swz(l32)) << 4);
  // V^T fragment of P.V step ps: dim row 32 dt + l32, piece 2 ps + hh (its
  // XOR key depends on l32 only)
  uint32_t v_off[4];
#pragma unroll
  for (int ps = 0; ps < 4; ++ps)
    v_off[ps] = static_cast<uint32_t>(l32) * T::V_ROW + (((2 * ps + hh) ^ T::vswz(l32)) << 4);
  auto qk = [&](const char* kimg, const char* simg, floatx16 (&s)[kSets][2])
      __attribute__((always_inline)) {
    // S~ starts from the keys' bias c_h s_j (register j of 32-key half t2
    // holds key 32 t2 + 8 (j/4) + 4 hh + j%4), so S~ = q.k + c_h s_j
#pragma unroll
    for (int r = 0; r < kSets; ++r) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        if (kBias) {
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const float4 b = *reinterpret_cast<const float4*>(simg + 4 * (32 * t2 + 8 * jg + 4 * hh));
            s[r][t2][4 * jg] = b.x; s[r][t2][4 * jg + 1] = b.y;
            s[r][t2][4 * jg + 2] = b.z; s[r][t2][4 * jg + 3] = b.w;
          }
        } else {
          s[r][t2] = zero16();
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint32_t off = k_base ^ static_cast<uint32_t>(32 * ks);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kimg + off + 32 * t2 * T::K_ROW);
#pragma unroll
        for (int r = 0; r < kSets; ++r) s[r][t2] = mfma_32x32x16(a, qf[r][ks], s[r][t2]);
      }
    }

  };

  // ---- online softmax of one set's tile, in two parts so that the next
  // tile's QK MFMAs can go between them: (1) here, causal mask (compile-time
  // MASK, diagonal tile only) and running max, raising it lazily (only when a
  // tile exceeds it by more than 2^8, which also rescales O and l); (2) in
  // the step below, P = exp2(S * alpha - m) as fp16 pairs [32-key
  // half][pair], the logit scale folded into the exponent's FMA.
  auto softmax_max = [&](auto mask_c, int r, floatx16 (&s)[2], int kb)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    // key kb + 32 t2 + 8 (j / 4) + 4 hh + j % 4 is visible iff
    // 32 t2 + 8 (j / 4) + j % 4 <= my_q - kb - 4 hh
    const int lim = my_q[r] - kb - 4 * hh;
    float mx = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = s[t2][j];
        if (MASK && 32 * t2 + 8 * (j >> 2) + (j & 3) > lim) x = -INFINITY;
        s[t2][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * alpha;
    }
    // Wave-uniform and rare after the first tiles: a real branch, not a select.
    if (__builtin_expect(__builtin_amdgcn_readfirstlane(__any(mx > m_run[r] + kRescaleThreshold)), 0)) {
      const float m_new = fmaxf(m_run[r], mx);
      const float corr = fast_exp2(m_run[r] - m_new);
      m_run[r] = m_new;
      l_run[r] *= corr;
#pragma unroll
      for (int i = 0; i < DT; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) o[r][i][j] *= corr;
      }
    }
  };
  // ---- one pipelined step, written out in issue order (sched_barrier fences
  // keep the compiler from regrouping it): S(t+1) = K~(t+1) Q~^T, one k-step
  // at a time with the next k-step's K fragments already in flight, each
  // k-step followed by exponentials of S(t)'s first 32 keys; then O += V(t)
  // P(t), 32 dims of V^T per fragment read, the first two of its four 16-key
  // steps followed by the exponentials of the last 32 keys (which the last two
  // steps consume).  The row sum adds the fp16 P values that the P.V product
  // uses (v_dot2_f32_f16 against (1, 1)), in key order.  sc holds S(t), sn
  // receives S(t+1); past the last tile the extra QK reads stale LDS and its
  // result is never used.
  // par_c: the step's parity (K~(t+1) in stage 1 - par, V^T(t) in stage par)
  auto step = [&](auto mask_c, auto par_c, floatx16 (&sc)[kSets][2], floatx16 (&sn)[kSets][2],
                  int t) __attribute__((always_inline)) {
    static_assert(kSets == 1, "the interleaved step is written for one query set");
    constexpr int par = decltype(par_c)::value;
    softmax_max(mask_c, 0, sc[0], t * kBN);
    const char* kimg = ring_k(std::integral_constant<int, 1 - par>{});
    const char* simg = ring_s(std::integral_constant<int, 1 - par>{}) + (wave_g >> 2) * T::S_TILE;
    const char* vimg = ring_v(par_c);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      if (kBias) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const float4 b = *reinterpret_cast<const float4*>(simg + 4 * (32 * t2 + 8 * jg + 4 * hh));
          sn[0][t2][4 * jg] = b.x; sn[0][t2][4 * jg + 1] = b.y;
          sn[0][t2][4 * jg + 2] = b.z; sn[0][t2][4 * jg + 3] = b.w;
        }
      } else {
        sn[0][t2] = zero16();
      }
    }
    const float nm = -m_run[0];
    const f16x2 ones = {static_cast<__fp16>(1.f), static_cast<__fp16>(1.f)};
    float rs = 0.f;
    uint32_t pk[2][8];
    auto exp_pair = [&](int t2, int jj) __attribute__((always_inline)) {
      const float p0 = fast_exp2(__builtin_fmaf(sc[0][t2][jj], alpha, nm));
      const float p1 = fast_exp2(__builtin_fmaf(sc[0][t2][jj + 1], alpha, nm));
      const f16x2 hv = __builtin_amdgcn_cvt_pkrtz(p0, p1);
      rs = __builtin_amdgcn_fdot2(hv, ones, rs, false);
      pk[t2][jj >> 1] = __builtin_bit_cast(uint32_t, hv);
    };
    bf16x8 ka[2][2];
    auto kread = [&](int ks, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
      const uint32_t off = k_base ^ static_cast<uint32_t>(32 * ks);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        dst[t2] = *reinterpret_cast<const bf16x8*>(kimg + off + 32 * t2 * T::K_ROW);
    };
    f16x8 va[2][DT];
    auto vread = [&](int ps, f16x8 (&dst)[DT]) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dst[dt] = *reinterpret_cast<const f16x8*>(vimg + 32 * dt * T::V_ROW + v_off[ps]);
    };
    kread(0, ka[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) kread(ks + 1, ka[(ks + 1) & 1]);
      else vread(0, va[0]);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) sn[0][t2] = mfma_32x32x16(ka[ks & 1][t2], qf[0][ks], sn[0][t2]);
#pragma unroll
      for (int e = 0; e < 8 / KS; ++e) exp_pair(0, 2 * ((8 / KS) * ks + e));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      if (ps + 1 < 4) vread(ps + 1, va[(ps + 1) & 1]);
      const uint32_t* src = &pk[ps >> 1][4 * (ps & 1)];
      const u32x4 pv4 = {src[0], src[1], src[2], src[3]};
      const f16x8 b = __builtin_bit_cast(f16x8, pv4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[0][dt] = mfma_f16(va[ps & 1][dt], b, o[0][dt]);
      if (ps < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) exp_pair(1, 8 * ps + 2 * e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run[0] += rs;
  };

  // ---- main loop, one barrier per tile.  At the barrier of step j the DMA of
  // K~(t+1) and V^T(t) (issued one step earlier) has landed and every wave is
  // done with K~(t) and V^T(t-1), whose buffers the new DMA refills.
  floatx16 sa[kSets][2], sb[kSets][2];
  dma_k(B0{}, t_begin);
  dma_v(B0{}, t_begin);
  if (t_begin + 1 < t_end) dma_k(B1{}, t_begin + 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t_begin < n_vis) qk(ring_k(B0{}), ring_s(B0{}) + (wave_g >> 2) * T::S_TILE, sa);
  // step j = t - t_begin has parity par (the loop below takes steps in pairs)
  auto run = [&](auto par_c, floatx16 (&sc)[kSets][2], floatx16 (&sn)[kSets][2], int t)
      __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA has landed
    __syncthreads();                 // ... and every other wave's
    if (t + 2 < t_end) dma_k(par_c, t + 2);
    if (t + 1 < t_end) dma_v(std::integral_constant<int, 1 - par>{}, t + 1);
    if (t < n_vis) {
      if (t * kBN + kBN - 1 > q0) step(std::true_type{}, par_c, sc, sn, t);   // the diagonal tile
      else step(std::false_type{}, par_c, sc, sn, t);
    }
  };
  for (int t = t_begin; t < t_end; t += 2) {
    run(B0{}, sa, sb, t);
    if (t + 1 < t_end) run(B1{}, sb, sa, t + 1);
  }

  // ---- epilogue per set: the output, or this chunk's normalised partial
#pragma unroll
  for (int r = 0; r < kSets; ++r) {
    const float m = m_run[r];
    const float l = l_run[r] + __shfl_xor(l_run[r], 32);
    if (n_chunks > 1) {
      char* pw = part + (split_slot0(head, qt, h, units, n_qt) + chunk) * T::PART +
                 (kSets * wave + r) * T::PART_SET;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        f16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = static_cast<_Float16>(o[r][i >> 1][8 * (i & 1) + e] * inv);
        // streamed past L2: read once, by the merge launch
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x),
                                    reinterpret_cast<u32x4*>(pw + i * 1024 + lane * 16));
      }
      __builtin_nontemporal_store(m, reinterpret_cast<float*>(pw + T::PART_O + lane * 8));
      __builtin_nontemporal_store(l, reinterpret_cast<float*>(pw + T::PART_O + lane * 8 + 4));
    } else {
      store_out<D>(o[r], m, l, my_q[r], M, Hq, head, hh, out, lse, out32);
    }
  }
}

// ---------------------------------------------------------------------------
// attn_merge: one single-wave work-group per (head, split query tile, wave of
// attn_fwd), on the XCD whose L2 received that head's partials (the same
// head -> XCD rule as attn_fwd).  Lanes read their own partial vectors, so
// every load is a contiguous 1 KiB.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_merge_kernel(const char* __restrict__ part, int M,
                                                        int Hq, int h, int units, int n_split,
                                                        bf16* __restrict__ out,
                                                        float* __restrict__ lse,
                                                        float* __restrict__ out32) {
  using T = Tile<D, false>;   // partial layout does not depend on the bias
  constexpr int DT = D / 32;
  constexpr int NV = DT * 2;
  constexpr int NW = kThreads / 64;
  const int n_qt = (M + kBM - 1) / kBM;
  int head, rest;
  {
    const int b = blockIdx.x;
    if ((Hq & 7) == 0) {
      const int hpx = Hq >> 3;
      const int xcd = b & 7, slot = b >> 3;
      head = xcd * hpx + slot % hpx;
      rest = slot / hpx;
    } else {
      head = b % Hq;
      rest = b / Hq;
    }
  }
  const int qt = h + rest / NW;
  const int wave = rest % NW;
  const int n_chunks = (qt + h) / h;
  const int lane = threadIdx.x;
  const int hh = lane >> 5;
  const char* p_base = part + split_slot0(head, qt, h, units, n_qt) * T::PART;

  for (int r = 0; r < kSets; ++r) {
    const int my_q = qt * kBM + wave * 32 * kSets + 32 * r + (lane & 31);
    const char* p0 = p_base + (kSets * wave + r) * T::PART_SET;
    floatx16 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = zero16();
    float m = -INFINITY, l = 0.f;
    // up to four chunks' partials in flight at once, combined in chunk order
    for (int c0 = 0; c0 < n_chunks; c0 += 4) {
      const int nc = min(4, n_chunks - c0);
      float2 st[4];
      f16x8 x[4][NV];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < nc) {
          const char* pr = p0 + static_cast<int64_t>(c0 + k) * T::PART;
          st[k] = *reinterpret_cast<const float2*>(pr + T::PART_O + lane * 8);
#pragma unroll
          for (int i = 0; i < NV; ++i) x[k][i] = *reinterpret_cast<const f16x8*>(pr + i * 1024 + lane * 16);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < nc) {
          const float m_new = fmaxf(m, st[k].x);
          const float a = m == m_new ? 1.f : fast_exp2(m - m_new);
          const float b = st[k].y > 0.f ? st[k].y * fast_exp2(st[k].x - m_new) : 0.f;
#pragma unroll
          for (int i = 0; i < NV; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              o[i >> 1][8 * (i & 1) + e] = o[i >> 1][8 * (i & 1) + e] * a + static_cast<float>(x[k][i][e]) * b;
          }
          l = l * a + b;
          m = m_new;
        }
      }
    }
    store_out<D>(o, m, l, my_q, M, Hq, head, hh, out, lse, out32);
  }
}

template <int D, bool kBias>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int M, int Hq, int Hkv,
                  const float* s, const float* g, const float* t, uint16_t* out, float* lse,
                  float* out32, void* ws, hipStream_t stream) {
  const Plan p = make_plan<D, kBias>(M, Hq, Hkv);
  char* img = static_cast<char*>(ws);
  char* sc = img + p.sc_off;
  char* part = img + p.part_off;
  hipLaunchKernelGGL((v_pack_kernel<D, kBias>), dim3(static_cast<unsigned>(p.n_tiles * Hkv)),
                     dim3(256), 0, stream, reinterpret_cast<const bf16*>(v), s, g, t, M, Hq, Hkv, img,
                     sc);
  if (Hq == 2 * Hkv && p.n_split == 0) {
    const dim3 grid(static_cast<unsigned>(p.units * Hkv));
    hipLaunchKernelGGL((attn_fwd_kernel<D, kBias, 2>), grid, dim3(2 * kThreads), 0, stream,
                       reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k), img, sc,
                       M, Hq, Hkv, g, t, reinterpret_cast<bf16*>(out), lse, out32, p.h,
                       static_cast<int>(p.units), part);
  } else {
    const dim3 grid(static_cast<unsigned>(p.units * Hq));
    hipLaunchKernelGGL((attn_fwd_kernel<D, kBias, 1>), grid, dim3(kThreads), 0, stream,
                       reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k), img, sc,
                       M, Hq, Hkv, g, t, reinterpret_cast<bf16*>(out), lse, out32, p.h,
                       static_cast<int>(p.units), part);
  }
  if (p.n_split > 0)
    hipLaunchKernelGGL((attn_merge_kernel<D>),
                       dim3(static_cast<unsigned>(Hq * p.n_split * (kThreads / 64))), dim3(64), 0,
                       stream, part, M, Hq, p.h, static_cast<int>(p.units),
                       static_cast<int>(p.n_split), reinterpret_cast<bf16*>(out), lse, out32);
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
  const int64_t img = head_dim == 128 ? Tile<128, true>::V_IMG : Tile<64, true>::V_IMG;
  (void)gated;
  return static_cast<size_t>(n_tiles * img);
}

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                           int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                           const float* gain, const float* tau, uint16_t* out, float* lse,
                           float* out32, void* workspace, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int M = static_cast<int>(n);
  const bool bias = gain != nullptr;
  if (head_dim == 128)
    return bias ? launch<128, true>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out,
                                    lse, out32, workspace, stream)
                : launch<128, false>(q, k, v, M, n_q_heads, n_kv_heads, nullptr, nullptr,
                                     nullptr, out, lse, out32, workspace, stream);
  return bias ? launch<64, true>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out,
                                 lse, out32, workspace, stream)
              : launch<64, false>(q, k, v, M, n_q_heads, n_kv_heads, nullptr, nullptr, nullptr,
                                  out, lse, out32, workspace, stream);
}

}  // namespace tg
