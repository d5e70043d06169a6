// Gate MLP scoring for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"): at the gate
// layer a small MLP scores every token from its post-attention residual.
// Read here as s_i = w2 . GELU(W1 h_i + b1) + b2 with the exact (erf) GELU.
//
// Design: the first layer is a dense contraction [n x H] . [H x Hg] on bf16
// MFMA, computed as Z^T = W1 . h^T so that each lane owns one token column and
// 16 gate units per 32x32 tile: GELU, the w2 weighting and the reduction over
// gate units stay lane-local, plus one exchange between lane halves and a
// fixed-order sum over the column waves in LDS (deterministic, no atomics, no
// workspace).
//  * One work-group takes BM tokens and all gate units (padded to 128 * CT;
//    padding units read as zeros and contribute nothing), so h streams from
//    HBM exactly once while W1 (2 MiB at Qwen3 shapes) is re-read from L2
//    once per BM tokens.
//  * Eight column waves per 64 tokens (two per SIMD) where the gate units
//    split evenly over them, else four.
//  * K is streamed in 64-wide (64-token work-groups) or 32-wide chunks
//    through double-buffered LDS tiles with one barrier per chunk; raw buffer loads run two chunks ahead of the
//    MFMAs (two register stage sets).  Scheduling barriers keep every chunk's
//    loads issued in chunk order, so the wait before storing chunk c counts
//    only chunk c's loads and chunk c + 1's stay in flight.  Per-chunk
//    descriptors put the hardware range check on the row boundary, so rows
//    past n read as zeros without per-row guards.
//  * Work-groups start their K loop at staggered chunks so the CUs of one XCD
//    do not all hit the same W1 lines of L2 at the same time.
//  * erf uses Abramowitz & Stegun formula 7.1.26 (|error| <= 1.5e-7),
//    branch-free, with the hardware exp2.
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {


// erf(x) by Abramowitz & Stegun 7.1.26: for x >= 0,
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x);  odd symmetry for x < 0.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-ax * ax * kLog2e);
  const float r = fmaf(-poly, e, 1.f);
  return copysignf(r, x);
}

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.f + erf_as(z * 0.70710678118654752f));
}

// BM tokens per work-group (BM / 64 row groups x CW column waves); the
// work-group covers 128 * CT gate units, each wave UT = 4 CT / CW tiles of 32.
// KC: K chunk (32 or 64).  LDS rows are unpadded and XOR-swizzled: rows of a
// 32-wide chunk are 64 B with 16-byte piece j of row r at slot j ^ ((r / 4)
// % 4), rows of a 64-wide chunk 128 B with piece j at slot j ^ ((r / 2) % 8).
// Either way the 16 lanes that one pass of a 16-byte LDS read serves (one
// piece of 16 consecutive rows; 64 banks of 4 bytes) hit 16 different bank
// groups, and so do those of a staging write (all pieces of 4 or 2
// consecutive rows: 256 contiguous bytes).
template <int BM, int CT, int CW, int KC>
__global__ __launch_bounds__(BM / 64 * CW * 64) void gate_score_kernel(
    const bf16* __restrict__ h, int64_t n, int64_t ld_h, int H, const bf16* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2, int Hg,
    float* __restrict__ scores) {
  constexpr int NT = BM / 64 * CW * 64;
  constexpr int HGP = 128 * CT;                 // padded gate units
  constexpr int UT = 4 * CT / CW;               // 32-unit tiles per wave
  static_assert(KC == 32 || KC == 64, "K chunk");
  constexpr int P = KC / 8;                     // 16-byte pieces per row of a chunk
  constexpr int LD = KC;                        // LDS row, bf16 elements
  constexpr int W_PIECES = HGP * P;             // 16-byte pieces of a W1 chunk
  constexpr int H_PIECES = BM * P;              // ... of an h chunk
  constexpr int W_PER_T = (W_PIECES + NT - 1) / NT;
  constexpr int H_PER_T = (H_PIECES + NT - 1) / NT;
  static_assert(4 * CT % CW == 0, "unit tiles split over the column waves");

  __shared__ __align__(16) bf16 w_lds[2][HGP * LD];
  __shared__ __align__(16) bf16 h_lds[2][BM * LD];
  auto lds_at = [](int row, int piece) {
    return row * LD + 8 * (KC == 64 ? piece ^ ((row >> 1) & 7) : piece ^ ((row >> 2) & 3));
  };
  __shared__ float red[CW][BM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int rw = wave / CW;   // 64-token group
  const int cw = wave % CW;   // column wave: gate-unit tiles cw + CW i
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t rows_left = n - row0;
  const uint32_t rows_valid = static_cast<uint32_t>(rows_left < BM ? rows_left : BM);
  const uint32_t h_row_bytes = static_cast<uint32_t>(ld_h) * 2;
  const uint32_t h_bytes = rows_valid * h_row_bytes;
  const uint32_t w_row_bytes = static_cast<uint32_t>(H) * 2;
  const uint32_t w_bytes = static_cast<uint32_t>(Hg) * w_row_bytes;
  const char* h_base = reinterpret_cast<const char*>(h + row0 * ld_h);
  const char* w_base = reinterpret_cast<const char*>(w1);

  uint32_t w_off[W_PER_T], h_off[H_PER_T];
#pragma unroll
  for (int p = 0; p < W_PER_T; ++p) {
    const int f = tid + p * NT;
    // threads without a piece read past every range (zeros, no memory access)
    w_off[p] = f < W_PIECES ? static_cast<uint32_t>(f / P) * w_row_bytes + 16 * (f % P)
                            : 0x80000000u;
  }
#pragma unroll
  for (int p = 0; p < H_PER_T; ++p) {
    const int f = tid + p * NT;
    // threads without a piece read past every range (zeros, no memory access)
    h_off[p] = f < H_PIECES ? static_cast<uint32_t>(f / P) * h_row_bytes + 16 * (f % P)
                            : 0x80000000u;
  }

  floatx16 acc[UT][2];
#pragma unroll
  for (int i = 0; i < UT; ++i) {
    acc[i][0] = zero16();
    acc[i][1] = zero16();
  }

  // NS register stage sets: chunk c is loaded at stage c - NS into set
  // c % NS, so each load has NS chunks of work to arrive (four sets measured
  // no faster).
  constexpr int NS = 2;
  u32x4 wreg[NS][W_PER_T];
  u32x4 hreg[NS][H_PER_T];
  const int n_chunks = H / KC;
  const int start = static_cast<int>(blockIdx.x >> 3) % n_chunks;

  auto load_chunk = [&](int set, int c) __attribute__((always_inline)) {
    const int k0 = ((start + c) % n_chunks) * KC;
    const uint32_t kb = static_cast<uint32_t>(k0) * 2;
    // Past the last chunk the loads still issue, against empty ranges (they
    // return zeros and touch no memory): every stage then issues the same
    // loads, and the compiler waits for exactly the set a stage stores while
    // the other set stays in flight.
    const bool live = c < n_chunks;
    const __amdgpu_buffer_rsrc_t rw_ =
        make_rsrc(w_base + kb, live && w_bytes > kb ? w_bytes - kb : 0u);
    const __amdgpu_buffer_rsrc_t rh_ =
        make_rsrc(h_base + kb, live && h_bytes > kb ? h_bytes - kb : 0u);
#pragma unroll
    for (int p = 0; p < W_PER_T; ++p) wreg[set][p] = bload16(rw_, w_off[p]);
#pragma unroll
    for (int p = 0; p < H_PER_T; ++p) hreg[set][p] = bload16(rh_, h_off[p]);
  };
  auto store_chunk = [&](int set, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < W_PER_T; ++p) {
      const int f = tid + p * NT;
      if (W_PIECES % NT == 0 || f < W_PIECES)
        st16(&w_lds[buf][lds_at(f / P, f % P)], wreg[set][p]);
    }
#pragma unroll
    for (int p = 0; p < H_PER_T; ++p) {
      const int f = tid + p * NT;
      if (H_PIECES % NT == 0 || f < H_PIECES)
        st16(&h_lds[buf][lds_at(f / P, f % P)], hreg[set][p]);
    }
  };
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      bf16x8 hb[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        hb[tt] = lds_bf16x8(&h_lds[buf][lds_at(64 * rw + 32 * tt + l32, 2 * ks + hh)]);
#pragma unroll
      for (int i = 0; i < UT; ++i) {
        const bf16x8 a = lds_bf16x8(&w_lds[buf][lds_at(32 * (cw + CW * i) + l32, 2 * ks + hh)]);
        acc[i][0] = mfma_32x32x16(a, hb[0], acc[i][0]);
        acc[i][1] = mfma_32x32x16(a, hb[1], acc[i][1]);
      }
    }
  };
  // One barrier per chunk: the LDS buffer written at chunk c was last read at
  // chunk c - 2, which every wave finished before passing barrier c - 1.
  auto stage = [&](auto set_c, int c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    constexpr int buf = set & 1;          // = c & 1 (NS is even)
    store_chunk(set, buf);
    __syncthreads();
    load_chunk(set, c + NS);
    __builtin_amdgcn_sched_barrier(0);   // issue the loads before this chunk's MFMAs
    compute(buf);
  };

  // Every trip runs all NS stages (keeping the accumulators in place across
  // the back-edge); stages past the last chunk load and add zeros.
  load_chunk(0, 0);
#pragma unroll
  for (int c = 1; c < NS; ++c) {
    __builtin_amdgcn_sched_barrier(0);   // keep chunk c - 1's loads older than chunk c's
    load_chunk(c, c);
  }
  for (int c = 0; c < n_chunks; c += NS) {
    stage(std::integral_constant<int, 0>{}, c);
    stage(std::integral_constant<int, 1>{}, c + 1);
  }

  // Epilogue: GELU, weight by w2, reduce over gate units (padding units have
  // b1 = w2 = 0 through the range-checked loads).
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(b1, 4u * Hg);
  const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(w2, 4u * Hg);
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < UT; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = 32 * (cw + CW * i) + 8 * (j >> 2) + 4 * hh + (j & 3);
      const float bu = bload4f(rb1, 4 * u), wu = bload4f(rw2, 4 * u);
      part[0] = fmaf(wu, gelu_erf(acc[i][0][j] + bu), part[0]);
      part[1] = fmaf(wu, gelu_erf(acc[i][1][j] + bu), part[1]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const float p = part[tt] + __shfl_xor(part[tt], 32);
    if (hh == 0) red[cw][64 * rw + 32 * tt + l32] = p;
  }
  __syncthreads();
  for (int r = tid; r < BM; r += NT) {
    if (r < static_cast<int>(rows_valid)) {
      float acc_r = red[0][r];
#pragma unroll
      for (int c = 1; c < CW; ++c) acc_r += red[c][r];   // fixed order
      scores[row0 + r] = acc_r + b2;
    }
  }
}

template <int BM, int CT, int CW, int KC>
void launch_bm_ct(const bf16* h, int64_t n, int64_t ld_h, int H, const bf16* w1, const float* b1,
                  const float* w2, float b2, int Hg, float* scores, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + BM - 1) / BM));
  hipLaunchKernelGGL((gate_score_kernel<BM, CT, CW, KC>), grid, dim3(BM / 64 * CW * 64), 0, stream,
                     h, n, ld_h, H, w1, b1, w2, b2, Hg, scores);
}

// CW8: eight column waves where the unit tiles split evenly (Hg > 128 and
// not in (256, 384]); else four.
template <int BM, bool CW8, int KC>
void launch_bm(const bf16* h, int64_t n, int64_t ld_h, int H, const bf16* w1, const float* b1,
               const float* w2, float b2, int Hg, float* scores, hipStream_t stream) {
  constexpr int CW = CW8 ? 8 : 4;
  switch ((Hg + 127) / 128) {
    case 1: launch_bm_ct<BM, 1, 4, KC>(h, n, ld_h, H, w1, b1, w2, b2, Hg, scores, stream); break;
    case 2: launch_bm_ct<BM, 2, CW, KC>(h, n, ld_h, H, w1, b1, w2, b2, Hg, scores, stream); break;
    case 3: launch_bm_ct<BM, 3, 4, KC>(h, n, ld_h, H, w1, b1, w2, b2, Hg, scores, stream); break;
    default: launch_bm_ct<BM, 4, CW, KC>(h, n, ld_h, H, w1, b1, w2, b2, Hg, scores, stream); break;
  }
}

}  // namespace

hipError_t launch_gate_score(const uint16_t* h, int64_t n, int64_t ld_h, int hidden,
                             const uint16_t* w1, const float* b1, const float* w2, float b2,
                             int gate_hidden, float* scores, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const bf16* hp = reinterpret_cast<const bf16*>(h);
  const bf16* wp = reinterpret_cast<const bf16*>(w1);
  // 128-token tiles halve the W1 re-reads; use them once they still give at
  // least two work-groups per compute unit.  64-wide K chunks (half the
  // barriers) fit LDS only with 64-token tiles.
  if (n >= 128 * 512)
    launch_bm<128, true, 32>(hp, n, ld_h, hidden, wp, b1, w2, b2, gate_hidden, scores, stream);
  else
    launch_bm<64, true, 64>(hp, n, ld_h, hidden, wp, b1, w2, b2, gate_hidden, scores, stream);
  return hipGetLastError();
}

}  // namespace tg
