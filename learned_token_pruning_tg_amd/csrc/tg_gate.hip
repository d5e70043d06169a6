// Gate MLP scoring for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"): at the gate
// layer a small MLP scores every token from its post-attention residual.
// Read here as s_i = w2 . GELU(W1 h_i + b1) + b2 with the exact erf GELU.
//
// Design: the first layer is a dense contraction [n x H] . [H x Hg], run on
// bf16 MFMA as Z^T = W1 . h^T so that each lane owns one token column and 16
// gate units per 32x32 tile: GELU, the w2 weighting and the reduction over
// gate units then stay lane-local, plus one exchange between lane halves and
// a fixed-order sum over the four column waves in LDS (deterministic, no
// atomics, no workspace).  One work-group takes BM tokens and all Hg <= 512
// gate units, so h is read from HBM exactly once and W1 (2 MiB at Qwen3
// shapes, L2-resident) is re-read once per BM tokens.  K is streamed in
// 32-wide chunks through padded LDS tiles with the next chunk held in
// registers while the current one is consumed.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kKC = 32;          // K chunk
constexpr int kLD = kKC + 8;     // padded LDS row (80 B): conflict-free 16-byte reads
constexpr int kMaxHg = 512;

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
}

// BM tokens per work-group; BM / 64 row groups x 4 column waves.
template <int BM>
__global__ __launch_bounds__(BM / 64 * 256) void gate_score_kernel(
    const bf16* __restrict__ h, int64_t n, int64_t ld_h, int H, const bf16* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2, int Hg,
    float* __restrict__ scores) {
  constexpr int NT = BM / 64 * 256;
  constexpr int W_TASKS = kMaxHg * (kKC / 8);       // 16-byte chunks of a W1 K-chunk
  constexpr int W_PER_T = W_TASKS / NT;
  constexpr int H_TASKS = BM * (kKC / 8);
  constexpr int H_PER_T = (H_TASKS + NT - 1) / NT;
  static_assert(W_TASKS % NT == 0, "W1 chunk split");

  __shared__ __align__(16) bf16 w_lds[kMaxHg * kLD];
  __shared__ __align__(16) bf16 h_lds[BM * kLD];
  __shared__ float red[4][BM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int rw = wave >> 2;   // 64-token group
  const int cw = wave & 3;    // column wave: gate-unit tiles cw, cw+4, cw+8, cw+12
  const int n_ct = Hg / 32;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * BM;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[i][0] = zero16();
    acc[i][1] = zero16();
  }

  u32x4 wreg[W_PER_T];
  u32x4 hreg[H_PER_T];
  const int w_tasks = Hg * (kKC / 8);

  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int p = 0; p < W_PER_T; ++p) {
      const int f = tid + p * NT;
      const int r = f >> 2, c = f & 3;
      wreg[p] = f < w_tasks ? ld16(w1 + static_cast<size_t>(r) * H + k0 + 8 * c) : zero_u32x4();
    }
#pragma unroll
    for (int p = 0; p < H_PER_T; ++p) {
      const int f = tid + p * NT;
      const int r = f >> 2, c = f & 3;
      const int64_t row = row0 + r;
      hreg[p] = (f < H_TASKS && row < n) ? ld16(h + row * ld_h + k0 + 8 * c) : zero_u32x4();
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int p = 0; p < W_PER_T; ++p) {
      const int f = tid + p * NT;
      if (f < w_tasks) st16(&w_lds[(f >> 2) * kLD + 8 * (f & 3)], wreg[p]);
    }
#pragma unroll
    for (int p = 0; p < H_PER_T; ++p) {
      const int f = tid + p * NT;
      if (f < H_TASKS) st16(&h_lds[(f >> 2) * kLD + 8 * (f & 3)], hreg[p]);
    }
  };

  load_chunk(0);
  for (int k0 = 0; k0 < H; k0 += kKC) {
    store_chunk();
    __syncthreads();
    if (k0 + kKC < H) load_chunk(k0 + kKC);
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      bf16x8 hb[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        hb[tt] = lds_bf16x8(&h_lds[(64 * rw + 32 * tt + l32) * kLD + 16 * ks + 8 * hh]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ct = cw + 4 * i;
        if (ct < n_ct) {
          const bf16x8 a = lds_bf16x8(&w_lds[(32 * ct + l32) * kLD + 16 * ks + 8 * hh]);
          acc[i][0] = mfma_32x32x16(a, hb[0], acc[i][0]);
          acc[i][1] = mfma_32x32x16(a, hb[1], acc[i][1]);
        }
      }
    }
    __syncthreads();
  }

  // Epilogue: GELU, weight by w2, reduce over gate units.
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ct = cw + 4 * i;
      if (ct < n_ct) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int u = 32 * ct + 8 * (j >> 2) + 4 * hh + (j & 3);
          part = fmaf(w2[u], gelu_erf(acc[i][tt][j] + b1[u]), part);
        }
      }
    }
    part += __shfl_xor(part, 32);
    if (hh == 0) red[cw][64 * rw + 32 * tt + l32] = part;
  }
  __syncthreads();
  for (int r = tid; r < BM; r += NT) {
    const int64_t row = row0 + r;
    if (row < n) scores[row] = (((red[0][r] + red[1][r]) + red[2][r]) + red[3][r]) + b2;
  }
}

}  // namespace

hipError_t launch_gate_score(const uint16_t* h, int64_t n, int64_t ld_h, int hidden,
                             const uint16_t* w1, const float* b1, const float* w2, float b2,
                             int gate_hidden, float* scores, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const bf16* hp = reinterpret_cast<const bf16*>(h);
  const bf16* wp = reinterpret_cast<const bf16*>(w1);
  // Prefer 128-token tiles (half the W1 re-reads) once they still give at
  // least two work-groups per compute unit.
  if (n >= 128 * 512) {
    const dim3 grid(static_cast<unsigned>((n + 127) / 128));
    hipLaunchKernelGGL(gate_score_kernel<128>, grid, dim3(512), 0, stream, hp, n, ld_h, hidden,
                       wp, b1, w2, b2, gate_hidden, scores);
  } else {
    const dim3 grid(static_cast<unsigned>((n + 63) / 64));
    hipLaunchKernelGGL(gate_score_kernel<64>, grid, dim3(256), 0, stream, hp, n, ld_h, hidden,
                       wp, b1, w2, b2, gate_hidden, scores);
  }
  return hipGetLastError();
}

}  // namespace tg
