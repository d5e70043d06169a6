// Query/key prologue of the layers above the gate at the kept tokens' own
// positions, for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"): only the
// kept tokens go up; they stay the tokens they were, so their rotary
// positions are their original indices.  The prologue is Qwen3's (model
// plumbing, not the method): a per-head RMS normalisation of q and k, then
// rotate-half rotary position embedding:
//     y = x / sqrt(mean(x^2) + eps) * w
//     out[f] = y[f] cos a_f - y[f + d/2] sin a_f,  out[f + d/2] = y[f + d/2] cos a_f + y[f] sin a_f
// with a_f = position * theta^(-2f/d).  Fused with the row gather, so a
// caller holding full-N rows gets the kept rows ready for attention in one
// pass over their bytes.
//
// Design: one work-group per output row (HBM-bound: each source byte read
// once, each output byte written once).  The row's d/2 angles are formed in
// fp64 (a position times a frequency reaches ~1.3e5 rad at 128k tokens, where
// an fp32 product is off by ~1e-2 rad) and their cos / sin kept in LDS for all
// heads of the row.  A head vector is d/8 lanes, each holding 4 dims of each
// half (8-byte loads and stores), so its rotation partner is in the same
// lane; the RMS is a reduction over those lanes.  fp32 arithmetic, bf16 out.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kRThreads = 256;

template <int D>
__global__ __launch_bounds__(kRThreads) void qk_norm_rope_kernel(
    const bf16* __restrict__ src, int64_t src_rows, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ pos, int H, const float* __restrict__ w, float eps,
    double log2_theta, bf16* __restrict__ dst) {
  constexpr int HALF = D / 2;
  constexpr int LPV = D / 8;                    // lanes per head vector
  constexpr int VPG = kRThreads / LPV;          // head vectors per pass
  __shared__ float cs[HALF], sn[HALF];
  const int64_t i = blockIdx.x;
  const int64_t r = rows != nullptr ? static_cast<int64_t>(rows[i]) : i;
  if (r < 0 || r >= src_rows) return;           // skipped row: left unwritten (uniform)
  const double p = static_cast<double>(pos[i]);
  for (int f = threadIdx.x; f < HALF; f += kRThreads) {
    const double a = p * exp2(-(2.0 * f / D) * log2_theta);
    double s, c;
    sincos(a, &s, &c);
    cs[f] = static_cast<float>(c);
    sn[f] = static_cast<float>(s);
  }
  __syncthreads();
  const int lq = threadIdx.x % LPV;
  float wl[4], wh[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wl[e] = w != nullptr ? w[4 * lq + e] : 1.f;
    wh[e] = w != nullptr ? w[HALF + 4 * lq + e] : 1.f;
  }
  for (int h0 = 0; h0 < H; h0 += VPG) {
    const int h = h0 + static_cast<int>(threadIdx.x) / LPV;
    if (h >= H) continue;                       // whole LPV groups drop out together
    const bf16* x = src + (r * H + h) * D;
    const uint2 ul = *reinterpret_cast<const uint2*>(x + 4 * lq);
    const uint2 uh = *reinterpret_cast<const uint2*>(x + HALF + 4 * lq);
    float xl[4], xh[4];
    xl[0] = __uint_as_float(ul.x << 16); xl[1] = __uint_as_float(ul.x & 0xFFFF0000u);
    xl[2] = __uint_as_float(ul.y << 16); xl[3] = __uint_as_float(ul.y & 0xFFFF0000u);
    xh[0] = __uint_as_float(uh.x << 16); xh[1] = __uint_as_float(uh.x & 0xFFFF0000u);
    xh[2] = __uint_as_float(uh.y << 16); xh[3] = __uint_as_float(uh.y & 0xFFFF0000u);
    float scale = 1.f;
    if (w != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(xl[e], xl[e], fmaf(xh[e], xh[e], ss));
#pragma unroll
      for (int o = 1; o < LPV; o <<= 1) ss += __shfl_xor(ss, o);
      scale = rsqrtf(ss / D + eps);
    }
    bf16 ol[4], oh[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float yl = xl[e] * scale * wl[e], yh = xh[e] * scale * wh[e];
      const float c = cs[4 * lq + e], s = sn[4 * lq + e];
      ol[e] = static_cast<bf16>(yl * c - yh * s);
      oh[e] = static_cast<bf16>(yh * c + yl * s);
    }
    bf16* y = dst + (i * H + h) * D;
    *reinterpret_cast<uint2*>(y + 4 * lq) = __builtin_bit_cast(uint2, ol);
    *reinterpret_cast<uint2*>(y + HALF + 4 * lq) = __builtin_bit_cast(uint2, oh);
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(const uint16_t* src, int64_t src_rows, const int32_t* rows,
                               const int32_t* pos, int64_t n, int n_heads, int head_dim,
                               const float* norm_weight, float eps, double theta, uint16_t* dst,
                               hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const bf16* s = reinterpret_cast<const bf16*>(src);
  bf16* d = reinterpret_cast<bf16*>(dst);
  const double lt = log2(theta);
  if (head_dim == 128)
    hipLaunchKernelGGL((qk_norm_rope_kernel<128>), dim3(static_cast<unsigned>(n)), dim3(kRThreads),
                       0, stream, s, src_rows, rows, pos, n_heads, norm_weight, eps, lt, d);
  else
    hipLaunchKernelGGL((qk_norm_rope_kernel<64>), dim3(static_cast<unsigned>(n)), dim3(kRThreads),
                       0, stream, s, src_rows, rows, pos, n_heads, norm_weight, eps, lt, d);
  return hipGetLastError();
}

}  // namespace tg
