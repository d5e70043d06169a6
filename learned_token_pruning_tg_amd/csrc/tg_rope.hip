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
// Design: four output rows per work-group (fewer when a row has many heads),
// all of a lane's loads issued first (HBM-bound: each source byte read once,
// each output byte written once).  The row's d/2 angles are formed in
// fp64 (a position times a frequency reaches ~1.3e5 rad at 128k tokens, where
// an fp32 product is off by ~1e-2 rad) and their cos / sin kept in LDS for all
// heads of the row.  A head vector is d/8 lanes, each holding 4 dims of each
// half (8-byte loads and stores), so its rotation partner is in the same
// lane; the RMS is a reduction over those lanes.  fp32 arithmetic, bf16 out.
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kRThreads = 256;

// R rows per work-group, each row on kRThreads / R threads; every lane loads
// its pieces of up to NP head vectors before anything else (more heads than
// that: the rest go one pass at a time).  Work-group count, not bytes, bounds
// a one-row-per-work-group launch at these sizes, hence several rows each.
template <int D, int R, int NP>
__global__ __launch_bounds__(kRThreads) void qk_norm_rope_kernel(
    const bf16* __restrict__ src, int64_t src_rows, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ pos, int64_t n, int H, const float* __restrict__ w, float eps,
    double log2_theta, bf16* __restrict__ dst) {
  constexpr int HALF = D / 2;
  constexpr int LPV = D / 8;                    // lanes per head vector
  constexpr int TPR = kRThreads / R;            // threads per row
  constexpr int VPG = TPR / LPV;                // head vectors per pass of a row
  __shared__ float cs[R][HALF], sn[R][HALF];
  const int rr = static_cast<int>(threadIdx.x) / TPR;    // this thread's row slot
  const int tr = static_cast<int>(threadIdx.x) % TPR;    // its thread index within the row
  const int64_t i = static_cast<int64_t>(blockIdx.x) * R + rr;
  int64_t r = -1;
  if (i < n) r = rows != nullptr ? static_cast<int64_t>(rows[i]) : i;
  const bool live = r >= 0 && r < src_rows;     // else: row skipped, left unwritten
  const int lq = tr % LPV;
  // This lane's pieces of a head vector: 4 dims of each half (8-byte loads).
  auto load = [&](int h, float (&xl)[4], float (&xh)[4]) {
    const bf16* x = src + (r * H + h) * D;
    const uint2 ul = *reinterpret_cast<const uint2*>(x + 4 * lq);
    const uint2 uh = *reinterpret_cast<const uint2*>(x + HALF + 4 * lq);
    xl[0] = __uint_as_float(ul.x << 16); xl[1] = __uint_as_float(ul.x & 0xFFFF0000u);
    xl[2] = __uint_as_float(ul.y << 16); xl[3] = __uint_as_float(ul.y & 0xFFFF0000u);
    xh[0] = __uint_as_float(uh.x << 16); xh[1] = __uint_as_float(uh.x & 0xFFFF0000u);
    xh[2] = __uint_as_float(uh.y << 16); xh[3] = __uint_as_float(uh.y & 0xFFFF0000u);
  };
  // The first NP head passes' loads go out before the angles are formed.
  const int hv = tr / LPV;
  float xl[NP][4], xh[NP][4];
#pragma unroll
  for (int q = 0; q < NP; ++q)
    if (live && hv + q * VPG < H) load(hv + q * VPG, xl[q], xh[q]);
  if (live) {
    const double p = static_cast<double>(pos[i]);
    for (int f = tr; f < HALF; f += TPR) {
      const double a = p * exp2(-(2.0 * f / D) * log2_theta);
      double s, c;
      sincos(a, &s, &c);
      cs[rr][f] = static_cast<float>(c);
      sn[rr][f] = static_cast<float>(s);
    }
  }
  __syncthreads();
  if (!live) return;
  float wl[4], wh[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wl[e] = w != nullptr ? w[4 * lq + e] : 1.f;
    wh[e] = w != nullptr ? w[HALF + 4 * lq + e] : 1.f;
  }
  // One head vector: RMS over its LPV lanes (whole lane groups drop out of a
  // pass together), rotation, bf16 store.
  auto emit = [&](int h, const float (&lo)[4], const float (&hi)[4]) {
    float scale = 1.f;
    if (w != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(lo[e], lo[e], fmaf(hi[e], hi[e], ss));
#pragma unroll
      for (int o = 1; o < LPV; o <<= 1) ss += __shfl_xor(ss, o);
      scale = rsqrtf(ss / D + eps);
    }
    bf16 ol[4], oh[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float yl = lo[e] * scale * wl[e], yh = hi[e] * scale * wh[e];
      const float c = cs[rr][4 * lq + e], s = sn[rr][4 * lq + e];
      ol[e] = static_cast<bf16>(yl * c - yh * s);
      oh[e] = static_cast<bf16>(yh * c + yl * s);
    }
    bf16* y = dst + (i * H + h) * D;
    *reinterpret_cast<uint2*>(y + 4 * lq) = __builtin_bit_cast(uint2, ol);
    *reinterpret_cast<uint2*>(y + HALF + 4 * lq) = __builtin_bit_cast(uint2, oh);
  };
#pragma unroll
  for (int q = 0; q < NP; ++q)
    if (hv + q * VPG < H) emit(hv + q * VPG, xl[q], xh[q]);
  for (int h = hv + NP * VPG; h < H; h += VPG) {
    float yl[4], yh[4];
    load(h, yl, yh);
    emit(h, yl, yh);
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
  // Rows per work-group: 4, unless a row's head vectors then take more than 4
  // passes of its lanes (2, then 1).  Preloaded passes: those passes, up to 4.
  const int vecs = kRThreads / (head_dim / 8);   // head vectors one work-group holds
  int r = 4;
  while (r > 1 && n_heads * r > 4 * vecs) r /= 2;
  const int passes = (n_heads * r + vecs - 1) / vecs;
  const int np = passes <= 1 ? 1 : passes <= 2 ? 2 : 4;
  auto go = [&](auto d_c, auto r_c, auto np_c) {
    constexpr int D = decltype(d_c)::value, R = decltype(r_c)::value;
    constexpr int NP = decltype(np_c)::value;
    hipLaunchKernelGGL((qk_norm_rope_kernel<D, R, NP>),
                       dim3(static_cast<unsigned>((n + R - 1) / R)), dim3(kRThreads), 0, stream,
                       s, src_rows, rows, pos, n, n_heads, norm_weight, eps, lt, d);
  };
  auto by_np = [&](auto d_c, auto r_c) {
    if (np == 1) go(d_c, r_c, std::integral_constant<int, 1>{});
    else if (np == 2) go(d_c, r_c, std::integral_constant<int, 2>{});
    else go(d_c, r_c, std::integral_constant<int, 4>{});
  };
  auto by_r = [&](auto d_c) {
    if (r == 4) by_np(d_c, std::integral_constant<int, 4>{});
    else if (r == 2) by_np(d_c, std::integral_constant<int, 2>{});
    else by_np(d_c, std::integral_constant<int, 1>{});
  };
  if (head_dim == 128) by_r(std::integral_constant<int, 128>{});
  else by_r(std::integral_constant<int, 64>{});
  return hipGetLastError();
}

}  // namespace tg
