// One decode step of token-gated GQA attention over the pruned KV cache, for
// gfx950.
//
// Method (lucasainews.com TokenGate article, lede: the speed-up is measured as
// time to first token; section "작동 방식": above the gate layer only the kept
// tokens have KV entries, and each kept key's score enters the logits there
// as a bias with a per-head gain and temperature).  Read here as one new
// query row per head against every cached row (the kept rows plus the new
// token's own row, appended by the caller):
//     logit_j = q.k_j / (sqrt(d) * tau_h) + gain_h * s_j,   out = softmax(logit) . V
// With no bias arguments the same kernels give plain attention (the gate
// layer's decode over all N rows).
//
// Design: a single query row makes this a pass over the K and V cache bytes
// (HBM-bound; a 16-row MFMA tile would be 1/8 used).  Split-KV: a work-group
// takes a chunk of C keys (C in {64, 128, 256}, see decode_plan) of one KV
// head for all G = Hq / Hkv query heads that share it, so each cache byte is
// read once, and requests all of the chunk's K and V bytes before it
// computes anything.  Eight lanes share a key row (16
// bytes each per 128 bytes of row: every wave-wide load covers whole 128-byte
// lines); fp32 dot products reduced across the eight lanes; the chunk's
// softmax in log2 units with block reductions; P.V again eight lanes per row,
// reduced across rows by lane exchanges and a fixed-order sum over the four
// waves.  Each chunk leaves (max, sum, unnormalised output) per head in the
// workspace; a combine launch merges the chunks in a fixed order
// (deterministic) and writes the bf16 output and the log-sum-exp.
// Everything after the bf16 inputs is fp32.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kDThreads = 256;
constexpr int kDWaves = kDThreads / 64;
constexpr int kParts = 8;                          // lanes per key row
constexpr int kRowsPerPass = kDThreads / kParts;   // 32 key rows per pass

struct DecodePlan {
  int chunk, n_chunks;
  size_t bytes;
};

// Chunk length, capped so that the chunk's K and V pieces and the group's
// query and accumulator registers fit (256 for groups of up to 2 query heads,
// 128 for 4, 64 for 8): 256 when that gives >= 512 work-groups, else 128 when
// that gives >= 128, else 64.  Measured at 16/8 heads: 1000 rows 9.1 us with
// 64 (128: 10.1), 2304 rows 10.0 us with 128 (64: 11.2), 4352 rows 12.1 us
// with 128 (64: 14.3), 8448 rows 15.3 us with 128 (256: 18.1); fewer, longer
// chunks also shorten the combine.
DecodePlan decode_plan(int64_t n, int Hq, int Hkv, int d) {
  DecodePlan p{};
  const int g = Hq / Hkv;
  int c = g <= 2 ? 256 : g == 4 ? 128 : 64;
  while (c > 64 && ((n + c - 1) / c) * Hkv < (c == 256 ? 512 : 128)) c >>= 1;
  p.chunk = c;
  p.n_chunks = static_cast<int>((n + c - 1) / c);
  // per (KV head, chunk, query head of the group): max, sum, d outputs
  p.bytes = static_cast<size_t>(Hkv) * p.n_chunks * (Hq / Hkv) * (d + 2) * 4;
  return p;
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Block-wide max / sum of one float per thread (fixed reduction order).
template <bool kMax>
__device__ __forceinline__ float block_reduce(float x, float* tmp) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = kMax ? fmaxf(x, y) : x + y;
  }
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = tmp[0];
#pragma unroll
  for (int w = 1; w < kDWaves; ++w) r = kMax ? fmaxf(r, tmp[w]) : r + tmp[w];
  __syncthreads();   // tmp is reused
  return r;
}

// One chunk of C keys of KV head blockIdx.y for its G query heads.
// part layout: [Hkv][n_chunks][G] x (max in log2 units, sum, out[D]).
template <int D, int G, int C, bool kBias>
__global__ __launch_bounds__(kDThreads) void decode_chunk_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, int n,
    int Hq, int Hkv, const float* __restrict__ key_score, const float* __restrict__ gain,
    const float* __restrict__ tau, float* __restrict__ part) {
  constexpr int NL = D / 64;        // 16-byte pieces per lane per key row
  constexpr int DPT = 8 * NL;       // dims per lane: [64 i + 8 r, +8) for i < NL
  constexpr int NP = C / kRowsPerPass;   // rows per lane
  __shared__ float logit[G][C];
  __shared__ float osum[kDWaves][G][D];
  __shared__ float tmp[kDWaves];

  const int chunk = blockIdx.x, kvh = blockIdx.y;
  const int n_chunks = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid % kParts, slot = tid / kParts;
  const int j0 = chunk * C;
  const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
  const uint32_t cache_bytes = row_bytes * static_cast<uint32_t>(n);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + static_cast<size_t>(kvh) * D, cache_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + static_cast<size_t>(kvh) * D, cache_bytes);

  // Every K and V piece of this lane's rows is requested before any
  // arithmetic (V does not wait for the softmax): the chunk's whole cache
  // traffic is in flight at once.  Rows past n read as zeros.
  u32x4 kx[NP][NL], vx[NP][NL];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const uint32_t off = static_cast<uint32_t>(j0 + kRowsPerPass * pp + slot) * row_bytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) kx[pp][i] = bload16(rk, off + (64 * i + 8 * r) * 2);
  }
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const uint32_t off = static_cast<uint32_t>(j0 + kRowsPerPass * pp + slot) * row_bytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) vx[pp][i] = bload16(rv, off + (64 * i + 8 * r) * 2);
  }

  // ---- logits of the chunk, log2 units: (q.k) * alpha_h + beta_h * s_j
  {
    float qv[G][DPT], alpha[G], beta[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int h = kvh * G + g;
      const float t_h = kBias ? tau[h] : 1.f;
      alpha[g] = kLog2e / (sqrtf(static_cast<float>(D)) * t_h);
      beta[g] = kBias ? kLog2e * gain[h] : 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const u32x4 x = ld16(q + static_cast<size_t>(h) * D + 64 * i + 8 * r);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          qv[g][8 * i + 2 * w] = bf16_lo(x[w]);
          qv[g][8 * i + 2 * w + 1] = bf16_hi(x[w]);
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int p0 = kRowsPerPass * pp;
      const int j = j0 + p0 + slot;
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const u32x4 x = kx[pp][i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float k0 = bf16_lo(x[w]), k1 = bf16_hi(x[w]);
#pragma unroll
          for (int g = 0; g < G; ++g)
            dot[g] = fmaf(qv[g][8 * i + 2 * w + 1], k1, fmaf(qv[g][8 * i + 2 * w], k0, dot[g]));
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        dot[g] += __shfl_xor(dot[g], 1);
        dot[g] += __shfl_xor(dot[g], 2);
        dot[g] += __shfl_xor(dot[g], 4);
      }
      if (r == 0) {
        const float sj = (kBias && j < n) ? key_score[j] : 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
          logit[g][p0 + slot] = j < n ? fmaf(dot[g], alpha[g], beta[g] * sj) : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- per head: chunk max, P = exp2(logit - max), chunk sum (P kept in LDS)
  float* prow = part + (static_cast<size_t>(kvh) * n_chunks + chunk) * G * (D + 2);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float x = tid < C ? logit[g][tid] : -INFINITY;
    const float m = block_reduce<true>(x, tmp);   // finite: key j0 < n is in every chunk
    const float p = tid < C ? fast_exp2(x - m) : 0.f;
    const float l = block_reduce<false>(p, tmp);
    if (tid < C) logit[g][tid] = p;
    if (tid == 0) {
      prow[g * (D + 2)] = m;
      prow[g * (D + 2) + 1] = l;
    }
  }
  __syncthreads();

  // ---- out = P . V over the chunk: lane (slot, r) accumulates its rows' dims
  float acc[G][DPT];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[g][e] = 0.f;
  }
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int p0 = kRowsPerPass * pp;
    float pj[G];
#pragma unroll
    for (int g = 0; g < G; ++g) pj[g] = logit[g][p0 + slot];   // 0 past n
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const u32x4 x = vx[pp][i];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float v0 = bf16_lo(x[w]), v1 = bf16_hi(x[w]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g][8 * i + 2 * w] = fmaf(pj[g], v0, acc[g][8 * i + 2 * w]);
          acc[g][8 * i + 2 * w + 1] = fmaf(pj[g], v1, acc[g][8 * i + 2 * w + 1]);
        }
      }
    }
  }
  // sum over the 8 rows of a wave sharing a dim group (lanes r, r + 8, ...)
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      float a = acc[g][e];
      a += __shfl_xor(a, 8);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[g][e] = a;
    }
  }
  if (lane < kParts) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) osum[wave][g][64 * i + 8 * r + e] = acc[g][8 * i + e];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDThreads) {
    const int g = idx / D, dim = idx % D;
    float o = osum[0][g][dim];
#pragma unroll
    for (int w = 1; w < kDWaves; ++w) o += osum[w][g][dim];
    prow[g * (D + 2) + 2 + dim] = o;
  }
}

// Merge the chunks of one query head in one pass: a work-group of 1024
// threads in NG = 1024 / (D / 4) groups of D / 4 threads; group cg folds the
// chunks cg, cg + NG, ... in that order into a running (max, sum, output)
// (each thread four dims, dim + D/4 i, so every load of a group is one
// contiguous run), then the groups' states are merged in group order
// (deterministic).  One pass over the partials, several chunks' loads in
// flight per thread: the merge is a few load latencies, not one per chunk.
constexpr int kCThreads = 1024;
template <int D>
__global__ __launch_bounds__(kCThreads) void decode_combine_kernel(const float* __restrict__ part,
                                                                  int n_chunks, int G,
                                                                  bf16* __restrict__ out,
                                                                  float* __restrict__ lse) {
  constexpr int TPR = D / 4;             // threads per chunk row
  constexpr int NG = kCThreads / TPR;    // chunk groups
  __shared__ float so[NG][D];
  __shared__ float sm[NG], sl[NG];
  const int h = blockIdx.x, kvh = h / G, g = h % G;
  const int tid = threadIdx.x, t = tid % TPR, cg = tid / TPR;
  const size_t stride = static_cast<size_t>(G) * (D + 2);
  const float* base = part + static_cast<size_t>(kvh) * n_chunks * stride + g * (D + 2);
  float m = -INFINITY, l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int c = cg; c < n_chunks; c += NG) {
    const float* pc = base + c * stride;
    const float mc = pc[0], lc = pc[1];   // mc is finite: every chunk holds a key below n
    float oc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oc[i] = pc[2 + t + TPR * i];
    const float mn = fmaxf(m, mc);
    const float a = fast_exp2(m - mn), b = fast_exp2(mc - mn);   // a = 0 on the first chunk
    l = fmaf(l, a, lc * b);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = fmaf(o[i], a, oc[i] * b);
    m = mn;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) so[cg][t + TPR * i] = o[i];
  if (t == 0) {
    sm[cg] = m;
    sl[cg] = l;
  }
  __syncthreads();
  if (tid < D) {
    float mx = -INFINITY;
    for (int i = 0; i < NG; ++i) mx = fmaxf(mx, sm[i]);
    float lt = 0.f, ot = 0.f;
    for (int i = 0; i < NG; ++i) {
      if (sl[i] > 0.f) {   // groups without chunks (m = -inf) contribute nothing
        const float w = fast_exp2(sm[i] - mx);
        lt = fmaf(sl[i], w, lt);
        ot = fmaf(so[i][tid], w, ot);
      }
    }
    out[static_cast<size_t>(h) * D + tid] = static_cast<bf16>(ot / lt);
    if (lse != nullptr && tid == 0) lse[h] = (mx + __log2f(lt)) * kLn2;
  }
}

template <int D, int G, int C, bool kBias>
void launch_chunks(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n, int Hq,
                   int Hkv, const float* s, const float* gain, const float* tau,
                   const DecodePlan& p, float* part, hipStream_t stream) {
  hipLaunchKernelGGL((decode_chunk_kernel<D, G, C, kBias>),
                     dim3(static_cast<unsigned>(p.n_chunks), static_cast<unsigned>(Hkv)),
                     dim3(kDThreads), 0, stream, reinterpret_cast<const bf16*>(q),
                     reinterpret_cast<const bf16*>(k), reinterpret_cast<const bf16*>(v), n, Hq,
                     Hkv, s, gain, tau, part);
}

template <int D, int G, bool kBias>
void launch_dg(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n, int Hq, int Hkv,
               const float* s, const float* gain, const float* tau, uint16_t* out, float* lse,
               const DecodePlan& p, float* part, hipStream_t stream) {
  if (p.chunk == 64)
    launch_chunks<D, G, 64, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, p, part, stream);
  else if constexpr (G <= 4) {
    if (p.chunk == 128)
      launch_chunks<D, G, 128, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, p, part, stream);
    else if constexpr (G <= 2)
      launch_chunks<D, G, 256, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, p, part, stream);
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(static_cast<unsigned>(Hq)), dim3(kCThreads),
                     0, stream, part, p.n_chunks, G, reinterpret_cast<bf16*>(out), lse);
}

template <int D, bool kBias>
void launch_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, int n, int Hq, int Hkv,
              const float* s, const float* gain, const float* tau, uint16_t* out, float* lse,
              const DecodePlan& p, float* part, hipStream_t stream) {
  switch (Hq / Hkv) {
    case 1: launch_dg<D, 1, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, out, lse, p, part, stream); break;
    case 2: launch_dg<D, 2, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, out, lse, p, part, stream); break;
    case 4: launch_dg<D, 4, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, out, lse, p, part, stream); break;
    default: launch_dg<D, 8, kBias>(q, k, v, n, Hq, Hkv, s, gain, tau, out, lse, p, part, stream); break;
  }
}

}  // namespace

size_t decode_workspace_bytes(int64_t n, int n_q_heads, int n_kv_heads, int head_dim) {
  if (n <= 0) return 0;
  return decode_plan(n, n_q_heads, n_kv_heads, head_dim).bytes;
}

hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                         int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                         const float* gain, const float* tau, uint16_t* out, float* lse,
                         void* workspace, hipStream_t stream) {
  const DecodePlan p = decode_plan(n, n_q_heads, n_kv_heads, head_dim);
  float* part = static_cast<float*>(workspace);
  const int ni = static_cast<int>(n);
  const bool bias = gain != nullptr;
  if (head_dim == 128) {
    if (bias) launch_d<128, true>(q, k, v, ni, n_q_heads, n_kv_heads, key_score, gain, tau, out, lse, p, part, stream);
    else launch_d<128, false>(q, k, v, ni, n_q_heads, n_kv_heads, nullptr, nullptr, nullptr, out, lse, p, part, stream);
  } else {
    if (bias) launch_d<64, true>(q, k, v, ni, n_q_heads, n_kv_heads, key_score, gain, tau, out, lse, p, part, stream);
    else launch_d<64, false>(q, k, v, ni, n_q_heads, n_kv_heads, nullptr, nullptr, nullptr, out, lse, p, part, stream);
  }
  return hipGetLastError();
}

}  // namespace tg
