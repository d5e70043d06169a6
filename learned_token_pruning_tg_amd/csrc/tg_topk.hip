// Top-K selection of document rows for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"): a top-K
// selector keeps the best-scoring tokens of the document part of the prompt;
// the question is never pruned.  Read here as: rank document rows by a total
// order on float32 scores (-0.0 == +0.0, NaN below -inf, ties to the lower
// index), keep the first min(K, N_doc), keep every non-document row, and emit
// the kept indices in ascending order.
//
// Design: the kept set is fixed by a threshold key T and a tie budget: every
// document key > T is kept, and the first `ties` keys == T in index order.
// T is found by a 3-pass MSB radix select (11 + 11 + 10 bits) with LDS
// histograms; the ordered output is one pass of block-wide scans.  The whole
// problem (<= 512 KiB of scores at 128k tokens, L2-resident after the first
// pass) is latency-bound, so one 1024-thread work-group does all of it: no
// global atomics, no workspace, no inter-block ordering, bit-exact and
// deterministic by construction.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kPerThread = 4;                      // rows per thread per output chunk
constexpr int kChunk = kThreads * kPerThread;

// Monotone 32-bit key of a float32 score.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;                    // -0.0 -> +0.0
  const uint32_t key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (x != x) ? 0u : key;                      // NaN below -inf
}

// Block-wide exclusive scan of one uint32 per thread; returns the prefix and
// writes the total to *total.  Uses `tmp` (kWaves entries of LDS).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* tmp,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  uint32_t wave_base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = tmp[w];
    wave_base += (w < wave) ? t : 0u;
    sum += t;
  }
  __syncthreads();  // tmp may be reused by the caller
  *total = sum;
  return wave_base + inc - x;
}

__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ scores,
                                                               int n, int db, int de, int k,
                                                               int m_total,
                                                               int32_t* __restrict__ out) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_tmp[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x;
  const int n_doc = de - db;
  uint32_t thresh;   // keys > thresh are kept
  uint32_t ties;     // number of keys == thresh kept, lowest index first

  if (k <= 0) {
    thresh = 0xFFFFFFFFu;  // no key exceeds it and none equals it (max key is +inf's)
    ties = 0;
  } else if (k >= n_doc) {
    thresh = 0u;
    ties = static_cast<uint32_t>(n_doc);
  } else {
    uint32_t prefix = 0, pmask = 0, remaining = static_cast<uint32_t>(k);
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = shifts[pass];
      const uint32_t dmask = (1u << widths[pass]) - 1u;
      for (int b = tid; b < kBins; b += kThreads) hist[b] = 0;
      __syncthreads();
      for (int i = db + tid; i < de; i += kThreads) {
        const uint32_t key = score_key(scores[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      // Thread t owns bins (2047 - 2t) and (2046 - 2t): thread order is
      // descending digit order.
      const int ba = kBins - 1 - 2 * tid, bb = ba - 1;
      const uint32_t ha = hist[ba], hb = hist[bb];
      uint32_t tot;
      const uint32_t above = block_exclusive_scan(ha + hb, scan_tmp, &tot);
      if (above < remaining && remaining <= above + ha) {
        sel_digit = static_cast<uint32_t>(ba);
        sel_above = above;
      } else if (above + ha < remaining && remaining <= above + ha + hb) {
        sel_digit = static_cast<uint32_t>(bb);
        sel_above = above + ha;
      }
      __syncthreads();
      remaining -= sel_above;
      prefix |= sel_digit << shift;
      pmask |= dmask << shift;
      __syncthreads();
    }
    thresh = prefix;
    ties = remaining;
  }

  // Ordered output over all rows.  Per thread: kPerThread consecutive rows.
  // Packed counts: low 16 bits = rows kept regardless of ties, high 16 bits =
  // document rows equal to the threshold.
  uint32_t out_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    const int i0 = c0 + tid * kPerThread;
    uint32_t sure = 0, eq = 0;
    uint32_t flags = 0;  // bit 2r: kept for sure, bit 2r+1: equal to threshold
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int i = i0 + r;
      if (i < n) {
        if (i < db || i >= de) {
          flags |= 1u << (2 * r);
          ++sure;
        } else {
          const uint32_t key = score_key(scores[i]);
          if (key > thresh) {
            flags |= 1u << (2 * r);
            ++sure;
          } else if (key == thresh) {
            flags |= 2u << (2 * r);
            ++eq;
          }
        }
      }
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan(sure | (eq << 16), scan_tmp, &tot);
    const uint32_t sure_pre = pre & 0xFFFFu, eq_pre = pre >> 16;
    const uint32_t sure_tot = tot & 0xFFFFu, eq_tot = tot >> 16;
    // ties still available when this thread's rows start
    const uint32_t ties_left_chunk = ties > eq_base ? ties - eq_base : 0u;
    uint32_t eq_seen = eq_pre;
    uint32_t taken_before = eq_pre < ties_left_chunk ? eq_pre : ties_left_chunk;
    uint32_t pos = out_base + sure_pre + taken_before;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const uint32_t f = (flags >> (2 * r)) & 3u;
      // pos < m_total holds by construction; the guard keeps a logic error
      // from ever writing past the caller's buffer.
      if (f == 1u) {
        if (pos < static_cast<uint32_t>(m_total)) out[pos] = i0 + r;
        ++pos;
      } else if (f == 2u) {
        if (eq_seen < ties_left_chunk) {
          if (pos < static_cast<uint32_t>(m_total)) out[pos] = i0 + r;
          ++pos;
        }
        ++eq_seen;
      }
    }
    const uint32_t taken_chunk = eq_tot < ties_left_chunk ? eq_tot : ties_left_chunk;
    out_base += sure_tot + taken_chunk;
    eq_base += eq_tot;
  }
}

}  // namespace

hipError_t launch_topk_select(const float* scores, int64_t n, int64_t doc_begin, int64_t doc_end,
                              int64_t k_doc, int32_t* kept_idx, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t n_doc = doc_end - doc_begin;
  const int k = static_cast<int>(k_doc < n_doc ? k_doc : n_doc);
  const int m_total = static_cast<int>(k + (n - n_doc));
  hipLaunchKernelGGL(topk_select_kernel, dim3(1), dim3(kThreads), 0, stream, scores,
                     static_cast<int>(n), static_cast<int>(doc_begin), static_cast<int>(doc_end), k,
                     m_total, kept_idx);
  return hipGetLastError();
}

}  // namespace tg
