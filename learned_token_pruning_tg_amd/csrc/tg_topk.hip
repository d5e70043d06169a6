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
// deterministic by construction.  Scores are read 16 bytes per lane (buffer
// loads: reads past n return zeros and are ignored); each pair of waves
// counts into its own copy of the histogram (scores bunch into a few top
// digits, so one shared histogram serialises on LDS atomics); the output pass
// works on 16-row-per-thread chunks laid out so that wave-wide loads and
// stores are contiguous, and loads the next chunk before scanning this one.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCopies = 8;                         // histogram copies (two waves each)
constexpr int kPerThread = 16;                     // rows per thread per output chunk
constexpr int kChunk = kThreads * kPerThread;      // block counts stay below 2^16

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
  __shared__ uint32_t hist[kCopies][kBins];
  __shared__ uint32_t scan_tmp[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x;
  const int n_doc = de - db;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scores, static_cast<uint32_t>(n) * 4u);
  uint32_t* my_hist = hist[(tid >> 6) % kCopies];
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
      for (int b = tid; b < kCopies * kBins; b += kThreads) (&hist[0][0])[b] = 0;
      __syncthreads();
#pragma unroll 4
      for (int j = (db & ~3) + 4 * tid; j < de; j += 4 * kThreads) {
        const u32x4 x = bload16(rs, static_cast<uint32_t>(j) * 4u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = score_key(__uint_as_float(x[e]));
          if (j + e >= db && j + e < de && (key & pmask) == prefix)
            atomicAdd(&my_hist[(key >> shift) & dmask], 1u);
        }
      }
      __syncthreads();
      // Thread t owns bins (2047 - 2t) and (2046 - 2t): thread order is
      // descending digit order.
      const int ba = kBins - 1 - 2 * tid, bb = ba - 1;
      uint32_t ha = 0, hb = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        ha += hist[c][ba];
        hb += hist[c][bb];
      }
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

  // Ordered output over all rows, in chunks of kChunk rows: thread t takes
  // rows c0 + kThreads * r + t (r < kPerThread), so every wave-wide load and
  // store touches consecutive rows / positions.  Per (r, wave): ballots of
  // the rows kept for sure and of the document rows equal to the threshold;
  // their counts are scanned in row order (r-major, wave-minor) by one wave,
  // and a lane's position adds the set bits of the ballots below it.
  __shared__ uint32_t cnt[kPerThread * kWaves];   // packed: sure | eq << 16
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t out_base = 0, eq_base = 0;
  uint32_t cur[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r)
    cur[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>((kThreads * r + tid) * 4), 0, 0);
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    uint32_t nxt[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r)   // zeros past n
      nxt[r] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, static_cast<int>(static_cast<uint32_t>(c0 + kChunk + kThreads * r + tid) * 4u), 0, 0);
    uint64_t b_sure[kPerThread], b_eq[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int i = c0 + kThreads * r + tid;
      bool sure = false, eq = false;
      if (i < n) {
        if (i < db || i >= de) {
          sure = true;
        } else {
          const uint32_t key = score_key(__uint_as_float(cur[r]));
          sure = key > thresh;
          eq = key == thresh;
        }
      }
      b_sure[r] = __ballot(sure);
      b_eq[r] = __ballot(eq);
      if (lane == 0)
        cnt[r * kWaves + wave] = static_cast<uint32_t>(__popcll(b_sure[r])) |
                                 (static_cast<uint32_t>(__popcll(b_eq[r])) << 16);
    }
    __syncthreads();
    uint32_t tot = 0;
    if (wave == 0) {
      // exclusive scan of the kPerThread * kWaves packed counts, 4 per lane
      constexpr int PL = kPerThread * kWaves / 64;
      uint32_t v[PL], run = 0;
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        v[e] = cnt[lane * PL + e];
        run += v[e];
      }
      uint32_t inc = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      uint32_t pre = inc - run;
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        cnt[lane * PL + e] = pre;
        pre += v[e];
      }
      if (lane == 63) scan_tmp[0] = inc;
    }
    __syncthreads();
    tot = scan_tmp[0];
    const uint32_t sure_tot = tot & 0xFFFFu, eq_tot = tot >> 16;
    // ties still available when this chunk starts
    const uint32_t ties_left_chunk = ties > eq_base ? ties - eq_base : 0u;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const uint32_t base = cnt[r * kWaves + wave];
      const uint64_t below = (1ull << lane) - 1ull;
      const uint32_t sure_pre = (base & 0xFFFFu) + static_cast<uint32_t>(__popcll(b_sure[r] & below));
      const uint32_t eq_pre = (base >> 16) + static_cast<uint32_t>(__popcll(b_eq[r] & below));
      const bool is_sure = (b_sure[r] >> lane) & 1ull, is_eq = (b_eq[r] >> lane) & 1ull;
      const uint32_t pos = out_base + sure_pre + (eq_pre < ties_left_chunk ? eq_pre : ties_left_chunk);
      // pos < m_total holds by construction; the guard keeps a logic error
      // from ever writing past the caller's buffer.
      if ((is_sure || (is_eq && eq_pre < ties_left_chunk)) && pos < static_cast<uint32_t>(m_total))
        out[pos] = c0 + kThreads * r + tid;
      cur[r] = nxt[r];
    }
    const uint32_t taken_chunk = eq_tot < ties_left_chunk ? eq_tot : ties_left_chunk;
    out_base += sure_tot + taken_chunk;
    eq_base += eq_tot;
    __syncthreads();   // cnt and scan_tmp are rewritten by the next chunk
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
