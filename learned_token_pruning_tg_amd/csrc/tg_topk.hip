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
// histograms; the ordered output is one pass of block-wide scans.  Bit-exact
// and deterministic by construction on both paths below.
//  * Short inputs: one 1024-thread work-group does all of it (no global
//    atomics, no inter-block ordering).  Every score is read once, into
//    registers as its key (16 rows per thread, laid out so that wave-wide
//    loads and output stores are contiguous; buffer loads past n return zeros
//    and are ignored), and the three digit passes and the ordered output pass
//    work from those registers; each pair of waves counts into its own copy
//    of the histogram (scores bunch into a few top digits, so one shared
//    histogram serialises on LDS atomics).
//  * Long inputs: the same passes spread over up to 1024 work-groups with
//    global histograms and per-range counts in the caller's workspace (see
//    the multi-work-group section).
#include <mutex>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCopies = 8;                         // histogram copies (two waves each)
constexpr int kPerThread = 16;                     // rows per thread
// Rows up to which one work-group does it all (each thread holding 16 keys):
// up to here the multi-group path's six dependent launches cost more than
// they save, above it less (measured: 16.8 vs 21 us at 16384 rows; 25.6 vs
// 21.9 us at 16400, 26.9 vs 22.6 us at 24576, 108 vs 24 us at 128k).
constexpr int64_t kSingleGroupMax = static_cast<int64_t>(kThreads) * kPerThread;   // 16384

// Monotone 32-bit key of a float32 score.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;                    // -0.0 -> +0.0
  const uint32_t key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (x != x) ? 0u : key;                      // NaN below -inf
}

// Block-wide exclusive scan of one uint32 per thread (NW waves); returns the
// prefix and writes the total to *total.  Uses `tmp` (NW entries of LDS).
template <int NW>
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
  for (int w = 0; w < NW; ++w) {
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
                                                               int32_t* __restrict__ out,
                                                               uint32_t* __restrict__ out_scores) {
  __shared__ uint32_t hist[kCopies][kBins];
  __shared__ uint32_t scan_tmp[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x;
  const int n_doc = de - db;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scores, static_cast<uint32_t>(n) * 4u);
  uint32_t* my_hist = hist[(tid >> 6) % kCopies];
  uint32_t thresh;   // keys > thresh are kept
  uint32_t ties;     // number of keys == thresh kept, lowest index first

  // Every score this thread handles is read once, as its key: row
  // kThreads * r + tid (the output pass's layout, so wave-wide loads are
  // contiguous); rows past n read as zeros and are never used.
  uint32_t key[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r)
    key[r] = score_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rs, static_cast<int>((kThreads * r + tid) * 4), 0, 0)));

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
#pragma unroll
      for (int r = 0; r < kPerThread; ++r) {
        const int i = kThreads * r + tid;
        if (i >= db && i < de && (key[r] & pmask) == prefix)
          atomicAdd(&my_hist[(key[r] >> shift) & dmask], 1u);
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
      const uint32_t above = block_exclusive_scan<kWaves>(ha + hb, scan_tmp, &tot);
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

  // Ordered output over all rows: thread t holds rows kThreads * r + t
  // (r < kPerThread), so every wave-wide store touches consecutive
  // positions.  Per (r, wave): ballots of the rows kept for sure and of the
  // document rows equal to the threshold; their counts (below 2^16 each) are
  // scanned in row order (r-major, wave-minor) by one wave, and a lane's
  // position adds the set bits of the ballots below it.
  __shared__ uint32_t cnt[kPerThread * kWaves];   // packed: sure | eq << 16
  const int lane = tid & 63, wave = tid >> 6;
  uint64_t b_sure[kPerThread], b_eq[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int i = kThreads * r + tid;
    bool sure = false, eq = false;
    if (i < n) {
      if (i < db || i >= de) {
        sure = true;
      } else {
        sure = key[r] > thresh;
        eq = key[r] == thresh;
      }
    }
    b_sure[r] = __ballot(sure);
    b_eq[r] = __ballot(eq);
    if (lane == 0)
      cnt[r * kWaves + wave] = static_cast<uint32_t>(__popcll(b_sure[r])) |
                               (static_cast<uint32_t>(__popcll(b_eq[r])) << 16);
  }
  __syncthreads();
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
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const uint32_t base = cnt[r * kWaves + wave];
    const uint64_t below = (1ull << lane) - 1ull;
    const uint32_t sure_pre = (base & 0xFFFFu) + static_cast<uint32_t>(__popcll(b_sure[r] & below));
    const uint32_t eq_pre = (base >> 16) + static_cast<uint32_t>(__popcll(b_eq[r] & below));
    const bool is_sure = (b_sure[r] >> lane) & 1ull, is_eq = (b_eq[r] >> lane) & 1ull;
    const uint32_t pos = sure_pre + (eq_pre < ties ? eq_pre : ties);
    // pos < m_total holds by construction; the guard keeps a logic error
    // from ever writing past the caller's buffer.
    if ((is_sure || (is_eq && eq_pre < ties)) && pos < static_cast<uint32_t>(m_total)) {
      out[pos] = kThreads * r + tid;
      // the kept score itself, bit for bit (re-read: the key above folds -0
      // and every NaN)
      if (out_scores != nullptr)
        out_scores[pos] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, static_cast<int>((kThreads * r + tid) * 4), 0, 0);
    }
  }
}


// ---------------------------------------------------------------------------
// Multi-work-group select for long score vectors.  The same threshold key
// and tie budget, found by the same three digit passes, but every pass is a
// launch of G work-groups over contiguous row ranges that add their LDS
// histograms into global ones (integer sums: the totals, and so the result,
// do not depend on the order of the atomics).  Each pass starts by
// re-deriving the digits chosen so far from the previous histograms; work-group
// 0 also records them for the later launches.  A count launch then gives
// every row range its number of surely kept rows and of threshold ties, and
// the write launch places each range's kept rows at the offset the ranges
// before it imply (ties go to the lowest indices).
// ---------------------------------------------------------------------------
constexpr int kMThreads = 256;
constexpr int kMWaves = kMThreads / 64;
constexpr int kMRowsPerThread = 8;                     // two 16-byte loads per sub-range
constexpr int kMSub = kMThreads * kMRowsPerThread;     // rows per sub-range (block counts < 2^16)
constexpr int kMaxGroups = 1024;

// Workspace words: three global histograms, the selection state, then a
// (sure, ties) count pair per work-group.
constexpr int kWsHist1 = 0, kWsHist2 = 2048, kWsHist3 = 4096;
constexpr int kWsSel = 5120;      // [0..2] after digit 1, [3..5] after digit 2, [6..7] T, ties
constexpr int kWsCounts = 5136;

struct TopkPlan {
  int groups, rows_per_group;
};

TopkPlan topk_plan(int64_t n) {
  const int64_t subs = (n + kMSub - 1) / kMSub;
  const int64_t subs_per_group = (subs + kMaxGroups - 1) / kMaxGroups;
  TopkPlan p;
  p.rows_per_group = static_cast<int>(subs_per_group * kMSub);
  p.groups = static_cast<int>((n + p.rows_per_group - 1) / p.rows_per_group);
  return p;
}

// Digit d (descending order over NB bins of global histogram h) with
// above(d) < rem <= above(d) + h[d], above(d) = sum of the bins above d.
// Needs 1 <= rem <= sum of h.  Every thread returns the same (d, above).
template <int NB>
__device__ __forceinline__ void select_digit(const uint32_t* __restrict__ h, uint32_t rem,
                                             uint32_t* tmp, uint32_t* sel, uint32_t& d,
                                             uint32_t& above) {
  constexpr int PER = NB / kMThreads;
  const int t = threadIdx.x;
  uint32_t v[PER], sum = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    v[e] = h[NB - 1 - (PER * t + e)];
    sum += v[e];
  }
  uint32_t tot;
  uint32_t a = block_exclusive_scan<kMWaves>(sum, tmp, &tot);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (a < rem && rem <= a + v[e]) {
      sel[0] = static_cast<uint32_t>(NB - 1 - (PER * t + e));
      sel[1] = a;
    }
    a += v[e];
  }
  __syncthreads();
  d = sel[0];
  above = sel[1];
  __syncthreads();
}

__global__ __launch_bounds__(kMThreads) void topk_clear_kernel(uint32_t* __restrict__ ws) {
  for (int i = threadIdx.x; i < kWsSel; i += kMThreads) ws[i] = 0u;
}

// Digit pass P (1: bits 31..21, 2: bits 20..10, 3: bits 9..0) over the
// document rows of this work-group's range that match the digits chosen so far.
template <int P>
__global__ __launch_bounds__(kMThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                              int n, int db, int de, int k,
                                                              int rows_per_group,
                                                              uint32_t* __restrict__ ws) {
  constexpr int NB = P == 3 ? 1024 : 2048;
  constexpr int SHIFT = P == 1 ? 21 : P == 2 ? 10 : 0;
  __shared__ uint32_t hist[kMWaves][NB];   // one copy per wave: few top digits take most rows
  __shared__ uint32_t tmp[kMWaves], sel[2];
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  if (P == 2) {
    uint32_t d, above;
    select_digit<2048>(ws + kWsHist1, static_cast<uint32_t>(k), tmp, sel, d, above);
    prefix = d << 21;
    pmask = 0x7FFu << 21;
    if (blockIdx.x == 0 && tid == 0) {
      ws[kWsSel + 0] = prefix;
      ws[kWsSel + 1] = pmask;
      ws[kWsSel + 2] = static_cast<uint32_t>(k) - above;
    }
  } else if (P == 3) {
    const uint32_t rem = ws[kWsSel + 2];
    uint32_t d, above;
    select_digit<2048>(ws + kWsHist2, rem, tmp, sel, d, above);
    prefix = ws[kWsSel + 0] | (d << 10);
    pmask = ws[kWsSel + 1] | (0x7FFu << 10);
    if (blockIdx.x == 0 && tid == 0) {
      ws[kWsSel + 3] = prefix;
      ws[kWsSel + 4] = pmask;
      ws[kWsSel + 5] = rem - above;
    }
  }
  for (int b = tid; b < kMWaves * NB; b += kMThreads) (&hist[0][0])[b] = 0u;
  __syncthreads();
  uint32_t* my_hist = hist[tid >> 6];
  const int r0 = blockIdx.x * rows_per_group;
  const int lo = max(r0, db), hi = min(min(r0 + rows_per_group, n), de);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scores, static_cast<uint32_t>(n) * 4u);
  for (int j = (lo & ~3) + 4 * tid; j < hi; j += 4 * kMThreads) {
    const u32x4 x = bload16(rs, static_cast<uint32_t>(j) * 4u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = score_key(__uint_as_float(x[e]));
      if (j + e >= lo && j + e < hi && (key & pmask) == prefix)
        atomicAdd(&my_hist[(key >> SHIFT) & (NB - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = ws + (P == 1 ? kWsHist1 : P == 2 ? kWsHist2 : kWsHist3);
  for (int b = tid; b < NB; b += kMThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) c += hist[w][b];
    if (c != 0u) atomicAdd(&gh[b], c);
  }
}

// Row r of [0, n): is it kept for sure (non-document, or key > T), or a tie?
__device__ __forceinline__ void classify(uint32_t bits, int r, int n, int db, int de, uint32_t T,
                                         bool& sure, bool& eq) {
  sure = false;
  eq = false;
  if (r < n) {
    if (r < db || r >= de) {
      sure = true;
    } else {
      const uint32_t key = score_key(__uint_as_float(bits));
      sure = key > T;
      eq = key == T;
    }
  }
}

// T and the tie budget (from the third histogram, or given), then this
// range's (sure, ties) counts.
__global__ __launch_bounds__(kMThreads) void topk_count_kernel(const float* __restrict__ scores,
                                                               int n, int db, int de, int derive,
                                                               uint32_t t_given, uint32_t ties_given,
                                                               int rows_per_group,
                                                               uint32_t* __restrict__ ws) {
  __shared__ uint32_t tmp[kMWaves], sel[2];
  const int tid = threadIdx.x;
  uint32_t T = t_given, ties = ties_given;
  if (derive) {
    const uint32_t rem = ws[kWsSel + 5];
    uint32_t d, above;
    select_digit<1024>(ws + kWsHist3, rem, tmp, sel, d, above);
    T = ws[kWsSel + 3] | d;
    ties = rem - above;
  }
  if (blockIdx.x == 0 && tid == 0) {
    ws[kWsSel + 6] = T;
    ws[kWsSel + 7] = ties;
  }
  const int r0 = blockIdx.x * rows_per_group;
  const int r1 = min(r0 + rows_per_group, n);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scores, static_cast<uint32_t>(n) * 4u);
  uint32_t sure_n = 0, eq_n = 0;
  for (int j = r0 + 4 * tid; j < r1; j += 4 * kMThreads) {
    const u32x4 x = bload16(rs, static_cast<uint32_t>(j) * 4u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool sure, eq;
      classify(x[e], j + e, r1, db, de, T, sure, eq);
      sure_n += sure;
      eq_n += eq;
    }
  }
  uint32_t tot_s, tot_e;
  block_exclusive_scan<kMWaves>(sure_n, tmp, &tot_s);
  block_exclusive_scan<kMWaves>(eq_n, tmp, &tot_e);
  if (tid == 0) {
    ws[kWsCounts + 2 * blockIdx.x] = tot_s;
    ws[kWsCounts + 2 * blockIdx.x + 1] = tot_e;
  }
}

// Ordered output: this range's offset from the counts of the ranges before
// it, then sub-ranges of kMSub rows, thread t taking rows 8 t .. 8 t + 7 of
// each, positions from block scans.
__global__ __launch_bounds__(kMThreads) void topk_write_kernel(const float* __restrict__ scores,
                                                               int n, int db, int de,
                                                               int rows_per_group, int m_total,
                                                               const uint32_t* __restrict__ ws,
                                                               int32_t* __restrict__ out,
                                                               uint32_t* __restrict__ out_scores) {
  __shared__ uint32_t tmp[kMWaves];
  const int tid = threadIdx.x;
  const uint32_t T = ws[kWsSel + 6], ties = ws[kWsSel + 7];
  uint32_t out_base = 0, eq_before = 0;
  for (int i0 = 0; i0 < static_cast<int>(blockIdx.x); i0 += kMThreads) {
    const int i = i0 + tid;
    const bool live = i < static_cast<int>(blockIdx.x);
    const uint32_t sure = live ? ws[kWsCounts + 2 * i] : 0u;
    const uint32_t eq = live ? ws[kWsCounts + 2 * i + 1] : 0u;
    uint32_t tot_eq, tot_kept;
    const uint32_t tb = eq_before + block_exclusive_scan<kMWaves>(eq, tmp, &tot_eq);
    const uint32_t left = ties > tb ? ties - tb : 0u;
    block_exclusive_scan<kMWaves>(sure + (eq < left ? eq : left), tmp, &tot_kept);
    out_base += tot_kept;
    eq_before += tot_eq;
  }
  const int r0 = blockIdx.x * rows_per_group;
  const int r1 = min(r0 + rows_per_group, n);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scores, static_cast<uint32_t>(n) * 4u);
  for (int s0 = r0; s0 < r1; s0 += kMSub) {
    const int row0 = s0 + kMRowsPerThread * tid;
    const u32x4 xa = bload16(rs, static_cast<uint32_t>(row0) * 4u);
    const u32x4 xb = bload16(rs, static_cast<uint32_t>(row0 + 4) * 4u);
    uint32_t sure_m = 0, eq_m = 0;   // bit e: row row0 + e
#pragma unroll
    for (int e = 0; e < kMRowsPerThread; ++e) {
      bool sure, eq;
      classify(e < 4 ? xa[e] : xb[e - 4], row0 + e, r1, db, de, T, sure, eq);
      sure_m |= static_cast<uint32_t>(sure) << e;
      eq_m |= static_cast<uint32_t>(eq) << e;
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan<kMWaves>(
        static_cast<uint32_t>(__builtin_popcount(sure_m)) |
            (static_cast<uint32_t>(__builtin_popcount(eq_m)) << 16), tmp, &tot);
    const uint32_t left = ties > eq_before ? ties - eq_before : 0u;   // ties still to take
    uint32_t sp = pre & 0xFFFFu, ep = pre >> 16;
#pragma unroll
    for (int e = 0; e < kMRowsPerThread; ++e) {
      const bool sure = (sure_m >> e) & 1u, eq = (eq_m >> e) & 1u;
      const uint32_t pos = out_base + sp + (ep < left ? ep : left);
      // pos < m_total holds by construction; the guard keeps a logic error
      // from ever writing past the caller's buffer.
      if ((sure || (eq && ep < left)) && pos < static_cast<uint32_t>(m_total)) {
        out[pos] = row0 + e;
        if (out_scores != nullptr) out_scores[pos] = e < 4 ? xa[e] : xb[e - 4];   // bit for bit
      }
      sp += sure;
      ep += eq;
    }
    const uint32_t eq_tot = tot >> 16;
    out_base += (tot & 0xFFFFu) + (eq_tot < left ? eq_tot : left);
    eq_before += eq_tot;
  }
}

}  // namespace

size_t topk_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return static_cast<size_t>(kWsCounts + 2 * topk_plan(n).groups) * 4u;
}

hipError_t launch_topk_select(const float* scores, int64_t n, int64_t doc_begin, int64_t doc_end,
                              int64_t k_doc, int32_t* kept_idx, float* kept_scores,
                              void* workspace, hipStream_t stream) {
  uint32_t* ks = reinterpret_cast<uint32_t*>(kept_scores);
  if (n == 0) return hipSuccess;
  const int64_t n_doc = doc_end - doc_begin;
  const int k = static_cast<int>(k_doc < n_doc ? k_doc : n_doc);
  const int m_total = static_cast<int>(k + (n - n_doc));
  const int ni = static_cast<int>(n), db = static_cast<int>(doc_begin), de = static_cast<int>(doc_end);
  if (n <= kSingleGroupMax) {
    hipLaunchKernelGGL(topk_select_kernel, dim3(1), dim3(kThreads), 0, stream, scores, ni, db, de,
                       k, m_total, kept_idx, ks);
    return hipGetLastError();
  }
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  const TopkPlan p = topk_plan(n);
  const dim3 grid(static_cast<unsigned>(p.groups)), block(kMThreads);
  const bool derive = k > 0 && k < n_doc;
  if (derive) {
    hipLaunchKernelGGL(topk_clear_kernel, dim3(1), block, 0, stream, ws);
    hipLaunchKernelGGL(topk_hist_kernel<1>, grid, block, 0, stream, scores, ni, db, de, k,
                       p.rows_per_group, ws);
    hipLaunchKernelGGL(topk_hist_kernel<2>, grid, block, 0, stream, scores, ni, db, de, k,
                       p.rows_per_group, ws);
    hipLaunchKernelGGL(topk_hist_kernel<3>, grid, block, 0, stream, scores, ni, db, de, k,
                       p.rows_per_group, ws);
  }
  // k == 0: nothing exceeds or equals the threshold; k == n_doc: everything
  // is kept (every key is >= 0, the ties budget covers all rows).
  const uint32_t t_given = k == 0 ? 0xFFFFFFFFu : 0u;
  const uint32_t ties_given = k == 0 ? 0u : static_cast<uint32_t>(n_doc);
  hipLaunchKernelGGL(topk_count_kernel, grid, block, 0, stream, scores, ni, db, de,
                     derive ? 1 : 0, t_given, ties_given, p.rows_per_group, ws);
  hipLaunchKernelGGL(topk_write_kernel, grid, block, 0, stream, scores, ni, db, de,
                     p.rows_per_group, m_total, ws, kept_idx, ks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The same selection for callers that cannot allocate: its scratch is a
// file-scope device array of kTopkScratchBytes, one per GPU, held until the
// process ends.  In host code `topk_scratch` names a host-side stand-in, not
// a device address: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in topk_scratch_dev.
// Every call on a GPU shares that GPU's array (calls that overlap on one GPU
// race); the clear kernel zeroes the histograms at the start of each call and
// every other word is written before it is read within the call.
// ---------------------------------------------------------------------------
namespace {
static __device__ __align__(256) char topk_scratch[kTopkScratchBytes];
static_assert((kWsCounts + 2 * kMaxGroups) * 4 <= kTopkScratchBytes, "scratch too small");
constexpr int kMaxDevices = 64;
std::mutex topk_scratch_mu;
void* topk_scratch_dev[kMaxDevices] = {};

hipError_t topk_scratch_ptr(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(topk_scratch_mu);
  if (topk_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(topk_scratch));
    if (e != hipSuccess) return e;
    topk_scratch_dev[dev] = p;
  }
  *ptr = topk_scratch_dev[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_topk_select_noalloc(const float* scores, int64_t n, int64_t doc_begin,
                                      int64_t doc_end, int64_t k_doc, int32_t* kept_idx,
                                      hipStream_t stream) {
  if (n == 0) return hipSuccess;
  void* ws = nullptr;
  if (n > kSingleGroupMax) {          // the one-work-group path uses no scratch
    const hipError_t e = topk_scratch_ptr(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_topk_select(scores, n, doc_begin, doc_end, k_doc, kept_idx, nullptr, ws, stream);
}

}  // namespace tg
