// Token-gated causal GQA attention, backward, for gfx950.
//
// Method (lucasainews.com TokenGate article, section "작동 방식"; fugumt.com
// abstract): the kept keys' gate scores enter the logits as a bias, scaled by
// a per-head gain, with a per-head temperature on q.k; the bias is how a
// training loss reaches the gate.  With c_h = 1 / (sqrt(d) tau_h),
//     logit_ij = c_h q_i.k_j + g_h s_j (j <= i),  P = softmax_j,  O_i = sum_j P_ij v_j,
// and given dO the gradients are (chain rule; D_i = dO_i.O_i = sum_j P_ij dP_ij):
//     dP_ij = dO_i.v_j,   dS_ij = P_ij (dP_ij - D_i)
//     dv_j = sum_h sum_i P_ij dO_i          dk_j = sum_h c_h sum_i dS_ij q_i
//     dq_i = c_h sum_j dS_ij k_j            ds_j = sum_h g_h sum_i dS_ij
//     dg_h = sum_ij dS_ij s_j               dtau_h = -(1 / tau_h) sum_i q_i.dq_i
// (the last because d logit / d tau_h = -c_h q.k / tau_h).
//
// Launches, all deterministic (every sum in a fixed order, no atomics):
// 1. bwd_pack: per (query head, 32-row tile) the rows' -lse / c_h (-inf past
//    n) and -D.
// 2. bwd_dkdv: one work-group per (query head, 128 keys), a wave per 32 keys
//    with their K and V fragments in registers, over 32-query steps from the
//    diagonal on: S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16_bf16 (lane
//    = key, registers = queries), P and dS in fp32, then dV += P^T dO and
//    dK += dS^T Q with P and dS as bf16 A fragments straight from registers
//    and the dO and Q B fragments read transposed (ds_read_b64_tr_b16) out of
//    the same row tiles the S and dP steps read.  Q and dO rows arrive by
//    buffer-to-LDS DMA into a double-buffered ring, one barrier per step; the
//    S and dP accumulators start from -lse / c_h and -D.  Writes fp32
//    per-head dK/dV partials and the per-head column sums sum_i dS_ij.
// 3. bwd_dq: one work-group per (query head, 128 queries), a wave per 32
//    queries with their Q and dO fragments in registers, over 32-key steps up
//    to the diagonal: S^T = K Q^T, dP^T = V dO^T (lane = query), dS^T, then
//    dQ^T += K^T dS^T with the K^T A fragments read transposed out of the K
//    rows tile.  Writes dQ (bf16) and per work-group sum_i q_i.dq_i.
// 4. bwd_finish: dK, dV = sum over the heads of each KV group (bf16) and the
//    score gradient ds_j = sum_h g_h colsum_hj; split dQ partials summed; the
//    gain and temperature gradients dg_h, dtau_h.
// Short kept prefixes leave too few long walks to fill the chip; then walks
// are cut into chunks whose fp32 partials the reduce launches add in order.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kThreads = 256;           // four waves
constexpr int kRows = 32;               // rows of a tile image / of one wave
constexpr int kWgRows = 128;            // rows (keys or queries) of a work-group

template <int D>
struct Bwd {
  static constexpr int KS = D / 16;                 // k-steps over d
  static constexpr int DT = D / 32;                 // 32-wide d tiles
  static constexpr int ROW = D * 2;                 // bytes of one row tile row (LDS, unpadded)
  static constexpr int ROWS_TILE = kRows * ROW;     // a 32-row tile in LDS
  static constexpr int N_ROW_DMA = ROWS_TILE / 1024;
  static_assert(ROWS_TILE % 1024 == 0, "whole 1 KiB DMA chunks");
  // XOR key of LDS row r: 16 consecutive rows hit 16 different 16-byte slots
  // modulo 256 bytes, so the A-fragment reads are free of bank conflicts.
  static __host__ __device__ constexpr int swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// MFMA fragment with the tile's rows as k and its dims as the 32 lanes of m
// (or n), read transposed out of a swizzled row tile (row r: 16-byte chunk c
// at slot c ^ swz(r)) by two ds_read_b64_tr_b16.  That instruction hands lane
// i = 4 a + c of each 16-lane group element c of the 8-byte rows that lanes
// a, a + 4, a + 8, a + 12 of the group address.  Lane j addresses row
// 16 g + 8 q + 4 hh + j / 4 at dims n0 + 16 (lane / 16 % 2) + 4 (j % 4), so
// lane l receives dim n0 + l % 32 of rows 16 g + 8 q + 4 hh + 0..3 in read
// q: element e of the fragment is row 16 g + 8 (e / 4) + 4 hh + e % 4, the
// row that C-register 8 g + e of lane half hh holds (the A or B fragment
// built from those registers on the other side of the product matches).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int g, int n0, int lane) {
  using T = Bwd<D>;
  const int j = lane & 15, hh = lane >> 5;
  const int d = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  v4i16 x[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 16 * g + 8 * q + 4 * hh + (j >> 2);
    const char* a = tile + r * T::ROW + (((d >> 3) ^ T::swz(r)) << 4) + (d & 7) * 2;
    x[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a));
  }
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 y = __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, y);
}

// Split walks.  A dK/dV work-group walks the 32-query steps from its
// diagonal to the end (key block kt: n_t - 4 kt steps), a dQ work-group the
// 32-key steps up to its diagonal (query block qt: at most 4 qt + 4).  When
// the longest walk exceeds 1.3x the average number of steps per resident
// work-group (512 of them), walks are cut into chunks of that length (never
// shorter than 8 steps), each a work-group writing its own fp32 partials;
// the reduce launches add the chunks in order.
struct Split {
  int len;   // steps per chunk
  int nc;    // chunks of the longest walk
};

Split choose_split(int64_t longest, double total_steps) {
  const double avg = total_steps / 512.0;
  int64_t len = longest;
  if (static_cast<double>(longest) > 1.3 * avg)
    len = std::max<int64_t>(8, static_cast<int64_t>(std::ceil(1.3 * avg)));
  len = std::max<int64_t>(1, std::min<int64_t>(len, longest));
  return Split{static_cast<int>(len), static_cast<int>((longest + len - 1) / len)};
}

// Workspace layout (byte offsets, each region 256-byte aligned).
struct BwdPlan {
  int64_t n_t32;     // 32-row tiles, rounded up to whole 128-row work-groups
  int64_t n_t128;
  int64_t mp;        // rows padded to n_t32 * 32
  Split kv, q;       // chunking of the dK/dV and dQ walks
  size_t ld, colsum, dkp, dvp, dgp, qdot, dqp, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

BwdPlan bwd_plan(int64_t n, int hq, int hkv, int d) {
  BwdPlan p{};
  p.n_t128 = (n + kWgRows - 1) / kWgRows;
  p.n_t32 = p.n_t128 * (kWgRows / kRows);
  p.mp = p.n_t32 * kRows;
  const int64_t t_real = (n + kRows - 1) / kRows;   // 32-row tiles holding rows
  double kv_steps = 0.0, q_steps = 0.0;
  for (int64_t b = 0; b < p.n_t128; ++b) {
    kv_steps += static_cast<double>(t_real - 4 * b);
    q_steps += static_cast<double>(std::min<int64_t>(4 * b + 4, t_real));
  }
  p.kv = choose_split(t_real, kv_steps * hq);
  p.q = choose_split(t_real, q_steps * hq);
  const size_t nkv = static_cast<size_t>(p.kv.nc), nq = static_cast<size_t>(p.q.nc);
  size_t o = 0;
  p.ld = o;     o = align256(o + static_cast<size_t>(hq) * p.n_t32 * 64 * 4);
  p.colsum = o; o = align256(o + nkv * hq * p.mp * 4);
  p.dkp = o;    o = align256(o + nkv * hq * p.mp * d * 4);
  p.dvp = o;    o = align256(o + nkv * hq * p.mp * d * 4);
  p.dgp = o;    o = align256(o + nkv * hq * p.n_t128 * 4);
  p.qdot = o;   o = align256(o + nq * hq * p.n_t128 * 4);
  p.dqp = o;    o = align256(o + (nq > 1 ? nq * p.mp * hq * d * 4 : 0));
  p.total = o;
  return p;
}

// Chunks of key block kt's dK/dV walk and of query block qt's dQ walk.
__host__ __device__ __forceinline__ int kv_chunks(int kt, int t_real, int len) {
  return (t_real - 4 * kt + len - 1) / len;
}
__host__ __device__ __forceinline__ int q_walk(int qt, int M) {
  return (min(qt * kWgRows + kWgRows, M) - 1) / kRows + 1;
}

// Work-group b -> (head, v): heads of one KV group on one XCD (work-groups
// are dealt round-robin over the 8 XCDs), v counting that head's units.
__device__ __forceinline__ void head_unit(int b, int hq, int& head, int& v) {
  if ((hq & 7) == 0) {
    const int hpx = hq >> 3, xcd = b & 7, slot = b >> 3;
    head = xcd * hpx + slot % hpx;
    v = slot / hpx;
  } else {
    head = b % hq;
    v = b / hq;
  }
}

// Round-to-nearest-even bf16 pair (lo in the low half): one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// Sum of x over lane l and lane l ^ 32.
__device__ __forceinline__ float add_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// bwd_pack: per (query head, 32-row tile) the rows' -lse / c_h (-inf past n)
// and -D, D_i = dO_i . O_i by eight lanes per row and a fixed butterfly.  O is
// the forward's fp32 output before its bf16 rounding: D then carries the
// forward's own arithmetic error only (with the rounded output, short rows,
// whose dS terms nearly cancel against D, lose most of their precision).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pack_kernel(
    const float* __restrict__ out, const float* __restrict__ lse, const bf16* __restrict__ dout,
    const float* __restrict__ tau, int M, int Hq, int n_t32, float* __restrict__ ld) {
  const int tid = threadIdx.x;
  const int h = blockIdx.x / n_t32, t = blockIdx.x % n_t32;
  const uint32_t stride = static_cast<uint32_t>(Hq) * D * 2;      // dout row bytes
  const uint32_t range = stride * static_cast<uint32_t>(M);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dout + static_cast<size_t>(h) * D, range);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + static_cast<size_t>(h) * D, 2 * range);
  const size_t tile = static_cast<size_t>(h) * n_t32 + t;
  const uint32_t row0 = static_cast<uint32_t>(t) * kRows;
  const int qi = tid >> 3, part = tid & 7;
  constexpr int PER = D / 8;        // dims per lane: 16 or 8
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    const uint32_t off = (row0 + qi) * stride + (part * PER + 8 * c) * 2;
    const u32x4 a = bload16(rd, off);
    const u32x4 o0 = bload16(ro, 2 * off), o1 = bload16(ro, 2 * off + 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4& o = w < 2 ? o0 : o1;
      acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(o[2 * (w & 1)]), acc);
      acc = fmaf(__uint_as_float(a[w] & 0xFFFF0000u), __uint_as_float(o[2 * (w & 1) + 1]), acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (part == 0) {
    // stored negated, lse in units of the head's q.k (lse / c_h): the dK/dV
    // steps start their S and dP accumulators from these values
    const int64_t row = static_cast<int64_t>(row0) + qi;
    const float inv_c = sqrtf(static_cast<float>(D)) * tau[h];
    float* dst = ld + tile * 64;
    dst[qi] = row < M ? -lse[static_cast<int64_t>(h) * M + row] * inv_c : -INFINITY;
    dst[32 + qi] = -acc;
  }
}

// ---------------------------------------------------------------------------
// bwd_dkdv
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void bwd_dkdv_body(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ tau, int M, int Hq, int Hkv,
    int n_t32, int mp, int clen, int nc, const float* __restrict__ ld, float* __restrict__ colsum,
    float* __restrict__ dkp, float* __restrict__ dvp, float* __restrict__ dgp, int bid,
    char* lds_all) {
  using T = Bwd<D>;
  constexpr int KS = T::KS, DT = T::DT;
  constexpr int NW = kThreads / 64;
  constexpr int NJR = T::N_ROW_DMA / NW;                     // row-tile DMA chunks per wave
  static_assert(T::N_ROW_DMA % NW == 0, "row tiles split evenly over the waves");

  // All of the kernel's LDS is one object.  The compiler tracks DMA into LDS
  // per object once there are several, and then makes every read of an
  // object wait for all DMA in flight into it, which would hold each step's
  // reads behind the next step's DMA; the explicit waits below order the ring.
  // The step's 64 (-lse/c_h, -D) values take 256 bytes of a 1 KiB stage: the
  // whole wave issues their DMA (a lane-divergent DMA made the compiler wait
  // for every DMA in flight before the step's first LDS read); lanes past 16
  // fetch the next steps' values, or zeros past the end, into the rest.
  auto* lds_qr = reinterpret_cast<char (*)[T::ROWS_TILE]>(lds_all);
  auto* lds_dr = reinterpret_cast<char (*)[T::ROWS_TILE]>(lds_all + 2 * T::ROWS_TILE);
  auto* lds_ld = reinterpret_cast<float (*)[256]>(lds_all + 4 * T::ROWS_TILE);
  float* lds_red = reinterpret_cast<float*>(lds_all + 4 * T::ROWS_TILE + 2 * 1024);

  int head, unit;
  head_unit(bid, Hq, head, unit);
  const int kt = unit / nc, ch = unit % nc;       // kt ascending: longest walks first
  const int t_end = (M + kRows - 1) / kRows;
  const int t_begin = kt * (kWgRows / kRows) + ch * clen;   // this chunk's query steps
  if (t_begin >= t_end) return;                   // past the walk: no chunk here
  const int t_stop = min(t_begin + clen, t_end);
  const int n_kt = (M + kWgRows - 1) / kWgRows;
  const int kvh = head / (Hq / Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int key0 = kt * kWgRows + wave * kRows;   // this wave's first key
  const int my_key = key0 + l32;

  // K and V fragments of this lane's key (B operands of S = Q K^T, dP = dO V^T)
  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;
  bf16x8 kf[KS], vf[KS];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + static_cast<size_t>(kvh) * D, kv_row * static_cast<uint32_t>(M));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + static_cast<size_t>(kvh) * D, kv_row * static_cast<uint32_t>(M));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = static_cast<uint32_t>(my_key) * kv_row + (16 * s + 8 * hh) * 2;
      kf[s] = as_bf16x8(bload16(rk, off));
      vf[s] = as_bf16x8(bload16(rv, off));
    }
  }
  const float c_h = 1.f / (sqrtf(static_cast<float>(D)) * tau[head]);
  const float alpha = kLog2e * c_h;
  const float bkey = my_key < M ? gain[head] * key_score[my_key] * kLog2e : 0.f;

  floatx16 dk[DT], dv[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }
  float csum = 0.f;

  // ---- DMA of one 32-query step into ring slot `buf`
  const uint32_t q_row = static_cast<uint32_t>(Hq) * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + static_cast<size_t>(head) * D, q_row * static_cast<uint32_t>(M));
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dout + static_cast<size_t>(head) * D, q_row * static_cast<uint32_t>(M));
  const __amdgpu_buffer_rsrc_t rld = make_rsrc(ld + static_cast<size_t>(head) * n_t32 * 64,
                                               static_cast<uint32_t>(n_t32) * 256);
  // Row tiles: the lane filling LDS slot s of row r fetches chunk s ^ swz(r)
  // of that row (Q and dO rows share the stride, hence one offset for both).
  // The offsets are formed at each DMA from a copy of the lane id the
  // compiler cannot see through: hoisted out of the loop they are live across
  // it, and at this register pressure they were spilled, and every reload's
  // wait also waited for the DMA issued just before it.
  auto fresh_lane = []() __attribute__((always_inline)) {
    int l = static_cast<int>(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
  };
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](int buf, int t) __attribute__((always_inline)) {
    const uint32_t row_off = static_cast<uint32_t>(t) * kRows * q_row;
    const int ln = fresh_lane();
#pragma unroll
    for (int jj = 0; jj < NJR; ++jj) {
      const int c = wave_s + NW * jj;
      const int byte = 1024 * c + 16 * ln;
      const int r = byte / T::ROW, slot = (byte % T::ROW) / 16;
      const uint32_t roff =
          static_cast<uint32_t>(r) * q_row + static_cast<uint32_t>((slot ^ T::swz(r)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_ptr)(&lds_qr[buf][0] + 1024 * c), 16,
                                               static_cast<int>(row_off + roff), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr)(&lds_dr[buf][0] + 1024 * c), 16,
                                               static_cast<int>(row_off + roff), 0, 0, 0);
    }
    if (wave_s == NW - 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rld, (lds_ptr)(&lds_ld[buf][0]), 16, 16 * ln, t * 256,
                                               0, 0);
  };

  // ---- one step: queries 32 t .. 32 t + 31 against this wave's keys
  const uint32_t a_base = static_cast<uint32_t>(l32) * T::ROW + ((hh ^ T::swz(l32)) << 4);
  // S and dP start from -lse_i / c_h and -D_i of their query rows (register
  // j holds query 8 (j/4) + 4 hh + j%4), so S = q.k - lse / c_h and dP = dO.v
  // - D.  The step reads them before the next step's DMA is issued: read
  // after it, the compiler makes the read wait for that DMA.
  auto start_values = [&](int buf, floatx16& s, floatx16& dp) __attribute__((always_inline)) {
    const float* ldb = &lds_ld[buf][4 * (fresh_lane() >> 5)];
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const float4 l2 = *reinterpret_cast<const float4*>(ldb + 8 * jg);
      const float4 dd = *reinterpret_cast<const float4*>(ldb + 32 + 8 * jg);
      s[4 * jg] = l2.x; s[4 * jg + 1] = l2.y; s[4 * jg + 2] = l2.z; s[4 * jg + 3] = l2.w;
      dp[4 * jg] = dd.x; dp[4 * jg + 1] = dd.y; dp[4 * jg + 2] = dd.z; dp[4 * jg + 3] = dd.w;
    }
  };
  auto step = [&](auto diag_c, int buf, int t, floatx16 s, floatx16 dp) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const char* qr = &lds_qr[buf][0];
    const char* dr = &lds_dr[buf][0];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = a_base ^ static_cast<uint32_t>(32 * ks);
      s = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(qr + off), kf[ks], s);
      dp = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(dr + off), vf[ks], dp);
    }
    // P and dS for this lane's key and its 16 queries
    uint32_t pk[8], dsk[8];
    const int qbase = t * kRows + 4 * hh;
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      float pj[4], dsj[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * jg + i;
        float p = fast_exp2(fmaf(s[j], alpha, bkey));
        if (DIAG && qbase + 8 * jg + i < my_key) p = 0.f;
        const float ds = p * dp[j];
        csum += ds;
        pj[i] = p;
        dsj[i] = ds;
      }
      pk[2 * jg] = pack_bf16(pj[0], pj[1]);
      pk[2 * jg + 1] = pack_bf16(pj[2], pj[3]);
      dsk[2 * jg] = pack_bf16(dsj[0], dsj[1]);
      dsk[2 * jg + 1] = pack_bf16(dsj[2], dsj[3]);
    }
    // dV += P^T dO, dK += dS^T Q: k-step ks2 takes registers 8 ks2 .. 8 ks2 + 7;
    // the dO and Q fragments are read transposed out of the row tiles
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const u32x4 pa = {pk[4 * ks2], pk[4 * ks2 + 1], pk[4 * ks2 + 2], pk[4 * ks2 + 3]};
      const u32x4 da = {dsk[4 * ks2], dsk[4 * ks2 + 1], dsk[4 * ks2 + 2], dsk[4 * ks2 + 3]};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[dt] = mfma_32x32x16(as_bf16x8(pa), tr_frag<D>(dr, ks2, 32 * dt, lane), dv[dt]);
        dk[dt] = mfma_32x32x16(as_bf16x8(da), tr_frag<D>(qr, ks2, 32 * dt, lane), dk[dt]);
      }
    }
  };

  // ---- main loop over this chunk's query tiles, one barrier per step
  dma(0, t_begin);
  for (int t = t_begin; t < t_stop; ++t) {
    const int buf = (t - t_begin) & 1;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA has landed
    __syncthreads();                 // ... and every other wave's; the other slot is free
    floatx16 s0, dp0;
    start_values(buf, s0, dp0);
    if (t + 1 < t_stop) dma(buf ^ 1, t + 1);
    // this wave's diagonal tile, formed here for the reason the DMA offsets are
    const int t_vis = kt * (kWgRows / kRows) + (wave_s * 64 + fresh_lane()) / 64;
    if (t == t_vis) step(std::true_type{}, buf, t, s0, dp0);
    else if (t > t_vis) step(std::false_type{}, buf, t, s0, dp0);
  }

  // ---- epilogue: fp32 partials of this head and chunk (rows = keys, columns = d)
  const size_t slot = static_cast<size_t>(ch) * Hq + head;
  float* dkh = dkp + slot * mp * D;
  float* dvh = dvp + slot * mp * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const size_t row = static_cast<size_t>(key0 + 8 * (j >> 2) + 4 * hh + (j & 3));
      dkh[row * D + 32 * dt + l32] = dk[dt][j] * c_h;
      dvh[row * D + 32 * dt + l32] = dv[dt][j];
    }
  }
  csum = add_halves(csum);
  if (hh == 0) colsum[slot * mp + my_key] = csum;
  // this chunk's share of the gain gradient: sum over the 128 keys of s_j colsum_j
  float gs = (hh == 0 && my_key < M) ? csum * key_score[my_key] : 0.f;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) gs += __shfl_xor(gs, o);
  if (lane == 0) lds_red[wave] = gs;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += lds_red[w];
    dgp[slot * n_kt + kt] = t;
  }
}

// ---------------------------------------------------------------------------
// bwd_dq
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void bwd_dq_body(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ tau, int M, int Hq, int Hkv,
    int n_t32, int n_t128, int mp, int clen, int nc, const float* __restrict__ ld,
    bf16* __restrict__ dq, float* __restrict__ dqp,
    float* __restrict__ qdot, int bid, char* lds_all) {
  using T = Bwd<D>;
  constexpr int KS = T::KS, DT = T::DT;
  constexpr int NW = kThreads / 64;
  constexpr int NJR = T::N_ROW_DMA / NW;
  static_assert(T::N_ROW_DMA % NW == 0, "row tiles split evenly over the waves");

  // all of the kernel's LDS is one object (as in the dK/dV kernel)
  auto* lds_kr = reinterpret_cast<char (*)[T::ROWS_TILE]>(lds_all);
  auto* lds_vr = reinterpret_cast<char (*)[T::ROWS_TILE]>(lds_all + 2 * T::ROWS_TILE);
  auto* lds_s = reinterpret_cast<float (*)[32]>(lds_all + 4 * T::ROWS_TILE);
  float* lds_red = reinterpret_cast<float*>(lds_all + 4 * T::ROWS_TILE + 2 * 32 * 4);

  int head, unit;
  head_unit(bid, Hq, head, unit);
  const int qt = n_t128 - 1 - unit / nc, ch = unit % nc;   // longest walks first
  const int u_end = q_walk(qt, M);
  const int u_begin = ch * clen;                 // this chunk's key steps
  if (u_begin >= u_end) return;                  // past the walk: no chunk here
  const int u_stop = min(u_begin + clen, u_end);
  const int kvh = head / (Hq / Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int q0 = qt * kWgRows + wave * kRows;
  const int my_q = q0 + l32;

  const uint32_t q_row = static_cast<uint32_t>(Hq) * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + static_cast<size_t>(head) * D, q_row * static_cast<uint32_t>(M));
  bf16x8 qf[KS], df[KS];
  {
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dout + static_cast<size_t>(head) * D, q_row * static_cast<uint32_t>(M));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = static_cast<uint32_t>(my_q) * q_row + (16 * s + 8 * hh) * 2;
      qf[s] = as_bf16x8(bload16(rq, off));
      df[s] = as_bf16x8(bload16(rd, off));
    }
  }
  const float c_h = 1.f / (sqrtf(static_cast<float>(D)) * tau[head]);
  const float alpha = kLog2e * c_h;
  const float gl = gain[head] * kLog2e;
  const float* ldt = ld + (static_cast<size_t>(head) * n_t32 + (q0 >> 5)) * 64;
  const float nlse2 = ldt[l32] * alpha, ndd = ldt[32 + l32];   // -lse (log2 units), -D

  floatx16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = zero16();

  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + static_cast<size_t>(kvh) * D, kv_row * static_cast<uint32_t>(M));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + static_cast<size_t>(kvh) * D, kv_row * static_cast<uint32_t>(M));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(key_score, static_cast<uint32_t>(M) * 4);
  const int lane16 = 16 * lane;
  uint32_t roff[NJR];   // as in bwd_dkdv: K and V rows share the stride
#pragma unroll
  for (int jj = 0; jj < NJR; ++jj) {
    const int byte = 1024 * (wave_s + NW * jj) + lane16;
    const int r = byte / T::ROW, slot = (byte % T::ROW) / 16;
    roff[jj] = static_cast<uint32_t>(r) * kv_row + static_cast<uint32_t>((slot ^ T::swz(r)) * 16);
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](int buf, int u) __attribute__((always_inline)) {
    const uint32_t row_off = static_cast<uint32_t>(u) * kRows * kv_row;
#pragma unroll
    for (int jj = 0; jj < NJR; ++jj) {
      const int c = wave_s + NW * jj;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(&lds_kr[buf][0] + 1024 * c), 16,
                                               static_cast<int>(row_off + roff[jj]), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(&lds_vr[buf][0] + 1024 * c), 16,
                                               static_cast<int>(row_off + roff[jj]), 0, 0, 0);
    }
    if (wave_s == NW - 1 && lane < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(&lds_s[buf][0]), 16, lane16, u * 128, 0, 0);
  };

  const uint32_t a_base = static_cast<uint32_t>(l32) * T::ROW + ((hh ^ T::swz(l32)) << 4);
  // The step's 16 key scores (register j: key 8 (j/4) + 4 hh + j%4), read
  // before the next step's DMA is issued: read after it, the compiler makes
  // the read wait for that DMA.
  auto key_scores = [&](int buf, float (&sk)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const float4 sv = *reinterpret_cast<const float4*>(&lds_s[buf][8 * jg + 4 * hh]);
      sk[4 * jg] = sv.x; sk[4 * jg + 1] = sv.y; sk[4 * jg + 2] = sv.z; sk[4 * jg + 3] = sv.w;
    }
  };
  auto step = [&](auto diag_c, int buf, int u, const float (&sk)[16]) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const char* kr = &lds_kr[buf][0];
    const char* vr = &lds_vr[buf][0];
    floatx16 st = zero16(), dpt = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = a_base ^ static_cast<uint32_t>(32 * ks);
      st = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(kr + off), qf[ks], st);
      dpt = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(vr + off), df[ks], dpt);
    }
    // dS^T for this lane's query and its 16 keys 8 (j/4) + 4 hh + j%4
    uint32_t dsk[8];
    const int kbase = u * kRows + 4 * hh;
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      float dsj[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * jg + i;
        float p = fast_exp2(fmaf(st[j], alpha, fmaf(sk[j], gl, nlse2)));
        if (DIAG && kbase + 8 * jg + i > my_q) p = 0.f;
        dsj[i] = p * (dpt[j] + ndd);
      }
      dsk[2 * jg] = pack_bf16(dsj[0], dsj[1]);
      dsk[2 * jg + 1] = pack_bf16(dsj[2], dsj[3]);
    }
    // dQ^T += K^T dS^T, the K^T fragments read transposed out of the K rows tile
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const u32x4 b = {dsk[4 * ks2], dsk[4 * ks2 + 1], dsk[4 * ks2 + 2], dsk[4 * ks2 + 3]};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = mfma_32x32x16(tr_frag<D>(kr, ks2, 32 * dt, lane), as_bf16x8(b), acc[dt]);
    }
  };

  // ---- this chunk's key tiles; this wave's diagonal tile is q0 / 32
  const int u_diag = q0 / kRows;
  dma(0, u_begin);
  for (int u = u_begin; u < u_stop; ++u) {
    const int buf = (u - u_begin) & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float sk[16];
    key_scores(buf, sk);
    if (u + 1 < u_stop) dma(buf ^ 1, u + 1);
    if (u == u_diag) step(std::true_type{}, buf, u, sk);
    else if (u < u_diag) step(std::false_type{}, buf, u, sk);
  }

  // ---- epilogue: dq = c_h (K^T dS^T)^T; lane = query, registers = dims
  // 32 dt + 8 (j/4) + 4 hh + j%4: bf16 dq, or this chunk's fp32 partial when
  // the walk is split.  Also q.dq for the temperature gradient.
  float qd = 0.f;
  if (my_q < M) {
    const size_t row = static_cast<size_t>(my_q) * Hq * D + static_cast<size_t>(head) * D;
    bf16* orow = dq + row;
    float* prow = dqp + static_cast<size_t>(ch) * mp * Hq * D + row;
    const bf16* qrow = q + row;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * dt + 8 * jj + 4 * hh;
        const uint2 qv = *reinterpret_cast<const uint2*>(qrow + d0);
        const float qx[4] = {__uint_as_float(qv.x << 16), __uint_as_float(qv.x & 0xFFFF0000u),
                             __uint_as_float(qv.y << 16), __uint_as_float(qv.y & 0xFFFF0000u)};
        float g[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g[r] = acc[dt][4 * jj + r] * c_h;
          qd = fmaf(qx[r], g[r], qd);
        }
        if (nc == 1) {
          const bf16 o4[4] = {static_cast<bf16>(g[0]), static_cast<bf16>(g[1]),
                              static_cast<bf16>(g[2]), static_cast<bf16>(g[3])};
          *reinterpret_cast<uint2*>(orow + d0) = __builtin_bit_cast(uint2, o4);
        } else {
          *reinterpret_cast<float4*>(prow + d0) = make_float4(g[0], g[1], g[2], g[3]);
        }
      }
    }
  }
  qd = add_halves(qd);
  if (hh == 1) qd = 0.f;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) qd += __shfl_xor(qd, o);
  if (lane == 0) lds_red[wave] = qd;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
    for (int w = 0; w < NW; ++w) s += lds_red[w];
    qdot[(static_cast<size_t>(ch) * Hq + head) * n_t128 + qt] = s;
  }
}

// One launch for both walks, which depend only on the pack pass: work-groups
// 0 .. n_dkdv - 1 take the dK/dV walks (longest first), the rest the dQ
// walks, so that the dQ work-groups start on the CUs the dK/dV walks leave
// instead of behind the whole dK/dV launch.  One LDS object, sized for the
// larger of the two.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_walks_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ tau, int M, int Hq, int Hkv,
    int n_t32, int n_t128, int mp, int kv_len, int kv_nc, int q_len, int q_nc,
    const float* __restrict__ ld, float* __restrict__ colsum, float* __restrict__ dkp,
    float* __restrict__ dvp, float* __restrict__ dgp, bf16* __restrict__ dq,
    float* __restrict__ dqp, float* __restrict__ qdot, int n_dkdv) {
  using T = Bwd<D>;
  constexpr int kDkdvLds = 4 * T::ROWS_TILE + 2 * 1024 + kThreads / 64 * 4;
  constexpr int kDqLds = 4 * T::ROWS_TILE + 2 * 32 * 4 + kThreads / 64 * 4;
  __shared__ __align__(16) char lds_all[kDkdvLds > kDqLds ? kDkdvLds : kDqLds];
  const int b = static_cast<int>(blockIdx.x);
  if (b < n_dkdv)
    bwd_dkdv_body<D>(q, k, v, dout, key_score, gain, tau, M, Hq, Hkv, n_t32, mp, kv_len, kv_nc, ld,
                     colsum, dkp, dvp, dgp, b, lds_all);
  else
    bwd_dq_body<D>(q, k, v, dout, key_score, gain, tau, M, Hq, Hkv, n_t32, n_t128, mp, q_len, q_nc,
                   ld, dq, dqp, qdot, b - n_dkdv, lds_all);
}

// ---------------------------------------------------------------------------
// Reductions (fixed order)
// ---------------------------------------------------------------------------
// dk, dv [key][kvh][d] = sum over the group's heads, then over the key block's
// chunks, of the fp32 partials (bf16 out); the threads of (key, KV head 0,
// dims 0..3) also form the score gradient ds_j = sum_h g_h sum_c colsum_chj.
template <int D>
__device__ __forceinline__ void reduce_dkdv_block(
    int blk, const float* __restrict__ dkp, const float* __restrict__ dvp,
    const float* __restrict__ colsum, const float* __restrict__ gain, int M, int Hq, int Hkv,
    int mp, int clen, int nc, bf16* __restrict__ dk, bf16* __restrict__ dv,
    float* __restrict__ dscore) {
  const int64_t e = static_cast<int64_t>(blk) * kThreads + threadIdx.x;  // one 4-dim group
  const int64_t per_row = static_cast<int64_t>(Hkv) * (D / 4);
  if (e >= static_cast<int64_t>(M) * per_row) return;
  const int64_t key = e / per_row;
  const int kvh = static_cast<int>((e % per_row) / (D / 4));
  const int d4 = static_cast<int>(e % (D / 4));
  const int G = Hq / Hkv;
  const int t_real = (M + kRows - 1) / kRows;
  const int nch = min(nc, kv_chunks(static_cast<int>(key / kWgRows), t_real, clen));
  float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    for (int c = 0; c < nch; ++c) {
      const size_t src = ((static_cast<size_t>(c) * Hq + kvh * G + g) * mp + key) * D + 4 * d4;
      const float4 x = *reinterpret_cast<const float4*>(dkp + src);
      const float4 y = *reinterpret_cast<const float4*>(dvp + src);
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
    }
  }
  const size_t dst = (static_cast<size_t>(key) * Hkv + kvh) * D + 4 * d4;
  const bf16 ka[4] = {static_cast<bf16>(a.x), static_cast<bf16>(a.y), static_cast<bf16>(a.z), static_cast<bf16>(a.w)};
  const bf16 va[4] = {static_cast<bf16>(b.x), static_cast<bf16>(b.y), static_cast<bf16>(b.z), static_cast<bf16>(b.w)};
  *reinterpret_cast<uint2*>(dk + dst) = __builtin_bit_cast(uint2, ka);
  *reinterpret_cast<uint2*>(dv + dst) = __builtin_bit_cast(uint2, va);
  if (kvh == 0 && d4 == 0) {
    float sc = 0.f;
    for (int h = 0; h < Hq; ++h) {
      float cs = 0.f;
      for (int c = 0; c < nch; ++c) cs += colsum[(static_cast<size_t>(c) * Hq + h) * mp + key];
      sc = fmaf(gain[h], cs, sc);
    }
    dscore[key] = sc;
  }
}

// dq [row][h][d] = sum over the query block's chunks of the fp32 partials
// (only launched when the dQ walks are split).
template <int D>
__device__ __forceinline__ void reduce_dq_block(int blk, const float* __restrict__ dqp, int M,
                                                int Hq, int mp, int clen, int nc,
                                                bf16* __restrict__ dq) {
  const int64_t e = static_cast<int64_t>(blk) * kThreads + threadIdx.x;
  const int64_t per_row = static_cast<int64_t>(Hq) * (D / 4);
  if (e >= static_cast<int64_t>(M) * per_row) return;
  const int64_t row = e / per_row;
  const int nch = min(nc, (q_walk(static_cast<int>(row / kWgRows), M) + clen - 1) / clen);
  float4 a = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    const float4 x = *reinterpret_cast<const float4*>(dqp + static_cast<size_t>(c) * mp * Hq * D + 4 * e);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
  }
  const bf16 o[4] = {static_cast<bf16>(a.x), static_cast<bf16>(a.y), static_cast<bf16>(a.z), static_cast<bf16>(a.w)};
  *reinterpret_cast<uint2*>(dq + 4 * e) = __builtin_bit_cast(uint2, o);
}

// One work-group per head: dg_h = sum over key blocks and their chunks of the
// work-groups' sum_j s_j colsum_j; dtau_h = -(1 / tau_h) sum of q.dq over
// query blocks and chunks.  Thread i takes blocks i, i + 256, ..., then a
// fixed tree (deterministic).
__device__ __forceinline__ void head_block(
    int h, const float* __restrict__ dgp, const float* __restrict__ qdot,
    const float* __restrict__ tau, int M, int Hq, int n_t128, int kv_len, int kv_nc, int q_len,
    int q_nc, float* __restrict__ dgain, float* __restrict__ dtau) {
  __shared__ float red_g[kThreads], red_t[kThreads];
  const int tid = threadIdx.x;
  const int t_real = (M + kRows - 1) / kRows;
  float g = 0.f, t = 0.f;
  for (int b = tid; b < n_t128; b += kThreads) {
    const int nkv = min(kv_nc, kv_chunks(b, t_real, kv_len));
    for (int c = 0; c < nkv; ++c) g += dgp[(static_cast<size_t>(c) * Hq + h) * n_t128 + b];
    const int nq = min(q_nc, (q_walk(b, M) + q_len - 1) / q_len);
    for (int c = 0; c < nq; ++c) t += qdot[(static_cast<size_t>(c) * Hq + h) * n_t128 + b];
  }
  red_g[tid] = g;
  red_t[tid] = t;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      red_g[tid] += red_g[tid + w];
      red_t[tid] += red_t[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    dgain[h] = red_g[0];
    dtau[h] = -red_t[0] / tau[h];
  }
}

// The launch after dQ: blocks [0, n_kv) reduce dK/dV (and form the score
// gradient), the next n_q reduce split dQ partials, the last Hq form the gain
// and temperature gradients: independent work, one launch.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(
    const float* __restrict__ dkp, const float* __restrict__ dvp,
    const float* __restrict__ colsum, const float* __restrict__ gain,
    const float* __restrict__ dqp, const float* __restrict__ dgp, const float* __restrict__ qdot,
    const float* __restrict__ tau, int M, int Hq, int Hkv, int mp, int n_t128, int kv_len,
    int kv_nc, int q_len, int q_nc, int n_kv, int n_q, bf16* __restrict__ dk,
    bf16* __restrict__ dv, bf16* __restrict__ dq, float* __restrict__ dscore,
    float* __restrict__ dgain, float* __restrict__ dtau) {
  const int b = blockIdx.x;   // block-uniform branches
  if (b < n_kv)
    reduce_dkdv_block<D>(b, dkp, dvp, colsum, gain, M, Hq, Hkv, mp, kv_len, kv_nc, dk, dv, dscore);
  else if (b < n_kv + n_q)
    reduce_dq_block<D>(b - n_kv, dqp, M, Hq, mp, q_len, q_nc, dq);
  else
    head_block(b - n_kv - n_q, dgp, qdot, tau, M, Hq, n_t128, kv_len, kv_nc, q_len, q_nc, dgain,
               dtau);
}

template <int D>
hipError_t launch_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, int M, int Hq,
                    int Hkv, const float* s, const float* g, const float* t, const float* out,
                    const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk,
                    uint16_t* dv, float* dscore, float* dgain, float* dtau, void* workspace,
                    hipStream_t stream) {
  const BwdPlan p = bwd_plan(M, Hq, Hkv, D);
  char* ws = static_cast<char*>(workspace);
  const bf16* bq = reinterpret_cast<const bf16*>(q);
  const bf16* bk = reinterpret_cast<const bf16*>(k);
  const bf16* bv = reinterpret_cast<const bf16*>(v);
  const bf16* bd = reinterpret_cast<const bf16*>(dout);
  const int n_t32 = static_cast<int>(p.n_t32), n_t128 = static_cast<int>(p.n_t128);
  const int mp = static_cast<int>(p.mp);
  float* ld = reinterpret_cast<float*>(ws + p.ld);
  float* colsum = reinterpret_cast<float*>(ws + p.colsum);
  float* dkp = reinterpret_cast<float*>(ws + p.dkp);
  float* dvp = reinterpret_cast<float*>(ws + p.dvp);
  float* dgp = reinterpret_cast<float*>(ws + p.dgp);
  float* qdot = reinterpret_cast<float*>(ws + p.qdot);
  float* dqp = reinterpret_cast<float*>(ws + p.dqp);
  hipLaunchKernelGGL((bwd_pack_kernel<D>), dim3(static_cast<unsigned>(Hq * n_t32)),
                     dim3(kThreads), 0, stream, out, lse, bd, t, M, Hq, n_t32, ld);
  const int n_dkdv = Hq * n_t128 * p.kv.nc, n_dq = Hq * n_t128 * p.q.nc;
  hipLaunchKernelGGL((bwd_walks_kernel<D>), dim3(static_cast<unsigned>(n_dkdv + n_dq)),
                     dim3(kThreads), 0, stream, bq, bk, bv, bd, s, g, t, M, Hq, Hkv, n_t32, n_t128,
                     mp, p.kv.len, p.kv.nc, p.q.len, p.q.nc, ld, colsum, dkp, dvp, dgp,
                     reinterpret_cast<bf16*>(dq), dqp, qdot, n_dkdv);
  const int64_t groups = static_cast<int64_t>(M) * Hkv * (D / 4);
  const int n_kv = static_cast<int>((groups + kThreads - 1) / kThreads);
  const int64_t qgroups = static_cast<int64_t>(M) * Hq * (D / 4);
  const int n_q = p.q.nc > 1 ? static_cast<int>((qgroups + kThreads - 1) / kThreads) : 0;
  hipLaunchKernelGGL((bwd_finish_kernel<D>), dim3(static_cast<unsigned>(n_kv + n_q + Hq)),
                     dim3(kThreads), 0, stream, dkp, dvp, colsum, g, dqp, dgp, qdot, t, M, Hq, Hkv,
                     mp, n_t128, p.kv.len, p.kv.nc, p.q.len, p.q.nc, n_kv, n_q,
                     reinterpret_cast<bf16*>(dk), reinterpret_cast<bf16*>(dv),
                     reinterpret_cast<bf16*>(dq), dscore, dgain, dtau);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t n, int n_q_heads, int n_kv_heads, int head_dim) {
  if (n <= 0) return 0;
  return bwd_plan(n, n_q_heads, n_kv_heads, head_dim).total;
}

hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n,
                           int n_q_heads, int n_kv_heads, int head_dim, const float* key_score,
                           const float* gain, const float* tau, const float* out,
                           const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk,
                           uint16_t* dv, float* dscore, float* dgain, float* dtau,
                           void* workspace, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int M = static_cast<int>(n);
  if (head_dim == 128)
    return launch_d<128>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out, lse, dout,
                         dq, dk, dv, dscore, dgain, dtau, workspace, stream);
  return launch_d<64>(q, k, v, M, n_q_heads, n_kv_heads, key_score, gain, tau, out, lse, dout, dq,
                      dk, dv, dscore, dgain, dtau, workspace, stream);
}

}  // namespace tg
