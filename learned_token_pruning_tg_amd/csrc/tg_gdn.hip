// Gated DeltaNet recurrence over the kept rows, for gfx950.
//
// The coverage pages (lucasainews.com TokenGate article, "성능 결과";
// miraibroadcast.com, "Resultados em modelos maiores"; heraldofai.com,
// "Vantaggi in velocità e memoria") report TokenGate on a hybrid model whose
// Gated DeltaNet layers sit between full-attention layers, and that it prunes
// those recurrent layers as well.  Above the gate such a layer runs its
// recurrence over the kept rows only, in original order.  The recurrence is
// the gated delta rule of Gated DeltaNet (Yang, Kautz, Hatamizadeh, ICLR 2025),
// per value head h with state S [dv, dk]:
//     S <- exp(g_t) S;   S <- S + beta_t (v_t - S k_t) k_t^T;   o_t = scale S q_t.
//
// Chunked form used here (chunks of C = 64 rows; within a chunk c_i is the
// cumulative log decay up to row i, Gam_i = exp(c_i), S the chunk's start
// state):
//   A_ij = beta_i exp(c_i - c_j) k_i.k_j (j < i),  T = (I + A)^-1,
//   W = T diag(beta Gam) K,  U' = T diag(beta) V
//   U    = U' - W S^T                           (the rows' written deltas)
//   O    = scale (diag(Gam) Q S^T + P U),  P_ij = exp(c_i - c_j) q_i.k_j (j <= i)
//   S    <- Gam_last S + U^T Kt,            Kt_j = exp(c_last - c_j) k_j
//
// Two roles of one kernel, gdn_fused_kernel, launched once per piece of
// about 2 sqrt(chunks) chunks (plus one): launch i runs the chain over piece
// i - 1 on work-groups 0 .. Hv - 1 (dispatched first, one CU each) beside the
// prep of piece i on the other work-groups, the state passing from piece to
// piece through the workspace.  The chain occupies Hv CUs; the prep of the
// next piece fills the rest instead of waiting for the whole chain.
// 1. prep: one 256-thread half work-group per (chunk, value head).
//    Forms K K^T and K Q^T on bf16 MFMA (exact products, fp32 sums), A and P
//    with their decays (P goes out straight from the accumulators), inverts
//    the unit lower-triangular I + A in fp32 by 16 x 16 blocks (diagonal
//    blocks by forward substitution, the blocks below by
//    T_IJ = -T_II sum_K A_IK T_KJ), and forms W and U' as bf16 MFMA products
//    of K and V with T's scaled columns split into bf16 high and low parts
//    (16 mantissa bits).  Every operand the chain needs leaves as fp16 MFMA
//    fragments: -W, U', scale P, Kt^T and the scaled queries
//    scale Gam_i q_i, then Gam_last.
// 2. chain: one work-group per value head walks the piece's chunks in order, a
//    wave per 32 value rows (the rows of S evolve independently), the head's
//    per-chunk operands DMAed once into a two-stage LDS ring for the four
//    state waves by four waves of their own.  Each state wave's fp32 slice
//    S^T [128 dk x 32 dv] lives in MFMA accumulators; per chunk:
//    U = U' - W S^T and O = (scale Gam Q) S^T (16 + 16 fp16 MFMAs),
//    O += (scale P) U (8), S^T = Gam_last S^T + Kt^T U (16).  The state's
//    accumulator layout is used directly as the B operand:
//    the contraction index k of every product (dk for W S^T and Q S^T, the
//    chunk row for P U and Kt^T U) is permuted within each 16-wide k-step to
//    the order in which the accumulators hold it, and the prep pass writes
//    the A operands in that same order.  Rows of the value dimension evolve
//    independently, which is what lets the chain split over 32-row blocks.
//
// Numerics: bf16 inputs; decays, the inverse, the state and every sum in
// fp32 (T's scaled entries carried to 16 mantissa bits into W and U');
// the MFMA operands (W, U', P, Kt, q and the fp32 state and deltas) rounded
// to fp16 (11-bit mantissa; q and k are unit vectors, values of v above 65504
// would saturate); output rounded to bf16.
#include <algorithm>
#include <cmath>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int kD = 128;      // dk = dv
constexpr int kC = 64;       // chunk rows
constexpr int kBV = 32;      // value rows per chain

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// Per (chunk, value head) workspace record.
constexpr int kOffW = 0;                        // -W fragments: [s 8][r 2][lane][8 fp16]
constexpr int kOffU = kOffW + kC * kD * 2;      // U' accumulator images: [b 4][r 2][lane][16 fp16]
constexpr int kOffP = kOffU + kC * kD * 2;      // P fragments: [s 4][r 2][lane][8 fp16]
constexpr int kOffK = kOffP + kC * kC * 2;      // Kt^T fragments: [s 4][t 4][lane][8 fp16]
constexpr int kOffQ = kOffK + kD * kC * 2;      // scaled q fragments: [s 8][r 2][lane][8 fp16]
constexpr int kOffG = kOffQ + kC * kD * 2;      // Gam_last (fp32), then padding to 256 B
constexpr int kRec = kOffG + 256;

// Index held by (k-step s, lane half hh, element e) of a fragment: the order
// of the rows an MFMA accumulator holds in its registers 8 (s % 2) .. + 7.
__device__ __forceinline__ int kperm(int s, int hh, int e) {
  return 16 * s + 8 * (e >> 2) + 4 * hh + (e & 3);
}
// Row (within a 32-row tile) of accumulator register j in lane half hh.
__device__ __forceinline__ int crow(int j, int hh) { return 8 * (j >> 2) + 4 * hh + (j & 3); }

__device__ __forceinline__ floatx16 mfma_f16(f16x8 a, f16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Row r of a 64 x 128 bf16 tile in LDS: 16-byte chunk cc at slot cc ^ (r & 15)
// (16 consecutive rows read the same chunk from 16 different slots).
__device__ __forceinline__ int tile_off(int r, int cc) { return r * 256 + ((cc ^ (r & 15)) << 4); }
__device__ __forceinline__ float tile_at(const char* t, int r, int col) {
  return bf2f(*reinterpret_cast<const uint16_t*>(t + tile_off(r, col >> 3) + 2 * (col & 7)));
}

// ---------------------------------------------------------------------------
// gdn_prep
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 to_f16x8(const floatx16& a, int half) {
  f16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<_Float16>(a[8 * half + e]);
  return x;
}

// MFMA fragment with a 64 x 128 bf16 tile's rows as k and its columns as the
// 32 lanes of m (or n), read transposed out of the swizzled row tile by two
// ds_read_b64_tr_b16: within each 16-lane group that instruction gives lane
// 4 a + c element c of the 8-byte rows that lanes a, a + 4, a + 8, a + 12
// address.  Lane j (of 16) addresses row 16 g + 8 q + 4 hh + j / 4 at columns
// n0 + 16 ((lane / 16) % 2) + 4 (j % 4), so element e of lane l's fragment is
// row kperm(g, hh, e) at column n0 + l % 32.
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int g, int n0, int lane) {
  const int j = lane & 15, hh = lane >> 5;
  const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  v4i16 x[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 16 * g + 8 * q + 4 * hh + (j >> 2);
    const char* a = tile + tile_off(r, col >> 3) + (col & 7) * 2;
    x[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a));
  }
  const v8i16 y = __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, y);
}

// A 64 x 64 bf16 matrix M[i][j] stored for fragment reads along j: row i
// (128 bytes) holds, in 16-byte piece q = 2 g + hh, the elements
// j = kperm(g, hh, 0..7); piece q sits at slot q ^ ((i / 2) % 8), so the 16
// rows one read pass serves hit 16 distinct bank groups.
__device__ __forceinline__ int tmat_off(int i, int q) { return i * 128 + ((q ^ ((i >> 1) & 7)) << 4); }

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<bf16>(x));
}

// LDS of one prep item: the K, Q and V tiles (48 KiB), A (16 KiB) and the
// per-row decays and write strengths (1 KiB)
constexpr int kPrepLds = 3 * kC * kD * 2 + kC * kC * 4 + 4 * kC * 4;

// The prep of one (chunk c, value head h) on 256 threads (tid 0..255) with
// kPrepLds bytes of LDS at lmem.  Contains work-group barriers: every thread
// of the work-group calls it the same way.
__device__ __forceinline__ void gdn_prep_item(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, int n, int Hk, int Hv,
    float scale, char* __restrict__ rec_base, int c, int h, int tid, char* lmem) {
  // LDS: the K, Q and V tiles (48 KiB) and A (16 KiB).  Once P and the
  // scaled q fragments are out, the Q tile holds T = (I + A)^-1 (fp32), then
  // the bf16 hi/lo parts of T diag(beta); once T is formed, A's space holds
  // those of -T diag(beta Gam).
  char* const lds_tiles = lmem;
  float (*const lds_a)[kC] = reinterpret_cast<float (*)[kC]>(lmem + 3 * kC * kD * 2);
  float* const lds_c = reinterpret_cast<float*>(lmem + 3 * kC * kD * 2 + kC * kC * 4);
  float* const lds_b = lds_c + kC;
  float* const lds_gam = lds_c + 2 * kC;
  float* const lds_fk = lds_c + 3 * kC;
  char* const lds_k = lds_tiles;
  char* const lds_q = lds_tiles + kC * kD * 2;
  char* const lds_v = lds_tiles + 2 * kC * kD * 2;
  float (*const lds_t)[kC] = reinterpret_cast<float (*)[kC]>(lds_q);
  char* const tv_hi = lds_q;                       // T diag(beta), bf16 hi / lo
  char* const tv_lo = lds_q + kC * kC * 2;
  char* const tk_hi = reinterpret_cast<char*>(&lds_a[0][0]);   // -T diag(beta Gam)
  char* const tk_lo = tk_hi + kC * kC * 2;

  const int kh = h / (Hv / Hk);
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, m = lane & 31;
  const int row0 = c * kC;
  char* rec = rec_base + (static_cast<size_t>(c) * Hv + h) * kRec;

  // K, Q and V rows of the chunk (rows past n read as zero), every load
  // issued before the first store
  {
    u32x4 kv[4], qv[4], vv[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = tid + 256 * p;
      const int r = i >> 4, cc = i & 15;
      kv[p] = qv[p] = vv[p] = zero_u32x4();
      if (row0 + r < n) {
        const size_t off = (static_cast<size_t>(row0 + r) * Hk + kh) * kD + 8 * cc;
        kv[p] = ld16(k + off);
        qv[p] = ld16(q + off);
        vv[p] = ld16(v + (static_cast<size_t>(row0 + r) * Hv + h) * kD + 8 * cc);
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = tid + 256 * p;
      const int r = i >> 4, cc = i & 15;
      st16(lds_k + tile_off(r, cc), kv[p]);
      st16(lds_q + tile_off(r, cc), qv[p]);
      st16(lds_v + tile_off(r, cc), vv[p]);
    }
  }
  // cumulative log decay c_i (inclusive, fixed order), beta, exp(c_i)
  if (wave == 0) {
    float gv = 0.f, bv = 0.f;
    if (row0 + lane < n) {
      gv = g[static_cast<size_t>(row0 + lane) * Hv + h];
      bv = beta[static_cast<size_t>(row0 + lane) * Hv + h];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(gv, o);
      if (lane >= o) gv += t;
    }
    lds_c[lane] = gv;
    lds_b[lane] = bv;
    lds_gam[lane] = __expf(gv);
    lds_fk[lane] = __expf(__shfl(gv, kC - 1) - gv);   // exp(c_last - c_j)
    if (lane == kC - 1) reinterpret_cast<float*>(rec + kOffG)[0] = __expf(gv);
  }
  __syncthreads();

  // K K^T -> A (lower-triangle 32 x 32 tiles (0,0), (1,0), (1,1): lane = j,
  // registers = i) and K Q^T -> scale P^T (tiles with j <= i: lane = i,
  // registers = j, which is the P fragment order: k-step s = 2 J + register
  // half), written straight out as fragments.
  for (int ti = wave; ti < 6; ti += 4) {
    const bool is_p = ti >= 3;
    const int I = (ti % 3) == 0 ? 0 : 1, J = (ti % 3) == 2 ? 1 : 0;   // rows i of tile I, j of J
    floatx16 acc = zero16();
    if (!is_p) {
      const int ra = 32 * I + m, rb = 32 * J + m;
#pragma unroll
      for (int s = 0; s < kD / 16; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + tile_off(ra, 2 * s + hh));
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(lds_k + tile_off(rb, 2 * s + hh));
        acc = mfma_32x32x16(a, bb, acc);
      }
      const int j = rb;
      const float cj = lds_c[j];
#pragma unroll
      for (int jr = 0; jr < 16; ++jr) {
        const int i = 32 * I + crow(jr, hh);
        lds_a[i][j] = j < i ? lds_b[i] * __expf(lds_c[i] - cj) * acc[jr] : 0.f;
      }
    } else {
      const int rj = 32 * J + m, ri = 32 * I + m;
#pragma unroll
      for (int s = 0; s < kD / 16; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + tile_off(rj, 2 * s + hh));
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(lds_q + tile_off(ri, 2 * s + hh));
        acc = mfma_32x32x16(a, bb, acc);
      }
      const int i = ri;
      const float ci = lds_c[i];
      f16x8 x[2];
#pragma unroll
      for (int jr = 0; jr < 16; ++jr) {
        const int j = 32 * J + crow(jr, hh);
        x[jr >> 3][jr & 7] = static_cast<_Float16>(j <= i ? scale * __expf(ci - lds_c[j]) * acc[jr] : 0.f);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        *reinterpret_cast<f16x8*>(rec + kOffP + ((2 * J + half) * 2 + I) * 1024 + lane * 16) = x[half];
    }
  }
  // the tile with j > i everywhere: zero P fragments (k-steps 2, 3 of row tile 0)
  if (wave == 3) {
    const f16x8 z = {};
#pragma unroll
    for (int half = 0; half < 2; ++half)
      *reinterpret_cast<f16x8*>(rec + kOffP + ((2 + half) * 2 + 0) * 1024 + lane * 16) = z;
  }

  // scaled q fragments: scale * Gam_i q_i, A operand [row][dk] (the rows' own
  // decay from the chunk start and the read-out scale, folded in here).
  // Elements 0-3 and 4-7 of a lane are dk 16 s + 4 hh .. + 3 and 8 further:
  // 8-byte reads of chunks 2 s and 2 s + 1 of the row.
  for (int u = tid; u < 8 * 2 * 64; u += 256) {
    const int ln = u & 63, r = (u >> 6) & 1, s = u >> 7;
    const int row = 32 * r + (ln & 31), h2 = ln >> 5;
    const float f = scale * lds_gam[row];
    const uint2 lo = *reinterpret_cast<const uint2*>(lds_q + tile_off(row, 2 * s) + 8 * h2);
    const uint2 hi = *reinterpret_cast<const uint2*>(lds_q + tile_off(row, 2 * s + 1) + 8 * h2);
    const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
    f16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      x[e] = static_cast<_Float16>(f * bf2f(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)))));
    *reinterpret_cast<f16x8*>(rec + kOffQ + static_cast<size_t>(u) * 16) = x;
  }
  // Kt^T fragments: exp(c_last - c_j) k_j, A operand [dk][row]: the transposed
  // read of K's tile, element e of lane l being row kperm(s, hh, e), dk 32 t + l % 32
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = wave;
    const bf16x8 kf = tr_frag(lds_k, s, 32 * t, lane);
    f16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      x[e] = static_cast<_Float16>(lds_fk[kperm(s, hh, e)] * static_cast<float>(kf[e]));
    *reinterpret_cast<f16x8*>(rec + kOffK + static_cast<size_t>((s * 4 + t) * 64 + lane) * 16) = x;
  }
  __syncthreads();   // A complete; the Q tile is free for T

  // T = (I + A)^-1, unit lower triangular, fp32, in 16 x 16 blocks.
  // Diagonal blocks by forward substitution (wave 0: lane = block * 16 +
  // column); the blocks above the diagonal are zeroed by the other waves.
  if (wave == 0) {
    const int I = lane >> 4, cl = lane & 15, b0 = 16 * I;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = r == cl ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < r; ++jj) acc = __builtin_fmaf(lds_a[b0 + r][b0 + jj], t[jj], acc);
      if (r > cl) t[r] = -acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) lds_t[b0 + r][b0 + cl] = t[r];
  } else {
    // blocks (I, J) with J > I: 6 blocks of 256 zeros, 8 per thread
    const int u0 = (tid - 64) * 8;                 // 0 .. 1535 + 7
    for (int u = u0; u < u0 + 8; ++u) {
      const int blk = u >> 8, e = u & 255;
      const int I = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
      const int J = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      lds_t[16 * I + (e >> 4)][16 * J + (e & 15)] = 0.f;
    }
  }
  __syncthreads();
  // Block rows 1..3: wave w forms T_IJ, J = w < I:
  //   X = sum_{K=J}^{I-1} A_IK T_KJ,  T_IJ = -T_II X.
  // Lane: row r = lane / 4 of the block, columns 4 (lane % 4) .. + 3.  X goes
  // through T_IJ's own slot (a wave's LDS accesses stay in order).
  for (int I = 1; I < 4; ++I) {
    if (wave < I) {
      const int J = wave;
      const int r = lane >> 2, c4 = 4 * (lane & 3);
      float4 x = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int mm = 0; mm < 16; ++mm) {
          const float a = lds_a[16 * I + r][16 * K + mm];
          const float4 tk = *reinterpret_cast<const float4*>(&lds_t[16 * K + mm][16 * J + c4]);
          x.x = __builtin_fmaf(a, tk.x, x.x); x.y = __builtin_fmaf(a, tk.y, x.y);
          x.z = __builtin_fmaf(a, tk.z, x.z); x.w = __builtin_fmaf(a, tk.w, x.w);
        }
      }
      *reinterpret_cast<float4*>(&lds_t[16 * I + r][16 * J + c4]) = x;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) {
        const float tii = lds_t[16 * I + r][16 * I + mm];
        const float4 xm = *reinterpret_cast<const float4*>(&lds_t[16 * I + mm][16 * J + c4]);
        y.x = __builtin_fmaf(-tii, xm.x, y.x); y.y = __builtin_fmaf(-tii, xm.y, y.y);
        y.z = __builtin_fmaf(-tii, xm.z, y.z); y.w = __builtin_fmaf(-tii, xm.w, y.w);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      *reinterpret_cast<float4*>(&lds_t[16 * I + r][16 * J + c4]) = y;
    }
    __syncthreads();
  }

  // T diag(beta) (for U') and -T diag(beta Gam) (for W) as bf16 hi + lo
  // parts (hi + lo carries 16 mantissa bits), stored along j in fragment
  // order.  Thread: row i = tid / 4, k-step block gj = tid % 4 (j = 16 gj ..).
  {
    const int i = tid >> 2, gj = tid & 3;
    float tr[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = *reinterpret_cast<const float4*>(&lds_t[i][16 * gj + 4 * q4]);
      tr[4 * q4] = x.x; tr[4 * q4 + 1] = x.y; tr[4 * q4 + 2] = x.z; tr[4 * q4 + 3] = x.w;
    }
    __syncthreads();   // all of T read: its space takes the bf16 parts
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 vh, vl, kh4, kl4;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t pvh = 0, pvl = 0, pkh = 0, pkl = 0;
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const int e = 2 * e2 + w2;
          const int jl = 8 * (e >> 2) + 4 * h2 + (e & 3);      // j - 16 gj = kperm(gj, h2, e) - 16 gj
          const int j = 16 * gj + jl;
          const float tvv = tr[jl] * lds_b[j];
          const float tkv = -tr[jl] * lds_b[j] * lds_gam[j];
          const uint16_t a = bf16_rne(tvv), bb = bf16_rne(tvv - __uint_as_float(static_cast<uint32_t>(a) << 16));
          const uint16_t cc = bf16_rne(tkv), dd = bf16_rne(tkv - __uint_as_float(static_cast<uint32_t>(cc) << 16));
          pvh |= static_cast<uint32_t>(a) << (16 * w2);
          pvl |= static_cast<uint32_t>(bb) << (16 * w2);
          pkh |= static_cast<uint32_t>(cc) << (16 * w2);
          pkl |= static_cast<uint32_t>(dd) << (16 * w2);
        }
        vh[e2] = pvh; vl[e2] = pvl; kh4[e2] = pkh; kl4[e2] = pkl;
      }
      const int off = tmat_off(i, 2 * gj + h2);
      st16(tv_hi + off, vh);
      st16(tv_lo + off, vl);
      st16(tk_hi + off, kh4);
      st16(tk_lo + off, kl4);
    }
  }
  __syncthreads();

  // -W = (-T diag(beta Gam)) K and U' = (T diag(beta)) V on bf16 MFMA, hi and
  // lo parts of T each a product.  Wave w: the W^T tiles of dk 32 w .. (rows
  // of the chunk as n: their accumulators are the -W fragments of k-steps
  // 2 w, 2 w + 1) and the U' tiles of value rows 32 w .. (accumulator images).
  {
    const int t = wave;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      floatx16 acc = zero16();
      const int i = 32 * r + m;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const bf16x8 a = tr_frag(lds_k, gg, 32 * t, lane);
        const int off = tmat_off(i, 2 * gg + hh);
        acc = mfma_32x32x16(a, *reinterpret_cast<const bf16x8*>(tk_hi + off), acc);
        acc = mfma_32x32x16(a, *reinterpret_cast<const bf16x8*>(tk_lo + off), acc);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        *reinterpret_cast<f16x8*>(rec + kOffW + ((2 * t + half) * 2 + r) * 1024 + lane * 16) =
            to_f16x8(acc, half);
    }
    const int bv = wave;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      floatx16 acc = zero16();
      const int i = 32 * r + m;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const bf16x8 bb = tr_frag(lds_v, gg, kBV * bv, lane);
        const int off = tmat_off(i, 2 * gg + hh);
        acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(tv_hi + off), bb, acc);
        acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(tv_lo + off), bb, acc);
      }
      f16x8* dst = reinterpret_cast<f16x8*>(rec + kOffU + ((bv * 2 + r) * 64 + lane) * 32);
      dst[0] = to_f16x8(acc, 0);
      dst[1] = to_f16x8(acc, 1);
    }
  }
}

// ---------------------------------------------------------------------------
// gdn_state
// ---------------------------------------------------------------------------

// One work-group of eight waves per value head.  Waves 0-3 carry the state:
// wave b the slice of value rows 32 b .. 32 b + 31.  Waves 4-7 only move each
// chunk's operand record (the -W, U', P, Kt^T and scaled q fragments and
// Gam_last, as the prep pass laid them out) into a two-stage LDS ring, once
// for the four state waves, the next chunk's DMA in flight during this chunk;
// one barrier per chunk for all eight.  The DMA (73 pieces of 1 KiB per
// chunk) costs its issuing waves time in proportion to their share of the
// pieces, so it runs on waves of its own, one beside each state wave on its
// SIMD (the kernel's 223 registers leave room for two waves per SIMD).
constexpr int kRecLds = (kRec + 1023) / 1024 * 1024;   // whole 1 KiB DMA pieces
constexpr int kStage = kRecLds;
constexpr int kPieces = kRecLds / 1024;
constexpr int kPiecesPerWave = (kPieces + 3) / 4;       // per DMA wave

// s_waitcnt immediate (gfx9 encoding) that waits until at most `vm` vector
// memory operations of this wave are outstanding and leaves the other
// counters alone.
constexpr int vm_wait(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

// The chain of value head h over chunks c0 .. c1 - 1 on 512 threads with
// 2 kStage bytes of LDS at lmem (the caller's single LDS object: with
// several, the compiler would make each read of the ring wait for all DMA in
// flight into it, the next chunk's included; the explicit waits below order
// the ring).  Stage (c - c0) & 1 holds chunk c.
__device__ __forceinline__ void gdn_chain_head(const char* __restrict__ rec_base, int n, int Hv,
                                               int h, int c0, int c1,
                                               const float* __restrict__ s_init,
                                               float* __restrict__ s_final,
                                               bf16* __restrict__ out, char* lmem) {
  auto* lds = reinterpret_cast<char (*)[kStage]>(lmem);
  const int lane = threadIdx.x & 63;
  const int b = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // provably wave-uniform
  const int m = lane & 31, hh = lane >> 5;
  const int dv = kBV * b + m;   // this lane's value row

  // DMA of chunk c into stage st by DMA wave b: pieces b - 4, b, b + 4, ...
  // of 1 KiB (lane i moves the 16 bytes at 16 i of its piece); bytes past the
  // record read as zeros.  The whole offset is per lane, the LDS address
  // wave-uniform.
  auto dma = [&](int st, int c) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rr =
        make_rsrc(rec_base + (static_cast<size_t>(c) * Hv + h) * kRec, kRec);
#pragma unroll
    for (int i = 0; i < kPiecesPerWave; ++i) {
      const int j = (b & 3) + 4 * i;
      if (j < kPieces)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rr, (__attribute__((address_space(3))) void*)(&lds[st][0] + 1024 * j), 16,
            16 * lane + 1024 * j, 0, 0, 0);
    }
  };

  // output rows of this head: byte offset row * row_bytes + (4 hh row part) +
  // dv * 2; the range ends at row n
  const uint32_t row_bytes = static_cast<uint32_t>(Hv) * kD * 2;   // n * row_bytes < 2^31
  const __amdgpu_buffer_rsrc_t rout =
      make_rsrc(reinterpret_cast<const char*>(out) + static_cast<size_t>(h) * kD * 2,
                static_cast<uint32_t>(n) * row_bytes - static_cast<uint32_t>(h) * kD * 2);
  const uint32_t lane_off = static_cast<uint32_t>(4 * hh) * row_bytes + 2u * dv;

  // A DMA wave waits for its own pieces of chunk c before the barrier at the
  // top of chunk c; the barrier then also means every state wave is done with
  // chunk c - 1, whose stage the next DMA refills.  A plain barrier: a
  // workgroup fence would also wait for the state waves' output stores; the
  // empty asm keeps the compiler from moving LDS accesses across it.
  if (b >= 4) {   // DMA waves: the ring's DMA only, one barrier per chunk like the others
    if (c0 < c1) dma(0, c0);
    for (int c = c0; c < c1; ++c) {
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (c + 1 < c1) dma((c + 1 - c0) & 1, c + 1);
    }
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    return;
  }
  // S^T slice of a state wave (value rows dv < 128; the DMA waves, whose dv
  // would run past the head, have left): tile t = dk rows 32 t .., register
  // jr = dk row 32 t + crow(jr, hh)
  floatx16 st[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int jr = 0; jr < 16; ++jr)
      st[t][jr] = s_init != nullptr
                      ? s_init[(static_cast<size_t>(h) * kD + dv) * kD + 32 * t + crow(jr, hh)]
                      : 0.f;
  }
  for (int c = c0; c < c1; ++c) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* rec = &lds[(c - c0) & 1][0];
    auto frag = [&](const char* base, int off) __attribute__((always_inline)) {
      return *reinterpret_cast<const f16x8*>(base + off + lane * 16);
    };
    // B operand of the state: k-step s = registers 8 (s % 2) .. + 7 of tile s / 2
    f16x8 bs[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) bs[s] = to_f16x8(st[s >> 1], s & 1);

    // U = U' - W S^T and O = Q S^T, the fragments of k-step s + 1 read while
    // k-step s multiplies
    floatx16 u[2], o[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const f16x8* src = reinterpret_cast<const f16x8*>(rec + kOffU + ((b * 2 + r) * 64 + lane) * 32);
      const f16x8 u0 = src[0], u1 = src[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u[r][e] = static_cast<float>(u0[e]);
        u[r][8 + e] = static_cast<float>(u1[e]);
      }
      o[r] = zero16();
    }
    f16x8 wf[2][2], qf[2][2];
    auto read_wq = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        wf[slot][r] = frag(rec, kOffW + (s * 2 + r) * 1024);
        qf[slot][r] = frag(rec, kOffQ + (s * 2 + r) * 1024);
      }
    };
    // the state's decay over the chunk, Gam_last S^T, applied while the U and
    // O products run (the fp16 copies bs above are of the undecayed state)
    const float gl = *reinterpret_cast<const float*>(rec + kOffG);
    read_wq(0, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) read_wq(s + 1, (s + 1) & 1);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        u[r] = mfma_f16(wf[s & 1][r], bs[s], u[r]);
        o[r] = mfma_f16(qf[s & 1][r], bs[s], o[r]);
      }
#pragma unroll
      for (int jr = 0; jr < 8; ++jr) st[s >> 1][8 * (s & 1) + jr] *= gl;
      __builtin_amdgcn_sched_barrier(0);
    }
    f16x8 bu[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) bu[s] = to_f16x8(u[s >> 1], s & 1);
    // O += P U
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int r = 0; r < 2; ++r) o[r] = mfma_f16(frag(rec, kOffP + (s * 2 + r) * 1024), bu[s], o[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // S^T = Gam_last S^T + Kt^T U
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int s = 0; s < 4; ++s) st[t] = mfma_f16(frag(rec, kOffK + (s * 4 + t) * 1024), bu[s], st[t]);
    }
    // outputs: lane (value row dv, half hh), register jr = row 32 r + crow(jr, hh);
    // the whole byte offset is in the per-lane offset, so rows past n fall
    // outside the buffer's range check and are dropped
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int jr = 0; jr < 16; ++jr) {
        const uint32_t row_u = static_cast<uint32_t>(c * kC + 32 * r + 8 * (jr >> 2) + (jr & 3));
        const bf16 x = static_cast<bf16>(o[r][jr]);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, x), rout,
                                              static_cast<int>(lane_off + row_u * row_bytes), 0, 0);
      }
    }
  }
  if (s_final != nullptr) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int jr = 0; jr < 16; ++jr)
        s_final[(static_cast<size_t>(h) * kD + dv) * kD + 32 * t + crow(jr, hh)] = st[t][jr];
    }
  }
}

// One launch of the layer: work-groups 0 .. n_chain - 1 run the chain of
// their value head over chunks c0 .. c1 - 1 (their prep done by an earlier
// launch); the others run the prep of items p0 Hv .. (chunk p0 + item / Hv,
// value head item % Hv), two per work-group on its two 256-thread halves
// (an odd last item is done by both halves, which write the same bytes).
struct GdnLaunch {
  const bf16* q; const bf16* k; const bf16* v; const float* g; const float* beta;
  int n, Hk, Hv;
  float scale;
  char* rec;
  bf16* out;
  int n_chain, c0, c1;            // chain work-groups (0 or Hv) and their chunks
  const float* s_init;
  float* s_final;
  int p0, n_items;                // first prep chunk and (chunk, value head) items
};

constexpr int kFusedLds = 2 * kStage > 2 * kPrepLds ? 2 * kStage : 2 * kPrepLds;

__global__ __launch_bounds__(512) void gdn_fused_kernel(GdnLaunch a) {
  __shared__ __align__(16) char lds_all[kFusedLds];
  if (static_cast<int>(blockIdx.x) < a.n_chain) {
    gdn_chain_head(a.rec, a.n, a.Hv, blockIdx.x, a.c0, a.c1, a.s_init, a.s_final, a.out, lds_all);
    return;
  }
  const int half = threadIdx.x >> 8;
  int item = 2 * (static_cast<int>(blockIdx.x) - a.n_chain) + half;
  if (item >= a.n_items) item = a.n_items - 1;
  gdn_prep_item(a.q, a.k, a.v, a.g, a.beta, a.n, a.Hk, a.Hv, a.scale, a.rec, a.p0 + item / a.Hv,
                item % a.Hv, threadIdx.x & 255, lds_all + half * kPrepLds);
}

}  // namespace

size_t gdn_workspace_bytes(int64_t n, int n_qk_heads, int n_v_heads) {
  if (n <= 0) return 0;
  const size_t nc = static_cast<size_t>((n + kC - 1) / kC);
  (void)n_qk_heads;
  // the records, then the state handed from one piece of the chain to the next
  return nc * static_cast<size_t>(n_v_heads) * kRec +
         static_cast<size_t>(n_v_heads) * kD * kD * sizeof(float);
}

hipError_t launch_gdn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                          const float* beta, int64_t n, int n_qk_heads, int n_v_heads, float scale,
                          const float* initial_state, float* final_state, uint16_t* out,
                          void* workspace, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int nc = static_cast<int>((n + kC - 1) / kC);
  char* rec = static_cast<char*>(workspace);
  float* state = reinterpret_cast<float*>(rec + static_cast<size_t>(nc) * n_v_heads * kRec);
  const int ni = static_cast<int>(n);
  // Pieces of pc chunks: launch i runs the chain over piece i - 1 (work-groups
  // 0 .. Hv - 1, dispatched first, one CU each) beside the prep of piece i on
  // the other CUs.  pc ~ 2 sqrt(nc) balances the extra launches against the
  // first piece's prep, which nothing overlaps.
  int pc = static_cast<int>(2.0 * std::sqrt(static_cast<double>(nc)) + 0.5);
  pc = std::max(8, std::min(pc, nc));
  const int pieces = (nc + pc - 1) / pc;
  for (int i = 0; i <= pieces; ++i) {
    GdnLaunch a{};
    a.q = reinterpret_cast<const bf16*>(q); a.k = reinterpret_cast<const bf16*>(k);
    a.v = reinterpret_cast<const bf16*>(v); a.g = g; a.beta = beta;
    a.n = ni; a.Hk = n_qk_heads; a.Hv = n_v_heads; a.scale = scale; a.rec = rec;
    a.out = reinterpret_cast<bf16*>(out);
    if (i > 0) {   // the chain over piece i - 1
      a.n_chain = n_v_heads;
      a.c0 = (i - 1) * pc;
      a.c1 = std::min(nc, i * pc);
      a.s_init = i == 1 ? initial_state : state;
      a.s_final = i == pieces ? final_state : state;
    }
    if (i < pieces) {   // the prep of piece i
      a.p0 = i * pc;
      a.n_items = (std::min(nc, (i + 1) * pc) - a.p0) * n_v_heads;
    }
    const unsigned grid = static_cast<unsigned>(a.n_chain + (a.n_items + 1) / 2);
    hipLaunchKernelGGL(gdn_fused_kernel, dim3(grid), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tg
