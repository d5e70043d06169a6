// Device-side helpers shared by the gfx950 kernels: vector types, the bf16
// MFMA wrapper and 16-byte memory moves.
//
// MFMA v_mfma_f32_32x32x16_bf16 register layout used throughout (wave64):
//   A (32 x 16): lane l supplies row (l % 32), eight k values of lane half
//                (l / 32);
//   B (16 x 32): lane l supplies column (l % 32), the same eight k values;
//   C (32 x 32): lane l, register j holds row 8*(j/4) + 4*(l/32) + (j%4),
//                column (l % 32).
// Only the C layout is load-bearing: A and B are always filled with the same
// logical k at the same (lane half, register), so the hardware's internal k
// order cannot change a product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma_32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Raw buffer descriptor (gfx9 layout: stride 0, range check on byte offset).
// Every field goes through readfirstlane so the descriptor is provably
// wave-uniform and lives in SGPRs; a descriptor the compiler cannot prove
// uniform makes it wrap each buffer load in a per-lane "waterfall" loop.
// Loads at offsets >= `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0), static_cast<int>(n), 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}

// Hardware base-2 exponential (v_exp_f32); arguments here are <= 0 or -inf.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace tg
