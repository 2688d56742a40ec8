// Shared device helpers for the Sep-Attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sep {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` strictly below this lane.
__device__ __forceinline__ uint32_t mbcnt(uint64_t mask) {
  uint32_t lo = __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u);
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32), lo);
}

// Exchange a value with lane (l ^ 32).
__device__ __forceinline__ float swap_half(float x) {
  return __shfl_xor(x, 32, kWave);
}

// Max and sum of a value over lanes l and l^32, without LDS. One
// v_permlane32_swap on two copies of x exchanges the high half of the first
// with the low half of the second, so that afterwards one copy holds the low
// half of x on every lane and the other the high half. The swap is written
// as inline asm: the compiler's builtin for it loses one of the two results
// when both inputs are the same value. The s_nop pairs cover the VALU
// write -> permlane read and permlane write -> VALU read hazards.
__device__ __forceinline__ void lane_halves(float x, float* lo, float* hi) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), w = u;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(u), "+v"(w));
  *lo = __builtin_bit_cast(float, u);
  *hi = __builtin_bit_cast(float, w);
}
__device__ __forceinline__ float half_max(float x) {
  float a, b;
  lane_halves(x, &a, &b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a, b;
  lane_halves(x, &a, &b);
  return a + b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Pack two floats into two bf16 (round to nearest even) in one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// MFMA wrappers. Operand layouts (wave64):
//  32x32x16 bf16: A lane l holds row l%32, 8 k-values of group l/32;
//                 B lane l holds column l%32, the same 8 k-values;
//                 C lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4.
//  32x32x2 f32:   A lane l holds row l%32, k = l/32; B column l%32, k = l/32;
//                 C as above.
//  16x16x32 bf16: A lane l holds row l%16, 8 k-values of group l/16;
//                 B column l%16, same k-values; C column l%16, rows 4*(l/16)+r.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Membership of `id` in a small id list held in LDS.
__device__ __forceinline__ bool in_set(int32_t id, const int32_t* set, int n) {
  bool hit = false;
  for (int i = 0; i < n; ++i) hit |= (set[i] == id);
  return hit;
}

}  // namespace sep
