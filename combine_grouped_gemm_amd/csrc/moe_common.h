// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------------------------
// scalar conversions
// ------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 with round-to-nearest-even, on gfx950's v_cvt_pk_bf16_f32 (one instruction
// for two values; NaN stays NaN).
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_cvt_t{lo, hi}, bf16x2_cvt_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// logistic sigmoid 1 / (1 + e^-x), written as 1 / (1 + 2^(-x log2 e)) on the hardware
// exp2 and reciprocal (each within about 1 ulp of fp32); SwiGLU's gate is silu(x) = x sigmoid(x)
__device__ __forceinline__ float sigmoid_f32(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_f32(float x) { return x * sigmoid_f32(x); }

// OCP e4m3fn encode of a finite fp32 value: round to nearest even, saturate to +-448.
// Normal range (|v| >= 2^-6): keep the 3 leading fraction bits of the fp32 significand
// and round on the 20 dropped bits; a carry propagates into the exponent field.
// Subnormal range: the grid is 2^-9, so round |v| * 2^9 to an integer (0..8; 8 is the
// code of 2^-6).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // 2^-6
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t au = u & 0x7FFFFFFFu;
    const uint32_t exp = (au >> 23) - 127u + 7u;  // e4m3 exponent field, 1..15
    const uint32_t keep = (au >> 20) & 7u;
    const uint32_t rem = au & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
    code = (exp << 3) + keep + up;
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

// e4m3fn code -> bf16 bits, exact (3 mantissa bits and exponents 2^-9..2^8 fit bf16).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 7u;
  if (e != 0) return s | ((e + 120u) << 7) | (m << 4);
  // subnormal m * 2^-9: the fp32 value is exact and has at most 3 significant bits
  return s | (__float_as_uint(static_cast<float>(m) * 0.001953125f) >> 16);
}

// four e4m3 codes (one per byte) -> four bf16 packed in two dwords
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
  uint2 r;
  r.x = e4m3_to_bf16_bits(w & 0xFFu) | (e4m3_to_bf16_bits((w >> 8) & 0xFFu) << 16);
  r.y = e4m3_to_bf16_bits((w >> 16) & 0xFFu) | (e4m3_to_bf16_bits(w >> 24) << 16);
  return r;
}

// Four e4m3 codes times one fp32 scale, rounded once to bf16 (the code's value is exact in
// fp32, so the product rounds once)
__device__ __forceinline__ uint2 e4m3x4_scaled_to_bf16x4(uint32_t w, float s) {
  const uint2 b = e4m3x4_to_bf16x4(w);
  auto val = [](uint32_t bits16) { return __uint_as_float(bits16 << 16); };
  uint2 r;
  r.x = pack_bf16x2(val(b.x & 0xFFFFu) * s, val(b.x >> 16) * s);
  r.y = pack_bf16x2(val(b.y & 0xFFFFu) * s, val(b.y >> 16) * s);
  return r;
}

// 8 e4m3 codes (one 8-byte fragment) times one fp32 scale, as 8 bf16 values: each code is
// decoded exactly by the hardware conversion, multiplied in fp32 and rounded to bf16
// the two e4m3 codes in the low (HI = false) or high half of w, times s, as packed bf16
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_scaled_to_bf16x2(uint32_t w, float s) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t p = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
  return pack_bf16x2(p.x * s, p.y * s);
}
__device__ __forceinline__ uint4 e4m3x8_scaled_to_bf16x8(uint2 raw, float s) {
  return make_uint4(e4m3x2_scaled_to_bf16x2<false>(raw.x, s), e4m3x2_scaled_to_bf16x2<true>(raw.x, s),
                    e4m3x2_scaled_to_bf16x2<false>(raw.y, s), e4m3x2_scaled_to_bf16x2<true>(raw.y, s));
}

// ------------------------------------------------------------------------------------
// wave-level reductions (all lanes receive the result)
// ------------------------------------------------------------------------------------

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// fp32 -> uint32 whose unsigned order is the float order; +0 and -0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace moe
