// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_amd.h"

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// ---- bf16 <-> fp32 --------------------------------------------------------
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
MOE_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// fp32 -> bf16, round to nearest even (the hardware convert, v_cvt_pk_bf16_f32).
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
MOE_DEV uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Logistic function from the hardware 2^x and reciprocal (about 1 ulp each):
// 1 / (1 + 2^(-x log2 e)). Saturates to 0 / 1 for large |x|.
MOE_DEV float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// ---- OCP FP8 E4M3 ("fn": no infinities, max 448) ---------------------------
// fp32 -> e4m3 code, round to nearest even: the gfx950 hardware convert
// (v_cvt_pk_fp8_f32, OCP format). Every caller divides by a scale of amax/448, so
// |v| <= 448 up to the division's rounding and nothing saturates; on every fp32 |v| < 464
// the hardware codes equal a round-to-nearest-even, saturate-to-448 conversion written
// out on the bit pattern (compared exhaustively on the device). NaN gives a NaN code.
MOE_DEV uint32_t f32_to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xffu;
}
// Four codes packed little-endian into one word: a | b << 8 | c << 16 | d << 24.
MOE_DEV uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

MOE_DEV float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xf, m = c & 7;
  float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// A NaN logit counts as -inf (the router's reading of non-finite logits).
MOE_DEV float nan_to_ninf(float v) { return v != v ? -__builtin_inff() : v; }

// ---- wave reductions -------------------------------------------------------
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

MOE_DEV uint64_t lanemask_lt() {
  int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe

// ---- host-side helpers (internal; not exported) ---------------------------
#define MOE_CHECK_LAUNCH()                                      \
  do {                                                          \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;    \
  } while (0)

#define MOE_REQUIRE(cond, err) \
  do {                         \
    if (!(cond)) return (err); \
  } while (0)

static inline bool moe_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
