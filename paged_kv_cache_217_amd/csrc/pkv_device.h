// Device-side helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16

// Two bfloat16 values packed in a 32-bit word -> two floats (exact).
__device__ __forceinline__ void bf16x2_to_f32(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  // round to nearest even; NaN stays NaN (quiet)
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------- FP8 E4M3FN

// Four E4M3FN codes in a 32-bit word -> four floats with the gfx950 hardware
// conversion (OCP E4M3FN on this target; exactness over all 256 codes is
// checked by the GPU tests).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// float -> E4M3FN code: round to nearest, ties to even; magnitudes >= 448
// (infinity included) saturate to 448; NaN -> 0x7F. Integer arithmetic on
// the binary32 pattern, so the result does not depend on any hardware mode.
__device__ __forceinline__ uint32_t f32_to_fp8_e4m3_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7fu;                        // NaN
  const float a = __uint_as_float(mag);
  if (a >= 448.0f) return sign | 0x7eu;                         // saturate
  uint32_t code;
  if (a < 0.015625f) {                                          // below 2^-6: step 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // 0..8, 8 == 2^-6 (0x08)
  } else {
    const int e = static_cast<int>(mag >> 23) - 127;            // -6 .. 8
    // a / 2^(e-3) lies in [8, 16); round half to even, 16 carries into e+1
    const float scaled = __builtin_ldexpf(a, 3 - e);
    const uint32_t m = static_cast<uint32_t>(__builtin_rintf(scaled));
    code = static_cast<uint32_t>(e + 7) * 8u + (m - 8u);
  }
  return sign | code;
}

// float32 -> FP4 E2M1 code (0..15): round to nearest, ties to the even code;
// magnitudes >= 6 (infinity included) saturate to 6; NaN stores +0 (the format
// has neither); the sign is kept. Magnitudes step by 0.5 below 2, by 1 in
// [2, 4) and by 2 in [4, 6]; rintf rounds half to even, which is the even code
// in every range.
__device__ __forceinline__ uint32_t f32_to_fp4_e2m1_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0u;                             // NaN
  const uint32_t sign = (u >> 28) & 0x8u;
  const float a = __uint_as_float(mag);
  if (a >= 6.0f) return sign | 0x7u;
  uint32_t code;
  if (a < 2.0f)
    code = static_cast<uint32_t>(__builtin_rintf(a * 2.0f));          // 0..4
  else if (a < 4.0f)
    code = static_cast<uint32_t>(__builtin_rintf(a)) + 2u;            // 4..6
  else
    code = static_cast<uint32_t>(__builtin_rintf(a * 0.5f)) + 4u;     // 6..7
  return sign | code;
}

// ---------------------------------------------------------------- misc

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace pkv
