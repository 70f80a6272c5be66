// Helpers shared by the matrix-core attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace mfma {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescale = 8.0f;     // log2 of the largest weight allowed before rescaling

template <int BYTES>
struct Vec;
template <>
struct Vec<16> {
  using T = uint4;
};
template <>
struct Vec<8> {
  using T = uint2;
};
template <>
struct Vec<4> {
  using T = uint32_t;
};

// Streaming (non-temporal) loads of KV bytes: every K/V byte is read once
// per step, so the loads ask the caches not to keep the lines.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void ld_stream(uint4& out, const uint8_t* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  out = make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void ld_stream(uint2& out, const uint8_t* p) {
  const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  out = make_uint2(x[0], x[1]);
}
__device__ __forceinline__ void ld_stream(uint32_t& out, const uint8_t* p) {
  out = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Buffer-resource form of the same streaming loads: the (block, head) tile's
// base and size sit in four scalar registers and each lane adds a 32-bit
// offset. A resource of size 0 (an absent block) makes every load return
// zeros without touching memory, so the tail of a chunk needs no branches.
// Word 3 is the raw (untyped, unswizzled) buffer configuration of CDNA.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;            // cache-policy bit of the load
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0),
                                           bytes, kRawBufferWord3);
}
// `off` is the per-lane part of the byte offset (one register shared by many
// loads), `soff` a wave-uniform part (a compile-time constant at every call).
__device__ __forceinline__ void ld_stream(uint4& out, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          int soff) {
  const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kLoadNonTemporal);
  out = make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void ld_stream(uint2& out, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          int soff) {
  const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, kLoadNonTemporal);
  out = make_uint2(x[0], x[1]);
}
__device__ __forceinline__ void ld_stream(uint32_t& out, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          int soff) {
  out = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, kLoadNonTemporal);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t word(const uint2& v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t word(const uint32_t& v, int) { return v; }

// 2 FP8 E4M3FN codes (bytes 0,1 or 2,3 of w) -> 2 bf16 in one word, exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// 2 FP4 E2M1 codes (byte B of w: low nibble first) -> 2 bf16 in one word,
// exact (every E2M1 value is a bf16 value).
template <int B>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

}  // namespace mfma

}  // namespace pkv
