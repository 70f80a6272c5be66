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

// KV element formats of the kernel templates
constexpr int kFmtBf16 = 0, kFmtFp8 = 1, kFmtFp4 = 2;

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

// A wave-uniform 32-bit read that stays a scalar load. A plain global read
// placed after a barrier or a store becomes a vector load (the compiler can
// no longer rule out that the memory was written), and a vector load used as
// a scalar waits on every vector load in flight. Read through the constant
// address space instead; only for data that nothing in flight writes (block
// tables).
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
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

// Two fp32 weights -> their bf16 heads (round to nearest even, packed) and
// bf16 tails (the exact remainders p - head, rounded the same way). The
// remainder is at most 2^-9 p, so head + tail carries p to about 2^-18
// relative; both halves are fed to the matrix cores as separate operands.
// The heads are widened back from the packed word itself (a shift and a
// mask); the empty asm hides the word's origin, without which the compiler
// converts the first weight a second time to get the low half.
struct Bf16Split {
  uint32_t hi, lo;
};
__device__ __forceinline__ Bf16Split split_bf16(float p0, float p1) {
  uint32_t hi = pack_bf16(p0, p1);
  asm("" : "+v"(hi));
  const float r0 = p0 - __uint_as_float(hi << 16);
  const float r1 = p1 - __uint_as_float(hi & 0xffff0000u);
  return Bf16Split{hi, pack_bf16(r0, r1)};
}

// max that propagates NaN (a NaN score of a live token makes the row NaN, as
// the definition does); gfx950 has it as one instruction for three operands
// and, unlike fmaxf, it needs no quieting of its inputs first
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

// FP4 V rows: x0, x1 hold 8 codes (dims 0..7, dim 2i in the low nibble of
// byte i) of two tokens. Interleaved so that byte i of `ev` holds dim 2i of
// both tokens (token 0 low) and byte i of `od` dim 2i + 1, one conversion
// yields the bf16 pair (token 0, token 1) of one dim: the transposed operand
// without byte permutes.
struct Fp4Pair {
  uint32_t ev, od;
};
__device__ __forceinline__ Fp4Pair fp4_interleave(uint32_t x0, uint32_t x1) {
  return Fp4Pair{(x0 & 0x0F0F0F0Fu) | ((x1 << 4) & 0xF0F0F0F0u),
                 ((x0 >> 4) & 0x0F0F0F0Fu) | (x1 & 0xF0F0F0F0u)};
}
// bf16 pair (token 0, token 1) of dim j (0..7; a constant after unrolling)
__device__ __forceinline__ uint32_t fp4_pair_dim(const Fp4Pair& p, int j) {
  switch (j) {
    case 0: return fp4x2_to_bf16x2<0>(p.ev);
    case 1: return fp4x2_to_bf16x2<0>(p.od);
    case 2: return fp4x2_to_bf16x2<1>(p.ev);
    case 3: return fp4x2_to_bf16x2<1>(p.od);
    case 4: return fp4x2_to_bf16x2<2>(p.ev);
    case 5: return fp4x2_to_bf16x2<2>(p.od);
    case 6: return fp4x2_to_bf16x2<3>(p.ev);
    default: return fp4x2_to_bf16x2<3>(p.od);
  }
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group,
// lane a supplies the address of 4 consecutive 16-bit elements M[a][0..3];
// lane j receives M[4 i + j / 4][j % 4] for i = 0..3 (layout measured on
// gfx950). Pointing lane a at row a / 4 of a matrix, columns 4 (a % 4) ..,
// hands lane j column j of 4 consecutive rows: a 4 x 16 block transposed.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4_t lds_s4_t;
  const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// x combined with the value of lane ^ 16 (resp. lane ^ 32) through the
// gfx950 row-swap moves instead of an LDS permute
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mfma

}  // namespace pkv
