// Shared device helpers of the q4moe HIP library (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#define Q4_DEVICE __device__ __forceinline__

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace q4 {

constexpr int kGroup = 128;
constexpr int kWave = 64;
constexpr int kTileBytes = 1024;  // one (16-column block, group) weight tile

// Activation element types of the matrix core.
enum class Act { BF16 = 0, F16 = 1, I8 = 2 };

// ---------------------------------------------------------------- bit casts
template <typename To, typename From>
Q4_DEVICE To bitcast(const From& v) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, v);
}

// SwiGLU of one element: silu(g) * u = g / (1 + e^-g) * u, with the hardware exp2 and
// reciprocal (about 1 ulp each; -g large gives e^-g = inf and a zero result).
Q4_DEVICE float swiglu(float g, float u) {
  const float e = __expf(-g);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

Q4_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16, round to nearest even (finite inputs; NaN kept quiet).
Q4_DEVICE uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

Q4_DEVICE float f16_bits_to_f32(uint16_t b) { return float(bitcast<_Float16>(b)); }

// ---------------------------------------------------------------- wave reductions
Q4_DEVICE float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
Q4_DEVICE float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- nibble widening
// A 32-bit device word holds 8 unsigned nibbles d of the lane's 8 consecutive k:
// byte j holds element j in its low nibble and element j + 4 in its high nibble.
// Placing a nibble in the low mantissa bits under a magic exponent byte yields the
// exact value magic + d: bf16 0x43xx = 128 + d (step 1 up to 256), f16 0x64xx =
// 1024 + d (step 1 up to 2048).  Output register r holds elements (2r, 2r + 1) =
// (low, high half).
template <Act A>
Q4_DEVICE void widen_word_fp(uint32_t w, uint32_t out[4]) {
  // lo: elements 0..3 (one per byte, high halves cleared); hi: elements 4..7.  A byte
  // permute pairs two of them with the magic's high byte (0x43 / 0x64).
  constexpr uint32_t magic_bytes = (A == Act::BF16) ? 0x43434343u : 0x64646464u;
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  out[0] = __builtin_amdgcn_perm(magic_bytes, lo, 0x04010400u);
  out[1] = __builtin_amdgcn_perm(magic_bytes, lo, 0x04030402u);
  out[2] = __builtin_amdgcn_perm(magic_bytes, hi, 0x04010400u);
  out[3] = __builtin_amdgcn_perm(magic_bytes, hi, 0x04030402u);
}

// The magic offset of the widened value (value = offset + d).
template <Act A>
constexpr float magic_offset() { return A == Act::BF16 ? 128.0f : 1024.0f; }

// INT8 widening: d - 8 as a two's-complement nibble, placed in the high half of a
// byte (16 * (d - 8), exact in int8).  Returns two int8x4 registers holding the
// lane's elements (0..3) and (4..7) in k order: the low nibbles shifted up, and the
// high nibbles in place.
Q4_DEVICE void widen_word_i8(uint32_t w, uint32_t& lo, uint32_t& hi) {
  // flipping a nibble's top bit maps d to d - 8 in two's complement; with the nibble
  // already in a byte's high half that is an xor with 0x80 per byte, applied after the
  // mask (a shift and one three-input bit operation for lo, one for hi)
  lo = ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
  hi = (w & 0xF0F0F0F0u) ^ 0x80808080u;
}

// INT8 widening of 2-bit codes: a 32-bit device word of the 2-bit layout holds 16
// unsigned fields d = q + 2, four per byte; field f of byte m is element 4 (f % 2) + m
// of K step f / 2 of the word's two steps.  Moving field f to a byte's top two bits and
// flipping the top bit gives 64 (d - 2) = 64 q, exact in int8, for the four elements of
// the field in k order: out[f] is the int8x4 register of field f.
Q4_DEVICE void widen_word_i8_2bit(uint32_t w, uint32_t out[4]) {
  out[0] = ((w << 6) & 0xC0C0C0C0u) ^ 0x80808080u;
  out[1] = ((w << 4) & 0xC0C0C0C0u) ^ 0x80808080u;
  out[2] = ((w << 2) & 0xC0C0C0C0u) ^ 0x80808080u;
  out[3] = (w & 0xC0C0C0C0u) ^ 0x80808080u;
}

// ---------------------------------------------------------------- MFMA wrappers
template <Act A>
Q4_DEVICE f32x4_t mfma16x16x32(const uint32_t a[4], const uint32_t b[4], f32x4_t c) {
  u32x4_t av = {a[0], a[1], a[2], a[3]};
  u32x4_t bv = {b[0], b[1], b[2], b[3]};
  if constexpr (A == Act::BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(av), bitcast<bf16x8_t>(bv), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(av), bitcast<f16x8_t>(bv), c, 0, 0, 0);
  }
}

Q4_DEVICE i32x4_t mfma_i8_16x16x64(const uint32_t a[4], const uint32_t b[4], i32x4_t c) {
  i32x4_t av = {int32_t(a[0]), int32_t(a[1]), int32_t(a[2]), int32_t(a[3])};
  i32x4_t bv = {int32_t(b[0]), int32_t(b[1]), int32_t(b[2]), int32_t(b[3])};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
}

template <Act A>
Q4_DEVICE f32x4_t mfma16x16x32(u32x4_t av, u32x4_t bv, f32x4_t c) {
  if constexpr (A == Act::BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(av), bitcast<bf16x8_t>(bv), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(av), bitcast<f16x8_t>(bv), c, 0, 0, 0);
  }
}

Q4_DEVICE i32x4_t mfma_i8_16x16x64(u32x4_t a, u32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(bitcast<i32x4_t>(a), bitcast<i32x4_t>(b), c, 0, 0, 0);
}

// INT8 16x16x32: lane (row l % 16, quarter l / 16) holds k = 8 (l / 16) .. + 7 of A and
// B, 8 bytes each -- the first or second 8 bytes of a 16x16x64 operand.
Q4_DEVICE i32x4_t mfma_i8_16x16x32(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, i32x4_t c) {
  const long a = static_cast<long>((uint64_t(a1) << 32) | a0);
  const long b = static_cast<long>((uint64_t(b1) << 32) | b0);
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
}

Q4_DEVICE f32x4_t mfma_f32_16x16x4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- global loads
Q4_DEVICE uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
Q4_DEVICE uint2 load8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Non-temporal 16-byte load for streamed (read-once) weights.
Q4_DEVICE uint4 load16_stream(const void* p) {
#ifdef Q4_NO_NT
  return load16(p);
#else
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
#endif
}

// Non-temporal 8-byte load (the 2-bit weight tiles: 8 bytes per lane).
Q4_DEVICE uint2 load8_stream(const void* p) {
#ifdef Q4_NO_NT
  return load8(p);
#else
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
#endif
}

}  // namespace q4
