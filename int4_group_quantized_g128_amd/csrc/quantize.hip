// A1 quantise + pack and A2 device repack.
//
// Format: page "从FP32到INT4：大语言模型量化压缩实战指南" §1.3 (groups of 128 along
// K, a scale per group from its own min/max, a zero point only when asymmetric);
// page "高效大语言模型推理实践：INT4量化与MoE架构的融合探索", INT4量化实现 (4-bit
// integers plus an independent per-group scale).
#include "common.h"
#include "internal.h"

namespace q4 {

// binary16 rounded toward +inf of a non-negative finite float: the smallest
// binary16 value that is >= t.
Q4_DEVICE uint16_t f32_to_f16_up(float t) {
  __half h = __float2half_rn(t);
  uint16_t b = __half_as_ushort(h);
  if (__half2float(h) < t) b = uint16_t(b + 1);   // next binary16 up (t >= 0)
  return b;
}

// One wave per (row, pair of groups).  Lane j covers k = 128 g + 2 j and 2 j + 1 and
// writes byte j of the group's 64 packed bytes.
template <int DT, bool ASYM>
__global__ void __launch_bounds__(64) k_quantize_g128(const void* __restrict__ w, int64_t n, int64_t k,
                                                     uint8_t* __restrict__ packed,
                                                     uint16_t* __restrict__ scales,
                                                     uint8_t* __restrict__ zeros,
                                                     int32_t* __restrict__ flags) {
  const int64_t G = k / kGroup;
  const int64_t pairs = (G + 1) / 2;
  const int64_t row = int64_t(blockIdx.x) / pairs;
  const int64_t pair = int64_t(blockIdx.x) % pairs;
  const int lane = threadIdx.x;
  uint32_t zbyte = 0;
  int flag = 0;
  for (int h = 0; h < 2; ++h) {
    const int64_t g = pair * 2 + h;
    if (g >= G) break;
    const int64_t base = row * k + g * kGroup + 2 * lane;
    float v0, v1;
    if constexpr (DT == 0) {
      const float2 p = *reinterpret_cast<const float2*>(static_cast<const float*>(w) + base);
      v0 = p.x;
      v1 = p.y;
    } else {
      const uint32_t p = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(w) + base);
      if constexpr (DT == 1) {
        v0 = f16_bits_to_f32(uint16_t(p & 0xffff));
        v1 = f16_bits_to_f32(uint16_t(p >> 16));
      } else {
        v0 = bf16_to_f32(uint16_t(p & 0xffff));
        v1 = bf16_to_f32(uint16_t(p >> 16));
      }
    }
    if (!__builtin_isfinite(v0) || !__builtin_isfinite(v1)) flag |= 1;
    uint32_t c0, c1;
    if constexpr (!ASYM) {
      const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
      const float t = __fdiv_rn(amax, 7.0f);
      const __half sh = __float2half_rn(t);
      const uint16_t sb = __half_as_ushort(sh);
      if ((sb & 0x7fff) >= 0x7c00) flag |= 2;
      const float s = __half2float(sh);
      float q0 = 0.f, q1 = 0.f;
      if (s > 0.f) {
        q0 = fminf(fmaxf(rintf(__fdiv_rn(v0, s)), -8.f), 7.f);
        q1 = fminf(fmaxf(rintf(__fdiv_rn(v1, s)), -8.f), 7.f);
      }
      c0 = uint32_t(int(q0)) & 0xF;
      c1 = uint32_t(int(q1)) & 0xF;
      if (lane == 0) scales[row * G + g] = sb;
    } else {
      const float mn = fminf(wave_min(fminf(v0, v1)), 0.f);
      const float mx = fmaxf(wave_max(fmaxf(v0, v1)), 0.f);
      const float t = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
      const uint16_t sb = f32_to_f16_up(t);
      if ((sb & 0x7fff) >= 0x7c00) flag |= 2;
      const float s = f16_bits_to_f32(sb);
      float z = 0.f, q0 = 0.f, q1 = 0.f;
      if (s > 0.f) {
        z = fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.f), 15.f);
        q0 = fminf(fmaxf(__fadd_rn(rintf(__fdiv_rn(v0, s)), z), 0.f), 15.f);
        q1 = fminf(fmaxf(__fadd_rn(rintf(__fdiv_rn(v1, s)), z), 0.f), 15.f);
      }
      c0 = uint32_t(int(q0));
      c1 = uint32_t(int(q1));
      zbyte |= uint32_t(int(z)) << (4 * h);
      if (lane == 0) scales[row * G + g] = sb;
    }
    packed[(row * k + g * kGroup) / 2 + lane] = uint8_t(c0 | (c1 << 4));
  }
  if constexpr (ASYM) {
    if (lane == 0) zeros[row * ((G + 1) / 2) + pair] = uint8_t(zbyte);
  }
  if (flags) {
    // any lane that saw a problem reports it
    const unsigned long long any = __ballot(flag != 0);
    if (any) {
      int all = flag;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) all |= __shfl_xor(all, o, 64);
      if (lane == 0) atomicOr(flags, all);
    }
  }
}

// Other group sizes (32, 64, 256; page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析"
// §5.3 sizes groups by expert hotness): one wave per (row, two 256-element chunks);
// lane j covers k = 256 c + 4 j .. 4 j + 3 and writes 2 packed bytes; a group spans
// group / 4 aligned lanes, reduced with xor shuffles.  Same arithmetic as the 128
// kernel.  Zero points (asymmetric, groups of 256 only): the two chunks of a wave are
// the two groups of one zero-point byte.
template <int DT, bool ASYM>
__global__ void __launch_bounds__(64) k_quantize_grp(const void* __restrict__ w, int64_t n, int64_t k, int group,
                                                    uint8_t* __restrict__ packed, uint16_t* __restrict__ scales,
                                                    uint8_t* __restrict__ zeros, int32_t* __restrict__ flags) {
  const int64_t chunks = (k + 255) / 256;
  const int64_t pairs = (chunks + 1) / 2;
  const int64_t row = int64_t(blockIdx.x) / pairs;
  const int64_t pair = int64_t(blockIdx.x) % pairs;
  const int64_t Gc = k / group;
  const int lane = threadIdx.x;
  const int lpg = group / 4;            // lanes per group: 8, 16 or 64
  uint32_t zbyte = 0;
  int flag = 0;
  for (int h = 0; h < 2; ++h) {
    const int64_t c = pair * 2 + h;
    if (c >= chunks) break;
    const int64_t k0 = c * 256 + 4 * lane;
    const bool valid = k0 < k;          // whole groups are valid or not (k % group == 0)
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      const int64_t base = row * k + k0;
      if constexpr (DT == 0) {
        const float4 p = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + base);
        v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
      } else {
        const uint2 p = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + base);
        const uint16_t b[4] = {uint16_t(p.x & 0xffff), uint16_t(p.x >> 16), uint16_t(p.y & 0xffff),
                               uint16_t(p.y >> 16)};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = DT == 1 ? f16_bits_to_f32(b[e]) : bf16_to_f32(b[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!__builtin_isfinite(v[e])) flag |= 1;
    }
    uint32_t codes = 0;
    if constexpr (!ASYM) {
      float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
      for (int o = 1; o < lpg; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const float t = __fdiv_rn(amax, 7.0f);
      const __half sh = __float2half_rn(t);
      const uint16_t sb = __half_as_ushort(sh);
      if (valid && (sb & 0x7fff) >= 0x7c00) flag |= 2;
      const float s = __half2float(sh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float q = 0.f;
        if (s > 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(v[e], s)), -8.f), 7.f);
        codes |= (uint32_t(int(q)) & 0xF) << (4 * e);
      }
      if (valid && lane % lpg == 0) scales[row * Gc + k0 / group] = sb;
    } else {
      float mn = fminf(fminf(v[0], v[1]), fminf(v[2], v[3]));
      float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      for (int o = 1; o < lpg; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      }
      mn = fminf(mn, 0.f);
      mx = fmaxf(mx, 0.f);
      const float t = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
      const uint16_t sb = f32_to_f16_up(t);
      if (valid && (sb & 0x7fff) >= 0x7c00) flag |= 2;
      const float s = f16_bits_to_f32(sb);
      float z = 0.f;
      if (s > 0.f) z = fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.f), 15.f);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float q = 0.f;
        if (s > 0.f) q = fminf(fmaxf(__fadd_rn(rintf(__fdiv_rn(v[e], s)), z), 0.f), 15.f);
        codes |= uint32_t(int(q)) << (4 * e);
      }
      zbyte |= uint32_t(int(z)) << (4 * h);
      if (valid && lane % lpg == 0) scales[row * Gc + k0 / group] = sb;
    }
    if (valid) *reinterpret_cast<uint16_t*>(packed + (row * k + k0) / 2) = uint16_t(codes);
  }
  if constexpr (ASYM) {
    if (lane == 0) zeros[row * ((Gc + 1) / 2) + pair] = uint8_t(zbyte);
  }
  if (flags) {
    const unsigned long long any = __ballot(flag != 0);
    if (any) {
      int all = flag;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) all |= __shfl_xor(all, o, 64);
      if (lane == 0) atomicOr(flags, all);
    }
  }
}

// A2: one thread per 32-bit word of the device weights.  Word index
// ((cb * G + g) * 64 + lane) * 4 + s; it gathers elements k = 128 g + 32 s + 8 kq + e,
// e in [0, 8) (4 canonical bytes) of device column 16 cb + lane % 16.
__global__ void k_repack_weights(const uint8_t* __restrict__ packed, int64_t n, int64_t k, int asym,
                                 int gate_up, uint32_t* __restrict__ out) {
  const int64_t G = k / kGroup;
  const int64_t total = n * k / 8;
  for (int64_t wi = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; wi < total;
       wi += int64_t(gridDim.x) * blockDim.x) {
    const int s = int(wi & 3);
    const int lane = int((wi >> 2) & 63);
    const int64_t tile = wi >> 8;
    const int64_t g = tile % G;
    const int64_t cb = tile / G;
    const int c = lane & 15, kq = lane >> 4;
    int64_t col = cb * 16 + c;
    int64_t src = col;
    if (gate_up) {
      const int64_t half = n / 2;
      src = (cb & 1) ? half + (cb >> 1) * 16 + c : (cb >> 1) * 16 + c;
    }
    const int64_t k0 = g * kGroup + 32 * s + 8 * kq;
    const uint32_t in = *reinterpret_cast<const uint32_t*>(packed + (src * k + k0) / 2);
    // in: nibble e (bits 4e..4e+3) is element e; out: element e at position p(e)
    uint32_t o = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t d = (in >> (4 * e)) & 0xF;
      if (!asym) d ^= 0x8;                         // two's complement q -> q + 8
      const int p = 2 * (e & 3) + (e >> 2);       // byte e % 4, high nibble for e >= 4
      o |= d << (4 * p);
    }
    out[wi] = o;
  }
}

// Scales (and zero points) into [n/16][G][16][SG] with the device column order.  SG
// scale entries per 128-element tile (128 / group for groups of 32 and 64, else 1),
// adjacent per column; entry (tile g, j) holds canonical group (128 g + j 128 / SG) /
// group, so a 256-group's scale (and zero point) is repeated on both of its tiles.
__global__ void k_repack_meta(const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
                              int64_t n, int64_t k, int group, int gate_up, uint16_t* __restrict__ sout,
                              uint8_t* __restrict__ zout) {
  const int64_t G = k / kGroup;
  const int SG = group < kGroup ? kGroup / group : 1;
  const int64_t Gc = k / group;
  const int64_t total = n * G * SG;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int j = int(i % SG);
    const int c = int((i / SG) & 15);
    const int64_t g = (i / SG >> 4) % G;
    const int64_t cb = (i / SG >> 4) / G;
    int64_t src = cb * 16 + c;
    if (gate_up) {
      const int64_t half = n / 2;
      src = (cb & 1) ? half + (cb >> 1) * 16 + c : (cb >> 1) * 16 + c;
    }
    const int64_t cg = (g * kGroup + j * (kGroup / SG)) / group;
    sout[i] = scales[src * Gc + cg];
    if (zout) {   // SG == 1
      const uint8_t zb = zeros[src * ((Gc + 1) / 2) + cg / 2];
      zout[i] = (cg & 1) ? (zb >> 4) : (zb & 0xF);
    }
  }
}

// Zero-fills alignment padding so the device image is fully defined.
__global__ void k_zero_bytes(uint8_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// INT8 g128 (the W8A8 weight format): one wave per (row, group), lane j covers
// k = 128 g + 2 j and 2 j + 1.  s = binary16 rounded up of fp32(amax) / 127,
// q = clamp(rint(w / s), -127, 127).
template <int DT>
__global__ void __launch_bounds__(64) k_quantize8_g128(const void* __restrict__ w, int64_t n, int64_t k,
                                                      int8_t* __restrict__ q, uint16_t* __restrict__ scales,
                                                      int32_t* __restrict__ flags) {
  const int64_t G = k / kGroup;
  const int64_t row = int64_t(blockIdx.x) / G, g = int64_t(blockIdx.x) % G;
  const int lane = threadIdx.x;
  const int64_t base = row * k + g * kGroup + 2 * lane;
  float v0, v1;
  if constexpr (DT == 0) {
    const float2 p = *reinterpret_cast<const float2*>(static_cast<const float*>(w) + base);
    v0 = p.x;
    v1 = p.y;
  } else {
    const uint32_t p = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(w) + base);
    if constexpr (DT == 1) {
      v0 = f16_bits_to_f32(uint16_t(p & 0xffff));
      v1 = f16_bits_to_f32(uint16_t(p >> 16));
    } else {
      v0 = bf16_to_f32(uint16_t(p & 0xffff));
      v1 = bf16_to_f32(uint16_t(p >> 16));
    }
  }
  int flag = (!__builtin_isfinite(v0) || !__builtin_isfinite(v1)) ? 1 : 0;
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const uint16_t sb = f32_to_f16_up(__fdiv_rn(amax, 127.0f));
  if ((sb & 0x7fff) >= 0x7c00) flag |= 2;
  const float s = f16_bits_to_f32(sb);
  float q0 = 0.f, q1 = 0.f;
  if (s > 0.f) {
    q0 = fminf(fmaxf(rintf(__fdiv_rn(v0, s)), -127.f), 127.f);
    q1 = fminf(fmaxf(rintf(__fdiv_rn(v1, s)), -127.f), 127.f);
  }
  const uint16_t pair = uint16_t((uint32_t(int(q0)) & 0xff) | ((uint32_t(int(q1)) & 0xff) << 8));
  *reinterpret_cast<uint16_t*>(q + base) = pair;
  if (lane == 0) scales[row * G + g] = sb;
  if (flags) {
    const unsigned long long any = __ballot(flag != 0);
    if (any) {
      int all = flag;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) all |= __shfl_xor(all, o, 64);
      if (lane == 0) atomicOr(flags, all);
    }
  }
}

// INT8 device tiles: one thread per (tile, half, lane) 16-byte chunk: bytes 0..7 are
// k = 128 g + 64 half + 8 kq + (0..7), bytes 8..15 the same + 32, of device column
// 16 cb + lane % 16.
__global__ void k_repack8_weights(const int8_t* __restrict__ q, int64_t n, int64_t k, int gate_up,
                                  uint4* __restrict__ out) {
  const int64_t G = k / kGroup;
  const int64_t total = n * k / 16;
  for (int64_t ci = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; ci < total;
       ci += int64_t(gridDim.x) * blockDim.x) {
    const int lane = int(ci & 63);
    const int half = int((ci >> 6) & 1);
    const int64_t tile = ci >> 7;
    const int64_t g = tile % G, cb = tile / G;
    const int c = lane & 15, kq = lane >> 4;
    int64_t src = cb * 16 + c;
    if (gate_up) {
      const int64_t hn = n / 2;
      src = (cb & 1) ? hn + (cb >> 1) * 16 + c : (cb >> 1) * 16 + c;
    }
    const int8_t* row = q + src * k + g * kGroup + 64 * half + 8 * kq;
    const uint2 lo = *reinterpret_cast<const uint2*>(row);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 32);
    out[ci] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// INT2 g128 (cold experts; page "大模型之Dense、MoE与量化", APEX section: rarely used
// experts in 2 bits): one wave per (row, group), lane j covers k = 128 g + 2 j and
// 2 j + 1.  s = binary16 rounded up of fp32(amax), q = clamp(rint(w / s), -2, 1), two's
// complement, four codes per byte (lane 2 b writes byte b: its two codes low, lane
// 2 b + 1's high).
template <int DT>
__global__ void __launch_bounds__(64) k_quantize2_g128(const void* __restrict__ w, int64_t n, int64_t k,
                                                      uint8_t* __restrict__ packed, uint16_t* __restrict__ scales,
                                                      int32_t* __restrict__ flags) {
  const int64_t G = k / kGroup;
  const int64_t row = int64_t(blockIdx.x) / G, g = int64_t(blockIdx.x) % G;
  const int lane = threadIdx.x;
  const int64_t base = row * k + g * kGroup + 2 * lane;
  float v0, v1;
  if constexpr (DT == 0) {
    const float2 p = *reinterpret_cast<const float2*>(static_cast<const float*>(w) + base);
    v0 = p.x;
    v1 = p.y;
  } else {
    const uint32_t p = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(w) + base);
    if constexpr (DT == 1) {
      v0 = f16_bits_to_f32(uint16_t(p & 0xffff));
      v1 = f16_bits_to_f32(uint16_t(p >> 16));
    } else {
      v0 = bf16_to_f32(uint16_t(p & 0xffff));
      v1 = bf16_to_f32(uint16_t(p >> 16));
    }
  }
  int flag = (!__builtin_isfinite(v0) || !__builtin_isfinite(v1)) ? 1 : 0;
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const uint16_t sb = f32_to_f16_up(amax);
  if ((sb & 0x7fff) >= 0x7c00) flag |= 2;
  const float s = f16_bits_to_f32(sb);
  float q0 = 0.f, q1 = 0.f;
  if (s > 0.f) {
    q0 = fminf(fmaxf(rintf(__fdiv_rn(v0, s)), -2.f), 1.f);
    q1 = fminf(fmaxf(rintf(__fdiv_rn(v1, s)), -2.f), 1.f);
  }
  const uint32_t two = (uint32_t(int(q0)) & 3u) | ((uint32_t(int(q1)) & 3u) << 2);
  const uint32_t other = uint32_t(__shfl_xor(int(two), 1, 64));
  if ((lane & 1) == 0) packed[(row * k + g * kGroup) / 4 + lane / 2] = uint8_t(two | (other << 4));
  if (lane == 0) scales[row * G + g] = sb;
  if (flags) {
    const unsigned long long any = __ballot(flag != 0);
    if (any) {
      int all = flag;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) all |= __shfl_xor(all, o, 64);
      if (lane == 0) atomicOr(flags, all);
    }
  }
}

// 2-bit device tiles: one thread per 32-bit device word, word index
// ((cb * G + g) * 64 + lane) * 2 + j; word j holds K steps 2 j and 2 j + 1 of device
// column 16 cb + lane % 16, quarter kq = lane / 16: element e of step s
// (k = 128 g + 32 s + 8 kq + e) in byte e % 4, field 2 (s % 2) + e / 4, as d = q + 2.
__global__ void k_repack2_weights(const uint8_t* __restrict__ packed, int64_t n, int64_t k, int gate_up,
                                  uint32_t* __restrict__ out) {
  const int64_t G = k / kGroup;
  const int64_t total = n * k / 16;
  for (int64_t wi = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; wi < total;
       wi += int64_t(gridDim.x) * blockDim.x) {
    const int j = int(wi & 1);
    const int lane = int((wi >> 1) & 63);
    const int64_t tile = wi >> 7;
    const int64_t g = tile % G, cb = tile / G;
    const int c = lane & 15, kq = lane >> 4;
    int64_t src = cb * 16 + c;
    if (gate_up) {
      const int64_t half = n / 2;
      src = (cb & 1) ? half + (cb >> 1) * 16 + c : (cb >> 1) * 16 + c;
    }
    uint32_t o = 0;
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      const int s = 2 * j + sp;
      const int64_t k0 = g * kGroup + 32 * s + 8 * kq;   // 8 codes = two canonical bytes
      const uint32_t in = *reinterpret_cast<const uint16_t*>(packed + (src * k + k0) / 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t d = ((in >> (2 * e)) & 3u) ^ 2u;   // two's complement q -> q + 2
        o |= d << (8 * (e & 3) + 2 * (2 * sp + (e >> 2)));
      }
    }
    out[wi] = o;
  }
}

hipError_t launch_quantize2(const void* w, int dtype, int64_t n, int64_t k, uint8_t* packed, uint16_t* scales,
                            int32_t* flags, hipStream_t st) {
  const dim3 grid(unsigned(n * (k / kGroup)));
  if (dtype == 0) hipLaunchKernelGGL(k_quantize2_g128<0>, grid, dim3(64), 0, st, w, n, k, packed, scales, flags);
  else if (dtype == 1) hipLaunchKernelGGL(k_quantize2_g128<1>, grid, dim3(64), 0, st, w, n, k, packed, scales, flags);
  else hipLaunchKernelGGL(k_quantize2_g128<2>, grid, dim3(64), 0, st, w, n, k, packed, scales, flags);
  return hipGetLastError();
}

hipError_t launch_repack2(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int gate_up, void* out,
                          hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(out);
  const int64_t G = k / kGroup;
  const int64_t words = n * k / 16;
  const int64_t sb = align256(n * k / 4);
  unsigned blocks = unsigned(std::min<int64_t>((words + 255) / 256, 65536));
  hipLaunchKernelGGL(k_repack2_weights, dim3(blocks), dim3(256), 0, st, packed, n, k, gate_up,
                     reinterpret_cast<uint32_t*>(base));
  const int64_t wpad = sb - n * k / 4;
  if (wpad > 0) hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(256), 0, st, base + n * k / 4, wpad);
  unsigned mblocks = unsigned(std::min<int64_t>((n * G + 255) / 256, 65536));
  hipLaunchKernelGGL(k_repack_meta, dim3(mblocks), dim3(256), 0, st, scales, nullptr, n, k, int(kGroup), gate_up,
                     reinterpret_cast<uint16_t*>(base + sb), nullptr);
  const int64_t scale_pad = align256(2 * n * G) - 2 * n * G;
  if (scale_pad > 0) hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(256), 0, st, base + sb + 2 * n * G, scale_pad);
  return hipGetLastError();
}

hipError_t launch_quantize8(const void* w, int dtype, int64_t n, int64_t k, int8_t* q, uint16_t* scales,
                            int32_t* flags, hipStream_t st) {
  const dim3 grid(unsigned(n * (k / kGroup)));
  if (dtype == 0) hipLaunchKernelGGL(k_quantize8_g128<0>, grid, dim3(64), 0, st, w, n, k, q, scales, flags);
  else if (dtype == 1) hipLaunchKernelGGL(k_quantize8_g128<1>, grid, dim3(64), 0, st, w, n, k, q, scales, flags);
  else hipLaunchKernelGGL(k_quantize8_g128<2>, grid, dim3(64), 0, st, w, n, k, q, scales, flags);
  return hipGetLastError();
}

hipError_t launch_repack8(const int8_t* q, const uint16_t* scales, int64_t n, int64_t k, int gate_up, void* out,
                          hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(out);
  const int64_t G = k / kGroup;
  const int64_t chunks = n * k / 16;
  const int64_t sb = align256(n * k);
  unsigned blocks = unsigned(std::min<int64_t>((chunks + 255) / 256, 65536));
  hipLaunchKernelGGL(k_repack8_weights, dim3(blocks), dim3(256), 0, st, q, n, k, gate_up, reinterpret_cast<uint4*>(base));
  unsigned mblocks = unsigned(std::min<int64_t>((n * G + 255) / 256, 65536));
  hipLaunchKernelGGL(k_repack_meta, dim3(mblocks), dim3(256), 0, st, scales, nullptr, n, k, int(kGroup), gate_up,
                     reinterpret_cast<uint16_t*>(base + sb), nullptr);
  const int64_t scale_pad = align256(2 * n * G) - 2 * n * G;
  if (scale_pad > 0) hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(256), 0, st, base + sb + 2 * n * G, scale_pad);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* w, int dtype, int64_t n, int64_t k, int asym, uint8_t* packed,
                           uint16_t* scales, uint8_t* zeros, int32_t* flags, hipStream_t st) {
  const int64_t G = k / kGroup;
  dim3 grid(unsigned(n * ((G + 1) / 2)));
#define Q4_QLAUNCH(DT, AS) \
  hipLaunchKernelGGL((k_quantize_g128<DT, AS>), grid, dim3(64), 0, st, w, n, k, packed, scales, zeros, flags)
  if (asym) {
    if (dtype == 0) Q4_QLAUNCH(0, true);
    else if (dtype == 1) Q4_QLAUNCH(1, true);
    else Q4_QLAUNCH(2, true);
  } else {
    if (dtype == 0) Q4_QLAUNCH(0, false);
    else if (dtype == 1) Q4_QLAUNCH(1, false);
    else Q4_QLAUNCH(2, false);
  }
#undef Q4_QLAUNCH
  return hipGetLastError();
}

hipError_t launch_quantize_grouped(const void* w, int dtype, int64_t n, int64_t k, int group, int asym,
                                   uint8_t* packed, uint16_t* scales, uint8_t* zeros, int32_t* flags,
                                   hipStream_t st) {
  if (group == kGroup) return launch_quantize(w, dtype, n, k, asym, packed, scales, zeros, flags, st);
  const int64_t chunks = (k + 255) / 256;
  dim3 grid(unsigned(n * ((chunks + 1) / 2)));
#define Q4_QLAUNCH(DT, AS) \
  hipLaunchKernelGGL((k_quantize_grp<DT, AS>), grid, dim3(64), 0, st, w, n, k, group, packed, scales, zeros, flags)
  if (asym) {
    if (dtype == 0) Q4_QLAUNCH(0, true);
    else if (dtype == 1) Q4_QLAUNCH(1, true);
    else Q4_QLAUNCH(2, true);
  } else {
    if (dtype == 0) Q4_QLAUNCH(0, false);
    else if (dtype == 1) Q4_QLAUNCH(1, false);
    else Q4_QLAUNCH(2, false);
  }
#undef Q4_QLAUNCH
  return hipGetLastError();
}

hipError_t launch_repack(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros, int64_t n,
                         int64_t k, int asym, int gate_up, void* out, hipStream_t st, int group) {
  uint8_t* base = static_cast<uint8_t*>(out);
  const int64_t G = k / kGroup;
  const int64_t SG = group < kGroup ? kGroup / group : 1;
  const int64_t words = n * k / 8;
  const int64_t sb = align256(n * k / 2);
  const int64_t zb = sb + align256(2 * n * G * SG);
  unsigned blocks = unsigned(std::min<int64_t>((words + 255) / 256, 65536));
  hipLaunchKernelGGL(k_repack_weights, dim3(blocks), dim3(256), 0, st, packed, n, k, asym, gate_up,
                     reinterpret_cast<uint32_t*>(base));
  unsigned mblocks = unsigned(std::min<int64_t>((n * G * SG + 255) / 256, 65536));
  hipLaunchKernelGGL(k_repack_meta, dim3(mblocks), dim3(256), 0, st, scales, asym ? zeros : nullptr, n, k, group,
                     gate_up, reinterpret_cast<uint16_t*>(base + sb), asym ? base + zb : nullptr);
  const int64_t scale_pad = zb - (sb + 2 * n * G * SG);
  if (scale_pad > 0)
    hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(256), 0, st, base + sb + 2 * n * G * SG, scale_pad);
  if (asym) {
    const int64_t zero_pad = align256(n * G) - n * G;
    if (zero_pad > 0) hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(256), 0, st, base + zb + n * G, zero_pad);
  }
  return hipGetLastError();
}

}  // namespace q4
