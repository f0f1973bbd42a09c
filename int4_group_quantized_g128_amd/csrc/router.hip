// A3 router logits and A4 softmax + top-k.
//
// Page "大模型之Dense、MoE与量化", MoE section: a Linear layer scores the experts and
// a few are chosen; page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" §3.2:
// the router is kept in floating point (float32 here) rather than INT8.
#include "common.h"
#include "internal.h"

namespace q4 {

// Partial logits over one K slice: a 16-token x 16-expert tile per wave, fp32 MFMA
// 16x16x4.  Lane (m = lane % 16, kq = lane / 16) feeds x[t0 + m][k0 + 4 kq + j] and
// W[e0 + m][k0 + 4 kq + j] to MFMA j of each 16-wide K step; 8 steps of loads are
// issued before their MFMAs.
constexpr int kRouteUnroll = 8;

__global__ void __launch_bounds__(64) k_router_partial(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                       int64_t t, int64_t h, int32_t e, int64_t kslice,
                                                       float* __restrict__ partial) {
  const int lane = threadIdx.x;
  const int m = lane & 15, kq = lane >> 4;
  const int64_t e0 = int64_t(blockIdx.x) * 16, t0 = int64_t(blockIdx.y) * 16;
  const int64_t ks = blockIdx.z;
  const int64_t kb = ks * kslice, ke = std::min<int64_t>(h, kb + kslice);
  const bool tv = t0 + m < t, ev = e0 + m < e;
  const uint16_t* xr = x + (tv ? t0 + m : 0) * h;
  const float* wrow = wr + (ev ? e0 + m : 0) * h;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = kb; k0 < ke; k0 += 16 * kRouteUnroll) {
    uint2 xv[kRouteUnroll];
    float4 wv[kRouteUnroll];
#pragma unroll
    for (int u = 0; u < kRouteUnroll; ++u) {
      const int64_t k = k0 + 16 * u + 4 * kq;
      const bool kv = k0 + 16 * u < ke;
      xv[u] = (tv && kv) ? load8(xr + k) : make_uint2(0, 0);
      wv[u] = (ev && kv) ? *reinterpret_cast<const float4*>(wrow + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kRouteUnroll; ++u) {
      acc = mfma_f32_16x16x4(bf16_to_f32(uint16_t(xv[u].x & 0xffff)), wv[u].x, acc);
      acc = mfma_f32_16x16x4(bf16_to_f32(uint16_t(xv[u].x >> 16)), wv[u].y, acc);
      acc = mfma_f32_16x16x4(bf16_to_f32(uint16_t(xv[u].y & 0xffff)), wv[u].z, acc);
      acc = mfma_f32_16x16x4(bf16_to_f32(uint16_t(xv[u].y >> 16)), wv[u].w, acc);
    }
  }
  // C layout: lane holds tokens t0 + 4 kq + i, expert e0 + m
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tt = t0 + 4 * kq + i;
    if (tt < t && ev) partial[(ks * t + tt) * e + e0 + m] = acc[i];
  }
}

constexpr int kMaxSlices = 32;

// One wave per token: logits = sum of the K-slice partials in slice order + bias, then
// k rounds of a wave-wide arg-max with the key (larger logit, then lower index), then
// the renormalised softmax weights of the selected experts.
__global__ void __launch_bounds__(64) k_topk(const float* __restrict__ partial, int32_t kslices,
                                             const float* __restrict__ bias, int64_t t, int32_t e,
                                             int32_t k, float* __restrict__ logits, int32_t* __restrict__ ids,
                                             float* __restrict__ weights) {
  constexpr int kMaxPerLane = 16;  // e <= 1024
  const int lane = threadIdx.x;
  const int64_t tok = blockIdx.x;
  float v[kMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int ex = lane + 64 * i;
    float s = -__builtin_inff();
    if (ex < e) {
      // all slice loads in flight, then summed in slice order
      float pv[kMaxSlices];
#pragma unroll
      for (int ks = 0; ks < kMaxSlices; ++ks) pv[ks] = ks < kslices ? partial[(int64_t(ks) * t + tok) * e + ex] : 0.f;
      s = pv[0];
#pragma unroll
      for (int ks = 1; ks < kMaxSlices; ++ks)
        if (ks < kslices) s += pv[ks];
      if (bias) s += bias[ex];
      logits[tok * e + ex] = s;
      if (s != s) s = -__builtin_inff();  // NaN never wins; every id stays in range
    } else {
      taken |= 1u << i;
    }
    v[i] = s;
  }
  float lmax = 0.f, denom = 0.f;
  for (int r = 0; r < k; ++r) {
    // local best among not-taken entries
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int ex = lane + 64 * i;
      if (!(taken & (1u << i)) && (v[i] > bv || (v[i] == bv && ex < bi))) {
        bv = v[i];
        bi = ex;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      ids[tok * k + r] = bi;
      if (r == 0) lmax = bv;
      const float ex = expf(bv - lmax);
      denom += ex;
      weights[tok * k + r] = ex;  // normalised below
    }
  }
  if (lane == 0) {
    for (int r = 0; r < k; ++r) weights[tok * k + r] = __fdiv_rn(weights[tok * k + r], denom);
  }
}

int route_kslices(int64_t t, int64_t h, int32_t e) {
  const int64_t tiles = ((e + 15) / 16) * ((t + 15) / 16);
  int64_t ks = (1024 + tiles - 1) / tiles;
  ks = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(ks, h / 256), kMaxSlices));
  return int(ks);
}

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int64_t t, int64_t h,
                        int32_t e, int32_t k, float* logits, int32_t* ids, float* w, float* partial,
                        hipStream_t st) {
  const int ks = route_kslices(t, h, e);
  int64_t kslice = (h + ks - 1) / ks;
  kslice = (kslice + 15) / 16 * 16;
  const int kused = int((h + kslice - 1) / kslice);
  dim3 grid(unsigned((e + 15) / 16), unsigned((t + 15) / 16), unsigned(kused));
  hipLaunchKernelGGL(k_router_partial, grid, dim3(64), 0, st, x, wr, t, h, e, kslice, partial);
  hipLaunchKernelGGL(k_topk, dim3(unsigned(t)), dim3(64), 0, st, partial, kused, bias, t, e, k, logits, ids, w);
  return hipGetLastError();
}

}  // namespace q4
