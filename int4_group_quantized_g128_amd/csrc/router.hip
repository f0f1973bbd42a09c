// A3 router logits and A4 softmax + top-k.
//
// Page "大模型之Dense、MoE与量化", MoE section: a Linear layer scores the experts and
// a few are chosen; page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" §3.2:
// the router is kept in floating point (float32 here) rather than INT8.
#include "common.h"
#include "internal.h"

namespace q4 {

// Partial logits over K slices: a (16 TB)-token x (16 EB)-expert tile per wave, fp32
// MFMA 16x16x4.  Lane (m = lane % 16, kq = lane / 16) feeds x[t0 + 16 i + m][k] and
// W[e0 + 16 j + m][k] for k = k0 + 4 kq + s to MFMA s of each 16-wide K step; U steps
// of loads are issued before their MFMAs.  Batches below 512 tokens (or with fewer than
// 64 experts) run (16, 32 or 64) x 16 tiles and many K slices, with RED the workgroup's waves (up to
// 16) on consecutive slices whose sums are added in LDS (in wave order) so that one
// partial per workgroup is written; larger batches take the split-weight kernel below.
template <int TB, int EB, int U, bool RED>
__global__ void __launch_bounds__(RED ? 1024 : 64) k_router_partial(const uint16_t* __restrict__ x,
                                                                   const float* __restrict__ wr, int64_t t, int64_t h,
                                                                   int32_t e, int64_t kslice,
                                                                   float* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int kw = RED ? int(blockDim.x >> 6) : 1;
  const int m = lane & 15, kq = lane >> 4;
  const int64_t e0 = int64_t(blockIdx.x) * 16 * EB, t0 = int64_t(blockIdx.y) * 16 * TB;
  const int64_t ks = int64_t(blockIdx.z) * kw + wave;
  const int64_t kb = std::min<int64_t>(h, ks * kslice), ke = std::min<int64_t>(h, kb + kslice);
  const uint16_t* xr[TB];
  const float* wrow[EB];
  bool tv[TB], ev[EB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    tv[i] = t0 + 16 * i + m < t;
    xr[i] = x + (tv[i] ? t0 + 16 * i + m : 0) * h;
  }
#pragma unroll
  for (int j = 0; j < EB; ++j) {
    ev[j] = e0 + 16 * j + m < e;
    wrow[j] = wr + (ev[j] ? e0 + 16 * j + m : 0) * h;
  }
  f32x4_t acc[TB][EB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = kb; k0 < ke; k0 += 16 * U) {
    uint2 xv[U][TB];
    float4 wv[U][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + 16 * u + 4 * kq;
      const bool kv = k0 + 16 * u < ke;
#pragma unroll
      for (int i = 0; i < TB; ++i) xv[u][i] = (tv[i] && kv) ? load8(xr[i] + k) : make_uint2(0, 0);
#pragma unroll
      for (int j = 0; j < EB; ++j)
        wv[u][j] = (ev[j] && kv) ? *reinterpret_cast<const float4*>(wrow[j] + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xa[TB][4];
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        xa[i][0] = bf16_to_f32(uint16_t(xv[u][i].x & 0xffff));
        xa[i][1] = bf16_to_f32(uint16_t(xv[u][i].x >> 16));
        xa[i][2] = bf16_to_f32(uint16_t(xv[u][i].y & 0xffff));
        xa[i][3] = bf16_to_f32(uint16_t(xv[u][i].y >> 16));
      }
      // consecutive MFMAs go to different accumulators (no back-to-back dependency)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < TB; ++i)
#pragma unroll
          for (int j = 0; j < EB; ++j) {
            const float wq = q == 0 ? wv[u][j].x : q == 1 ? wv[u][j].y : q == 2 ? wv[u][j].z : wv[u][j].w;
            acc[i][j] = mfma_f32_16x16x4(xa[i][q], wq, acc[i][j]);
          }
    }
  }
  if constexpr (RED) {
    __shared__ f32x4_t red[15][TB * EB][64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) red[wave - 1][i * EB + j][lane] = acc[i][j];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 1; w < kw; ++w)
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) acc[i][j] += red[w - 1][i * EB + j][lane];
  }
  // C layout: lane holds tokens t0 + 16 i + 4 kq + r, expert e0 + 16 j + m
  const int64_t slot = blockIdx.z;
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tt = t0 + 16 * i + 4 * kq + r;
        if (tt < t && ev[j]) partial[(slot * t + tt) * e + e0 + 16 * j + m] = acc[i][j][r];
      }
}

// Large batches run the logits on the bf16 matrix cores at fp32 accuracy.  Each fp32
// weight w is split into three bf16 parts with w = hi + mid + lo: hi is w truncated to
// bf16, mid is (w - hi) truncated, lo is the rest truncated.  Both differences are exact
// in fp32 and the rest has at most eight significant bits, so the sum is exact (for
// |w| below about 2^-110 the last part can lose bits to underflow).  x is bf16 already,
// so every product of x with a part is exact, and the matrix core adds them in fp32.
// A non-finite w goes whole into hi (a NaN stays a NaN), with mid = lo = 0.
// w3 holds the parts as three consecutive [n] bf16 arrays; each thread splits 8 values.
__global__ void __launch_bounds__(256) k_router_split3(const float* __restrict__ w, int64_t n,
                                                       uint16_t* __restrict__ w3) {
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  const float4 a = *reinterpret_cast<const float4*>(w + i);
  const float4 b = *reinterpret_cast<const float4*>(w + i + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t part[3][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t hpart[3][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float x = v[2 * q + s];
      const uint32_t u = __float_as_uint(x);
      if (!__builtin_isfinite(x)) {
        hpart[0][s] = (u >> 16) | (x != x ? 0x40u : 0u);
        hpart[1][s] = 0;
        hpart[2][s] = 0;
      } else {
        const float r = x - __uint_as_float(u & 0xffff0000u);
        const uint32_t ru = __float_as_uint(r);
        const float r2 = r - __uint_as_float(ru & 0xffff0000u);
        hpart[0][s] = u >> 16;
        hpart[1][s] = ru >> 16;
        hpart[2][s] = __float_as_uint(r2) >> 16;
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) part[p][q] = hpart[p][0] | (hpart[p][1] << 16);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p)
    *reinterpret_cast<uint4*>(w3 + p * n + i) = make_uint4(part[p][0], part[p][1], part[p][2], part[p][3]);
}

// Partial logits from the split weights: a (16 TB)-token x (16 EB)-expert tile per
// wave, bf16 MFMA 16x16x32, one wave per K slice.  Lane (m = lane % 16, kq = lane / 16)
// feeds x[t0 + 16 i + m][k .. k + 7] and part p of W[e0 + 16 j + m][k .. k + 7] with
// k = k0 + 8 kq; each K step runs the three parts' MFMAs on one accumulator per tile
// (hi, then mid, then lo), U steps of loads issued before their MFMAs.  Rows past t or
// e and K past the slice load zeros for both operands.  Same partial layout as above.
// The grid is one-dimensional, a multiple of 8 workgroups: workgroup b runs on XCD
// b % 8 (round-robin dispatch), and each XCD takes one contiguous range of tiles in
// (slice, token block, expert block) order, so its L2 holds the weight parts of about
// one K slice for every expert block and each x block serves all expert blocks there.
template <int TB, int EB, int U>
__global__ void __launch_bounds__(64) k_router_x3(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w3,
                                                  int64_t t, int64_t h, int32_t e, int64_t kslice, int32_t neb,
                                                  int32_t ntb, int32_t nslices, float* __restrict__ partial) {
  const int lane = threadIdx.x;
  const int m = lane & 15, kq = lane >> 4;
  const int64_t chunk = gridDim.x / 8;
  const int64_t tile = int64_t(blockIdx.x % 8) * chunk + blockIdx.x / 8;
  if (tile >= int64_t(neb) * ntb * nslices) return;
  const int64_t eb = tile % neb, tb = (tile / neb) % ntb, slot = tile / (int64_t(neb) * ntb);
  const int64_t e0 = eb * 16 * EB, t0 = tb * 16 * TB;
  const int64_t kb = std::min<int64_t>(h, slot * kslice), ke = std::min<int64_t>(h, kb + kslice);
  const int64_t pn = int64_t(e) * h;   // elements from one part to the next
  const uint16_t* xr[TB];
  const uint16_t* wrow[EB];
  bool tv[TB], ev[EB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    tv[i] = t0 + 16 * i + m < t;
    xr[i] = x + (tv[i] ? t0 + 16 * i + m : 0) * h + 8 * kq;
  }
#pragma unroll
  for (int j = 0; j < EB; ++j) {
    ev[j] = e0 + 16 * j + m < e;
    wrow[j] = w3 + (ev[j] ? e0 + 16 * j + m : 0) * h + 8 * kq;
  }
  f32x4_t acc[TB][EB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int64_t k0 = kb; k0 < ke; k0 += 32 * U) {
    uint4 xv[U][TB];
    uint4 wv[U][3][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + 32 * u;
      const bool kv = k + 8 * kq < ke;   // ke and k are multiples of 16: all 8 or none
#pragma unroll
      for (int i = 0; i < TB; ++i) xv[u][i] = (tv[i] && kv) ? load16(xr[i] + k) : zero;
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < EB; ++j) wv[u][p][j] = (ev[j] && kv) ? load16(wrow[j] + p * pn + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int i = 0; i < TB; ++i)
#pragma unroll
          for (int j = 0; j < EB; ++j) {
            const u32x4_t av = {xv[u][i].x, xv[u][i].y, xv[u][i].z, xv[u][i].w};
            const u32x4_t bv = {wv[u][p][j].x, wv[u][p][j].y, wv[u][p][j].z, wv[u][p][j].w};
            acc[i][j] = mfma16x16x32<Act::BF16>(av, bv, acc[i][j]);
          }
  }
  #pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tt = t0 + 16 * i + 4 * kq + r;
        if (tt < t && ev[j]) partial[(slot * t + tt) * e + e0 + 16 * j + m] = acc[i][j][r];
      }
}

constexpr int kMaxSlices = 32;

// Tuning defaults, overridable at build time: token blocks of 16 per wave tile from
// 2048 tokens, and the waves the K slices aim for there (one per SIMD measured faster
// than two: 86 vs 87-119 us at 4096 tokens on the 256-expert router) and below it.
#ifndef Q4_ROUTE_HUGE_TB
#define Q4_ROUTE_HUGE_TB 8
#endif
#ifndef Q4_ROUTE_HUGE_WAVES
#define Q4_ROUTE_HUGE_WAVES 1024
#endif
#ifndef Q4_ROUTE_WAVES
#define Q4_ROUTE_WAVES 2048
#endif
// workgroups of the small-batch logit kernel to aim for (one per CU)
#ifndef Q4_ROUTE_WGS
#define Q4_ROUTE_WGS 256
#endif

// Unsigned image of a float that orders like the float (non-NaN inputs).
Q4_DEVICE uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
Q4_DEVICE float ordered_to_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// 64-bit maximum over the wave, in every lane: DPP exchanges inside each 16-lane row
// (lane ^ 1, lane ^ 2, then the 8- and 16-lane mirrors), then the four row results.
template <int CTRL>
Q4_DEVICE uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(x)), CTRL, 0xf, 0xf, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(x >> 32)), CTRL, 0xf, 0xf, false));
  return (uint64_t(hi) << 32) | lo;
}
Q4_DEVICE uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
Q4_DEVICE uint64_t wave_max_u64(uint64_t x) {
  x = max_u64(x, dpp_u64<0xb1>(x));    // quad_perm [1,0,3,2]
  x = max_u64(x, dpp_u64<0x4e>(x));    // quad_perm [2,3,0,1]
  x = max_u64(x, dpp_u64<0x141>(x));   // row_half_mirror
  x = max_u64(x, dpp_u64<0x140>(x));   // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(x), 16 * row);
    const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(x >> 32), 16 * row);
    m = max_u64(m, (uint64_t(hi) << 32) | lo);
  }
  return m;
}

// One wave per token: logits = sum of the K-slice partials in slice order + bias, then
// k rounds of a wave-wide arg-max of the key (larger logit, then lower index), then
// the renormalised softmax weights of the selected experts.  Lane l holds experts
// l + 64 i (i < NI, NI = ceil(e / 64)); the round winners go through LDS so that ids
// and weights are written once, coalesced.
template <int NI, int MS>
__global__ void __launch_bounds__(64) k_topk(const float* __restrict__ partial, int32_t kslices,
                                             const float* __restrict__ bias, int64_t t, int32_t e,
                                             int32_t k, float* __restrict__ logits, int32_t* __restrict__ ids,
                                             float* __restrict__ weights) {
  __shared__ int32_t s_id[64 * NI];
  __shared__ float s_w[64 * NI];
  const int lane = threadIdx.x;
  const int64_t tok = blockIdx.x;
  float v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) v[i] = 0.f;
  // slice sums in slice order (0 + p0 = p0 exactly); addresses clamped into range
  int ks = 0;
  if constexpr (NI <= 4) {
    // every partial load in flight at once (MS >= kslices; clamped slice index, unused
    // slices add 0)
    float p[MS][NI];
#pragma unroll
    for (int u = 0; u < MS; ++u)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        p[u][i] = partial[(int64_t(min(u, kslices - 1)) * t + tok) * e + min(lane + 64 * i, e - 1)];
#pragma unroll
    for (int u = 0; u < MS; ++u)
#pragma unroll
      for (int i = 0; i < NI; ++i) v[i] += u < kslices ? p[u][i] : 0.f;
    ks = kslices;
  }
  for (; ks + 4 <= kslices; ks += 4) {
    float p[4][NI];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        p[u][i] = partial[(int64_t(ks + u) * t + tok) * e + min(lane + 64 * i, e - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NI; ++i) v[i] += p[u][i];
  }
  for (; ks < kslices; ++ks)
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] += partial[(int64_t(ks) * t + tok) * e + min(lane + 64 * i, e - 1)];
  // selection key: larger logit first, then lower expert index (0 = taken / absent)
  uint64_t key[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ex = lane + 64 * i;
    if (ex < e) {
      if (bias) v[i] += bias[ex];
      logits[tok * e + ex] = v[i];
      if (v[i] != v[i]) v[i] = -__builtin_inff();  // NaN never wins; every id stays in range
      // -0 keyed as +0: equal logits tie on the index alone
      key[i] = (uint64_t(ordered_bits(v[i] == 0.f ? 0.f : v[i])) << 32) | uint32_t(~uint32_t(ex));
    } else {
      key[i] = 0;
    }
  }
  float lmax = 0.f, denom = 0.f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NI; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int bi = int(~uint32_t(best));
    const float bv = ordered_to_float(uint32_t(best >> 32));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (bi == lane + 64 * i) key[i] = 0;
    if (r == 0) lmax = bv;
    const float ex = expf(bv - lmax);   // the same in every lane
    denom += ex;
    if (lane == 0) {
      s_id[r] = bi;
      s_w[r] = ex;
    }
  }
  __syncthreads();
  for (int r = lane; r < k; r += 64) {
    ids[tok * k + r] = s_id[r];
    weights[tok * k + r] = __fdiv_rn(s_w[r], denom);
  }
}

// Wave tile of the partial-logit kernel: 16 x 16 for small batches (fp32 matrix
// cores); with enough tiles to fill the chip without splitting K much, the split-weight
// kernel with 32 tokens x 64 experts, and from 2048 tokens 16 Q4_ROUTE_HUGE_TB tokens.
static bool route_big_tiles(int64_t t, int32_t e) { return t >= 512 && e >= 64; }
static bool route_huge_tiles(int64_t t, int32_t e) { return t >= 2048 && e >= 64; }

// K slices: enough waves to cover the chip (about 2048; 1024 from 2048 tokens), at
// least 256 of K per slice, at most kMaxSlices partial sums.
// Token blocks of 16 per wave tile of the small-batch kernel.  With 16-token tiles each
// router weight row is re-read by every token tile; from 65 tokens (64 experts or more)
// two or four token blocks per tile read it half or a quarter as often (router + top-k
// per call, 256 experts: T = 96 / 128 23.6 / 22.8 -> 16.9 / 18.3 us with two, T = 192 /
// 256 / 384 34.5 / 37.9 / 62.3 -> 24.0 / 26.8 / 49.1 us with four; T = 64 and the
// 8-expert router, whose weights are 64 KB, stay fastest with one).
static int small_tb(int64_t t, int32_t e) {
  if (e < 64 || t <= 64) return 1;
  return t < 160 ? 2 : 4;
}
int route_kslices(int64_t t, int64_t h, int32_t e) {
  constexpr int64_t hrows = 16 * Q4_ROUTE_HUGE_TB;
  const int64_t srows = 16 * small_tb(t, e);
  const bool huge = route_huge_tiles(t, e);
  const int64_t tiles = huge                    ? ((e + 63) / 64) * ((t + hrows - 1) / hrows)
                        : route_big_tiles(t, e) ? ((e + 63) / 64) * ((t + 31) / 32)
                                                : ((e + 15) / 16) * ((t + srows - 1) / srows);
  const int64_t waves = huge ? Q4_ROUTE_HUGE_WAVES : Q4_ROUTE_WAVES;
  int64_t ks = (waves + tiles - 1) / tiles;
  ks = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(ks, h / 256), kMaxSlices));
  return int(ks);
}

// One wave per token; up to 8 or 16 partial sums are all loaded by variants sized for them.
template <int NI>
static hipError_t launch_topk(const float* partial, int nparts, const float* bias, int64_t t, int32_t e, int32_t k,
                              float* logits, int32_t* ids, float* w, hipStream_t st) {
  if constexpr (NI <= 4) {
    if (nparts <= 8) {
      hipLaunchKernelGGL((k_topk<NI, 8>), dim3(unsigned(t)), dim3(64), 0, st, partial, nparts, bias, t, e, k, logits,
                         ids, w);
      return hipGetLastError();
    }
    if (nparts <= 16) {
      hipLaunchKernelGGL((k_topk<NI, 16>), dim3(unsigned(t)), dim3(64), 0, st, partial, nparts, bias, t, e, k, logits,
                         ids, w);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_topk<NI, kMaxSlices>), dim3(unsigned(t)), dim3(64), 0, st, partial, nparts, bias, t, e, k,
                     logits, ids, w);
  return hipGetLastError();
}

// Bytes of the partial sums, and with the split weights of large batches (the big
// tiles) behind them at the next 256-byte boundary.
static size_t route_partial_bytes(int64_t t, int64_t h, int32_t e) {
  return size_t(route_kslices(t, h, e)) * size_t(t) * size_t(e) * sizeof(float);
}
size_t route_workspace_bytes(int64_t t, int64_t h, int32_t e) {
  const size_t p = route_partial_bytes(t, h, e);
  if (!route_big_tiles(t, e)) return p;
  return (p + 255) / 256 * 256 + 3 * size_t(e) * size_t(h) * sizeof(uint16_t);
}

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int64_t t, int64_t h,
                        int32_t e, int32_t k, float* logits, int32_t* ids, float* w, float* partial,
                        hipStream_t st) {
  const bool x3 = route_big_tiles(t, e);
  const int ks = route_kslices(t, h, e);
  const int64_t kalign = x3 ? 32 : 16;   // the K step of the logit kernel
  int64_t kslice = (h + ks - 1) / ks;
  kslice = (kslice + kalign - 1) / kalign * kalign;
  const int kused = int((h + kslice - 1) / kslice);
  int nparts = kused;   // partial sums written (one per K slice, or per workgroup of slices)
  if (x3) {
    uint16_t* w3 = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(partial) +
                                               (route_partial_bytes(t, h, e) + 255) / 256 * 256);
    const int64_t n = int64_t(e) * h;
    hipLaunchKernelGGL(k_router_split3, dim3(unsigned((n / 8 + 255) / 256)), dim3(256), 0, st, wr, n, w3);
    if (route_huge_tiles(t, e)) {
      constexpr int TB = Q4_ROUTE_HUGE_TB;
      const int neb = int((e + 63) / 64), ntb = int((t + 16 * TB - 1) / (16 * TB));
      const dim3 grid(unsigned((int64_t(neb) * ntb * kused + 7) / 8 * 8));
      hipLaunchKernelGGL((k_router_x3<TB, 4, 1>), grid, dim3(64), 0, st, x, w3, t, h, e, kslice, neb, ntb, kused,
                         partial);
    } else {
      const int neb = int((e + 63) / 64), ntb = int((t + 31) / 32);
      const dim3 grid(unsigned((int64_t(neb) * ntb * kused + 7) / 8 * 8));
      hipLaunchKernelGGL((k_router_x3<2, 4, 2>), grid, dim3(64), 0, st, x, w3, t, h, e, kslice, neb, ntb, kused,
                         partial);
    }
  } else {
    // about one workgroup per CU: the slices of a tile are shared out over
    // Q4_ROUTE_WGS / tiles workgroups (at least one), at most 16 waves each
    const int tb = small_tb(t, e);
    const int64_t tiles = int64_t((e + 15) / 16) * ((t + 16 * tb - 1) / (16 * tb));
    const int want = int(std::max<int64_t>(1, std::min<int64_t>(kused, Q4_ROUTE_WGS / tiles)));
    const int kw = std::min(16, (kused + want - 1) / want);
    nparts = (kused + kw - 1) / kw;
    dim3 grid(unsigned((e + 15) / 16), unsigned((t + 16 * tb - 1) / (16 * tb)), unsigned(nparts));
    if (tb == 4)   // (fewer steps per load batch: the registers of four token blocks)
      hipLaunchKernelGGL((k_router_partial<4, 1, 4, true>), grid, dim3(64 * kw), 0, st, x, wr, t, h, e, kslice,
                         partial);
    else if (tb == 2)
      hipLaunchKernelGGL((k_router_partial<2, 1, 8, true>), grid, dim3(64 * kw), 0, st, x, wr, t, h, e, kslice,
                         partial);
    else
      hipLaunchKernelGGL((k_router_partial<1, 1, 16, true>), grid, dim3(64 * kw), 0, st, x, wr, t, h, e, kslice,
                         partial);
  }
  if (e <= 64) return launch_topk<1>(partial, nparts, bias, t, e, k, logits, ids, w, st);
  if (e <= 128) return launch_topk<2>(partial, nparts, bias, t, e, k, logits, ids, w, st);
  if (e <= 256) return launch_topk<4>(partial, nparts, bias, t, e, k, logits, ids, w, st);
  if (e <= 512) return launch_topk<8>(partial, nparts, bias, t, e, k, logits, ids, w, st);
  return launch_topk<16>(partial, nparts, bias, t, e, k, logits, ids, w, st);
}

}  // namespace q4
