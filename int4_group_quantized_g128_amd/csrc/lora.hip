// LoRA-mode experts: per-expert low-rank adapters on one frozen INT4 g128 dense FFN.
//
// Page "高效大语言模型推理实践：INT4量化与MoE架构的融合探索", 第三阶段 (LoRA mode:
// experts start from LoRA adapters on frozen dense weights); expert e of matrix m is
// W_hat_m + B_m,e A_m,e.  The forward uses two exact identities of that definition:
//  - gate/up: (W_hat + B A) x = W_hat x + B (A x), so the INT4 base GEMM runs once per
//    token and every (token, choice) slot adds a rank-r update;
//  - down is linear: sum_j w_j (W_hat + B_j A_j) h_j = W_hat (sum_j w_j h_j)
//    + sum_j w_j B_j (A_j h_j), so the INT4 base down GEMM also runs once per token.
// Kernels here: the rank-r input projections (k_lora_in), SwiGLU + weighted sum + the
// down-adapter input projection (k_lora_mid), the final combine (k_lora_out), and the
// row-tile list of a dense matrix for the prefill GEMM (k_dense_tiles).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace q4 {

__global__ void k_dense_tiles(int64_t t, int tile_rows, TileDesc* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  const int64_t n = (t + tile_rows - 1) / tile_rows;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i == 0) *num_tiles = int32_t(n);
  if (i < n) {
    TileDesc d;
    d.expert = 0;
    d.row_start = int32_t(i * tile_rows);
    d.rows = int32_t(std::min<int64_t>(tile_rows, t - i * tile_rows));
    d.pad = 0;
    tiles[i] = d;
  }
}

Q4_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Partial input projections: a_part[p][ks][q] = sum_{k in chunk ks} A_e[q][k] x_t[k]
// (q < 2R: A_gate,e rows then A_up,e rows) for slot p = t * kk + j, e = ids[p], and
// the 512-wide K chunk ks (one wave per (slot, chunk); lane l covers k = 512 ks + 8 l
// .. + 7).  The 64 lane partials of each q are summed in lane order through LDS.  The
// rank R is a template argument, so every adapter load of a lane is issued at once.
template <int R>
__global__ void __launch_bounds__(64) k_lora_in(const uint16_t* __restrict__ x, int64_t h, const int32_t* __restrict__ ids,
                                                int32_t kk, int32_t e_count, const uint16_t* __restrict__ a_gu,
                                                float* __restrict__ a_part) {
  constexpr int R2 = 2 * R;
  __shared__ float part[R2][65];
  const int lane = threadIdx.x;
  const int64_t p = blockIdx.x, ks = blockIdx.y, nks = gridDim.y;
  const int64_t t = p / kk;
  const int e = min(max(ids[p], 0), e_count - 1);
  const int64_t k0 = ks * 512 + int64_t(lane) * 8;
  float acc[R2];
#pragma unroll
  for (int q = 0; q < R2; ++q) acc[q] = 0.f;
  if (k0 < h) {
    const uint4 xv = load16(x + t * h + k0);
    uint4 av[R2];
#pragma unroll
    for (int q = 0; q < R2; ++q) av[q] = load16(a_gu + (int64_t(e) * R2 + q) * h + k0);
    float xf[8];
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[2 * i] = bf16_to_f32(uint16_t(xw[i] & 0xffff));
      xf[2 * i + 1] = bf16_to_f32(uint16_t(xw[i] >> 16));
    }
#pragma unroll
    for (int q = 0; q < R2; ++q) {
      const uint32_t aw[4] = {av[q].x, av[q].y, av[q].z, av[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[q] = fmaf(bf16_to_f32(uint16_t(aw[i] & 0xffff)), xf[2 * i], acc[q]);
        acc[q] = fmaf(bf16_to_f32(uint16_t(aw[i] >> 16)), xf[2 * i + 1], acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < R2; ++q) part[q][lane] = acc[q];
  __syncthreads();
  for (int q = lane; q < R2; q += 64) {   // 2R can exceed the 64 lanes
    float s = 0.f;
    for (int l = 0; l < 64; ++l) s += part[q][l];
    a_part[(p * nks + ks) * R2 + q] = s;
  }
}

// Column block cb of token t (256 threads; thread tid owns columns
// c_i = 1024 cb + tid + 256 i, i < 4): for each choice j (expert e, weight w_j, slot p),
// with a = sum over K chunks of a_part[p] (in order):
//   g_c = base_gu[t][c] + sum_q B_gate,e[c][q] a[q]
//   u_c = base_gu[t][I + c] + sum_q B_up,e[c][q] a[R + q]
//   h_c = silu(g_c) u_c;  hw_c += w_j h_c;  d_part[p][cb][q] = sum_{c in block} A_down,e[q][c] h_c
// then hw[t][c] = bf16(hw_c).  With consecutive columns on consecutive lanes, one
// 16-byte load of a wave covers R / 8 * 64 * 16 bytes of B rows (16 cache lines at
// R = 16, not 64 as with four consecutive columns per lane).  A thread's adapter rows
// are all loaded before any is used; columns past I load the last column (in bounds)
// and are masked.
constexpr int kMidNC = 4;                // columns per thread (measured faster than 1 or 2)
constexpr int kMidCols = 256 * kMidNC;   // columns per workgroup
template <int R>
__global__ void __launch_bounds__(256) k_lora_mid(const float* __restrict__ base_gu, int64_t inter,
                                                  const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                  int32_t kk, int32_t e_count, int nks,
                                                  const float* __restrict__ a_part, const uint16_t* __restrict__ b_gate,
                                                  const uint16_t* __restrict__ b_up, const uint16_t* __restrict__ a_down,
                                                  float* __restrict__ d_part, uint16_t* __restrict__ hw) {
  __shared__ float s_a[2 * R];
  __shared__ float s_red[4][R];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t t = blockIdx.y, cb = blockIdx.x, ncb = gridDim.x;
  int64_t col[kMidNC];   // clamped into [0, inter)
  bool cv[kMidNC];
#pragma unroll
  for (int i = 0; i < kMidNC; ++i) {
    const int64_t c = cb * kMidCols + tid + 256 * i;
    cv[i] = c < inter;
    col[i] = cv[i] ? c : inter - 1;
  }
  float hacc[kMidNC], g0[kMidNC], u0[kMidNC];
#pragma unroll
  for (int i = 0; i < kMidNC; ++i) {
    hacc[i] = 0.f;
    g0[i] = base_gu[t * 2 * inter + col[i]];
    u0[i] = base_gu[t * 2 * inter + inter + col[i]];
  }
  for (int j = 0; j < kk; ++j) {
    const int64_t p = t * kk + j;
    const int e = min(max(ids[p], 0), e_count - 1);
    const float wj = w[p];
    // adapter loads first (they do not depend on s_a): the B rows of CB columns and QB
    // rows of A_down at a time, all of a batch issued together (every batch at once for
    // R <= 16; larger ranks keep the registers within bounds)
    constexpr int CB = R <= 16 ? kMidNC : R <= 32 ? (kMidNC >= 2 ? 2 : 1) : 1;
    constexpr int QB = R <= 16 ? R : R % 16 == 0 ? 16 : 8;   // divides R
    static_assert(R % QB == 0 && kMidNC % CB == 0, "load batches must tile the rows and columns");
    const uint16_t* bg = b_gate + int64_t(e) * inter * R;
    const uint16_t* bu = b_up + int64_t(e) * inter * R;
    const uint16_t* ad = a_down + int64_t(e) * R * inter;
    uint4 vg[CB][R / 8], vu[CB][R / 8];
    uint16_t va[QB][kMidNC];
    auto load_b = [&](int i0) {
#pragma unroll
      for (int i = 0; i < CB; ++i)
#pragma unroll
        for (int q8 = 0; q8 < R / 8; ++q8) {
          vg[i][q8] = load16(bg + col[i0 + i] * R + 8 * q8);
          vu[i][q8] = load16(bu + col[i0 + i] * R + 8 * q8);
        }
    };
    auto load_a = [&](int q0) {
#pragma unroll
      for (int q = 0; q < QB; ++q)
#pragma unroll
        for (int i = 0; i < kMidNC; ++i) va[q][i] = ad[int64_t(q0 + q) * inter + col[i]];
    };
    load_b(0);
    load_a(0);
    __syncthreads();   // s_a / s_red of the previous choice are consumed
    if (tid < 2 * R) {
      float s = 0.f;
      for (int ks = 0; ks < nks; ++ks) s += a_part[(p * nks + ks) * 2 * R + tid];
      s_a[tid] = s;
    }
    __syncthreads();
    float dp[R];
#pragma unroll
    for (int q = 0; q < R; ++q) dp[q] = 0.f;
    float hv[kMidNC];
#pragma unroll
    for (int i0 = 0; i0 < kMidNC; i0 += CB) {
      if (i0 > 0) load_b(i0);
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        float g = g0[i0 + i], u = u0[i0 + i];
#pragma unroll
        for (int q8 = 0; q8 < R / 8; ++q8) {
          const uint32_t wg[4] = {vg[i][q8].x, vg[i][q8].y, vg[i][q8].z, vg[i][q8].w};
          const uint32_t wu[4] = {vu[i][q8].x, vu[i][q8].y, vu[i][q8].z, vu[i][q8].w};
#pragma unroll
          for (int z = 0; z < 4; ++z) {
            g = fmaf(bf16_to_f32(uint16_t(wg[z] & 0xffff)), s_a[8 * q8 + 2 * z], g);
            g = fmaf(bf16_to_f32(uint16_t(wg[z] >> 16)), s_a[8 * q8 + 2 * z + 1], g);
            u = fmaf(bf16_to_f32(uint16_t(wu[z] & 0xffff)), s_a[R + 8 * q8 + 2 * z], u);
            u = fmaf(bf16_to_f32(uint16_t(wu[z] >> 16)), s_a[R + 8 * q8 + 2 * z + 1], u);
          }
        }
        hv[i0 + i] = swiglu(g, u);
        hacc[i0 + i] = fmaf(wj, hv[i0 + i], hacc[i0 + i]);
      }
    }
#pragma unroll
    for (int q0 = 0; q0 < R; q0 += QB) {
      if (q0 > 0) load_a(q0);
#pragma unroll
      for (int q = 0; q < QB; ++q)
#pragma unroll
        for (int i = 0; i < kMidNC; ++i)
          if (cv[i]) dp[q0 + q] = fmaf(bf16_to_f32(va[q][i]), hv[i], dp[q0 + q]);
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float s = wave_sum(dp[q]);
      if (lane == 0) s_red[wid][q] = s;
    }
    __syncthreads();
    if (tid < R) d_part[(p * ncb + cb) * R + tid] = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
  }
#pragma unroll
  for (int i = 0; i < kMidNC; ++i)
    if (cv[i]) hw[t * inter + col[i]] = f32_to_bf16(hacc[i]);
}

// Large batches, grouped by expert: the routed slots sorted by expert (the permutation's
// row tiles of at most 64 slots), a workgroup per (tile, 256 columns).  Each thread owns
// one column: it loads that column's B_gate / B_up rows once for the whole tile (the
// token-major kernel above reloads them for every slot), and for every slot of the tile
// forms g, u and h with the same arithmetic as that kernel, writing h per slot.  The
// down-adapter input projection d[slot][q] = sum_c A_down,e[q][c] h[slot][c] over the
// workgroup's columns is a 16 x R x 256 fp32 matrix-core product per 16 slots (each
// wave a quarter of the columns, the four partials added in wave order).  hw (the
// weighted sum over a token's choices) is formed afterwards by k_lora_hsum.
constexpr int kGrpCols = 256;    // columns per workgroup
constexpr int kGrpSlots = 64;    // slots per tile (the permutation's tile rows)
template <int R>
__global__ void __launch_bounds__(256) k_lora_mid_grp(const float* __restrict__ base_gu, int64_t inter,
                                                      const int32_t* __restrict__ perm,
                                                      const TileDesc* __restrict__ tiles,
                                                      const int32_t* __restrict__ num_tiles, int32_t kk, int nks,
                                                      const float* __restrict__ a_part,
                                                      const uint16_t* __restrict__ b_gate,
                                                      const uint16_t* __restrict__ b_up,
                                                      const uint16_t* __restrict__ a_down, float* __restrict__ d_part,
                                                      float* __restrict__ h_slot) {
  static_assert(R % 16 == 0 && R <= 32, "rank: 16 or 32");
  __shared__ float s_a[kGrpSlots][2 * R];
  __shared__ float s_h[16][kGrpCols + 1];
  __shared__ float s_ad[R][kGrpCols + 1];
  __shared__ f32x4_t s_dred[4][R / 16][64];
  __shared__ int32_t s_slot[kGrpSlots];
  if (int(blockIdx.y) >= *num_tiles) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int m = lane & 15, kq = lane >> 4;
  const int64_t cb = blockIdx.x, ncb = gridDim.x;
  const TileDesc td = tiles[blockIdx.y];
  const int e = td.expert, rows = td.rows;
  const int64_t p0 = td.row_start;
  const int64_t c = cb * kGrpCols + tid;
  const bool cv = c < inter;
  const int64_t cc = cv ? c : inter - 1;   // columns past I load the last one, masked
  // this column's adapter rows, loaded once for the tile
  float bg[R], bu[R];
#pragma unroll
  for (int q8 = 0; q8 < R / 8; ++q8) {
    const uint4 vg = load16(b_gate + (int64_t(e) * inter + cc) * R + 8 * q8);
    const uint4 vu = load16(b_up + (int64_t(e) * inter + cc) * R + 8 * q8);
    const uint32_t wg[4] = {vg.x, vg.y, vg.z, vg.w}, wu[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      bg[8 * q8 + 2 * z] = bf16_to_f32(uint16_t(wg[z] & 0xffff));
      bg[8 * q8 + 2 * z + 1] = bf16_to_f32(uint16_t(wg[z] >> 16));
      bu[8 * q8 + 2 * z] = bf16_to_f32(uint16_t(wu[z] & 0xffff));
      bu[8 * q8 + 2 * z + 1] = bf16_to_f32(uint16_t(wu[z] >> 16));
    }
  }
#pragma unroll
  for (int q = 0; q < R; ++q)
    s_ad[q][tid] = cv ? bf16_to_f32(a_down[(int64_t(e) * R + q) * inter + cc]) : 0.f;
  if (tid < rows) s_slot[tid] = perm[p0 + tid];
  // the slots' input projections: the sum of their K-chunk partials, in chunk order
  for (int idx = tid; idx < rows * 2 * R; idx += 256) {
    const int i = idx / (2 * R), q = idx - i * 2 * R;
    const int64_t sl = perm[p0 + i];
    float sum = 0.f;
    for (int ks = 0; ks < nks; ++ks) sum += a_part[(sl * nks + ks) * 2 * R + q];
    s_a[i][q] = sum;
  }
  __syncthreads();
  // the base gate/up values of 16 slots, all loads in flight together; the next 16
  // slots' loads are issued before the current ones are computed
  float g0[16], u0[16], g1[16], u1[16];
  auto load_base = [&](int i0, float (&g)[16], float (&u)[16]) {
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int i = min(i0 + ii, rows - 1);
      const int64_t t = s_slot[i] / kk;
      g[ii] = base_gu[t * 2 * inter + cc];
      u[ii] = base_gu[t * 2 * inter + inter + cc];
    }
  };
  load_base(0, g0, u0);
  for (int i0 = 0; i0 < rows; i0 += 16) {
    if (i0 + 16 < rows) load_base(i0 + 16, g1, u1);
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int i = i0 + ii;
      float hv = 0.f;
      if (i < rows) {
        const int64_t sl = s_slot[i];
        float g = g0[ii], u = u0[ii];
#pragma unroll
        for (int q = 0; q < R; ++q) g = fmaf(bg[q], s_a[i][q], g);
#pragma unroll
        for (int q = 0; q < R; ++q) u = fmaf(bu[q], s_a[i][R + q], u);
        hv = swiglu(g, u);
        if (cv) h_slot[sl * inter + c] = hv;
      }
      s_h[ii][tid] = cv ? hv : 0.f;
    }
    __syncthreads();
    // D[slot ii][q] over this wave's 64 columns: lane (m, kq) feeds s_h[m][k] and
    // s_ad[16 nb + m][k] for k = 64 wid + 4 st + kq to MFMA st
#pragma unroll
    for (int nb = 0; nb < R / 16; ++nb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int k = 64 * wid + 4 * st + kq;
        acc = mfma_f32_16x16x4(s_h[m][k], s_ad[16 * nb + m][k], acc);
      }
      s_dred[wid][nb][lane] = acc;
    }
    __syncthreads();
    // C layout: lane (m, kq) element r holds slot 4 kq + r, q = 16 nb + m
    for (int o = tid; o < 16 * R; o += 256) {
      const int ii = o / R, q = o - ii * R;
      if (i0 + ii >= rows) continue;
      const int nb = q / 16, l = 16 * (ii / 4) + (q % 16), r = ii % 4;
      const float v = ((s_dred[0][nb][l][r] + s_dred[1][nb][l][r]) + s_dred[2][nb][l][r]) + s_dred[3][nb][l][r];
      d_part[(int64_t(s_slot[i0 + ii]) * ncb + cb) * R + q] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      g0[ii] = g1[ii];
      u0[ii] = u1[ii];
    }
  }
}

// hw[t][c] = bf16( sum_j w[t][j] h[t kk + j][c] ), choices in order from 0 (the
// token-major kernel's own accumulation); four columns per thread.  rs (optional): the
// row sums of hw per group of 128 columns (the down projection's prefill kernel takes
// them), summed over the group's 32 threads in a fixed tree.
__global__ void __launch_bounds__(256) k_lora_hsum(const float* __restrict__ h_slot, const float* __restrict__ w,
                                                   int64_t t, int32_t kk, int64_t inter, uint16_t* __restrict__ hw,
                                                   float* __restrict__ rs) {
  const int64_t per = inter / 4;   // a multiple of 32: a group's 32 threads share a wave half
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= t * per) return;
  const int64_t tok = i / per, c = (i - tok * per) * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < kk; ++j) {
    const int64_t sl = tok * kk + j;
    const float wj = w[sl];
    const float4 v = *reinterpret_cast<const float4*>(h_slot + sl * inter + c);
    a0 = fmaf(wj, v.x, a0);
    a1 = fmaf(wj, v.y, a1);
    a2 = fmaf(wj, v.z, a2);
    a3 = fmaf(wj, v.w, a3);
  }
  const uint16_t b0 = f32_to_bf16(a0), b1 = f32_to_bf16(a1), b2 = f32_to_bf16(a2), b3 = f32_to_bf16(a3);
  const uint32_t lo = uint32_t(b0) | (uint32_t(b1) << 16);
  const uint32_t hi = uint32_t(b2) | (uint32_t(b3) << 16);
  *reinterpret_cast<uint2*>(hw + tok * inter + c) = make_uint2(lo, hi);
  if (rs) {
    float s = ((bf16_to_f32(b0) + bf16_to_f32(b1)) + bf16_to_f32(b2)) + bf16_to_f32(b3);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) s += __shfl_xor(s, o, 32);
    if ((threadIdx.x & 31) == 0) rs[tok * (inter / 128) + c / 128] = s;
  }
}

// out[t][c] = bf16( y[t][c] + sum_j w_j sum_q B_down,e_j[c][q] d[t kk + j][q] ), d the
// sum over column blocks of d_part (in order).
template <int R>
__global__ void __launch_bounds__(256) k_lora_out(const float* __restrict__ y, int64_t hidden,
                                                  const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                  int32_t kk, int32_t e_count, int ncb,
                                                  const float* __restrict__ d_part, const uint16_t* __restrict__ b_down,
                                                  uint16_t* __restrict__ out) {
  extern __shared__ float s_d[];   // [kk][R], then the experts [kk] and weights [kk]
  int32_t* s_e = reinterpret_cast<int32_t*>(s_d + kk * R);
  float* s_w = s_d + kk * R + kk;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.y;
  const int64_t c = int64_t(blockIdx.x) * 256 + tid;
  const bool cv = c < hidden;
  const float y0 = cv ? y[t * hidden + c] : 0.f;   // in flight while d is summed
  for (int i = tid; i < kk * R; i += 256) {
    const int j = i / R, q = i - j * R;
    const float* dp = d_part + (t * kk + j) * ncb * R + q;
    float s = 0.f;
#pragma unroll 8
    for (int cb = 0; cb < ncb; ++cb) s += dp[cb * R];
    s_d[i] = s;
  }
  if (tid < kk) {
    s_e[tid] = min(max(ids[t * kk + tid], 0), e_count - 1);
    s_w[tid] = w[t * kk + tid];
  }
  __syncthreads();
  if (!cv) return;
  // sum_q B_down,e[c][q] d[j][q] for choice j, the row's loads issued together
  auto proj = [&](const uint4 (&v)[R / 8], int j) {
    float s = 0.f;
#pragma unroll
    for (int q8 = 0; q8 < R / 8; ++q8) {
      const uint32_t wv[4] = {v[q8].x, v[q8].y, v[q8].z, v[q8].w};
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        s = fmaf(bf16_to_f32(uint16_t(wv[z] & 0xffff)), s_d[j * R + 8 * q8 + 2 * z], s);
        s = fmaf(bf16_to_f32(uint16_t(wv[z] >> 16)), s_d[j * R + 8 * q8 + 2 * z + 1], s);
      }
    }
    return s;
  };
  auto load_row = [&](uint4 (&v)[R / 8], int j) {
    const uint16_t* bd = b_down + (int64_t(s_e[j]) * hidden + c) * R;
#pragma unroll
    for (int q8 = 0; q8 < R / 8; ++q8) v[q8] = load16(bd + 8 * q8);
  };
  float acc = y0;
  int j = 0;
  for (; j + 1 < kk; j += 2) {   // two choices' rows in flight at once
    uint4 va[R / 8], vb[R / 8];
    load_row(va, j);
    load_row(vb, j + 1);
    acc = fmaf(s_w[j], proj(va, j), acc);
    acc = fmaf(s_w[j + 1], proj(vb, j + 1), acc);
  }
  if (j < kk) {
    uint4 va[R / 8];
    load_row(va, j);
    acc = fmaf(s_w[j], proj(va, j), acc);
  }
  out[t * hidden + c] = f32_to_bf16(acc);
}

// Calls f(integral_constant<int, R>) for the rank r in {8, 16, ..., 64}.
template <typename F>
static hipError_t with_rank(int r, F&& f) {
  switch (r) {
    case 8: return f(std::integral_constant<int, 8>{});
    case 16: return f(std::integral_constant<int, 16>{});
    case 24: return f(std::integral_constant<int, 24>{});
    case 32: return f(std::integral_constant<int, 32>{});
    case 40: return f(std::integral_constant<int, 40>{});
    case 48: return f(std::integral_constant<int, 48>{});
    case 56: return f(std::integral_constant<int, 56>{});
    case 64: return f(std::integral_constant<int, 64>{});
    default: return hipErrorInvalidValue;
  }
}

int lora_kchunks(int64_t h) { return int((h + 511) / 512); }
int lora_col_blocks(int64_t inter) { return int((inter + kMidCols - 1) / kMidCols); }

hipError_t launch_dense_tiles(int64_t t, int tile_rows, TileDesc* tiles, int32_t* num_tiles, hipStream_t st) {
  const int64_t n = (t + tile_rows - 1) / tile_rows;
  const unsigned blocks = unsigned(std::max<int64_t>(1, (n + 255) / 256));
  hipLaunchKernelGGL(k_dense_tiles, dim3(blocks), dim3(256), 0, st, t, tile_rows, tiles, num_tiles);
  return hipGetLastError();
}

hipError_t launch_lora_in(const uint16_t* x, int64_t t, int64_t h, const int32_t* ids, int32_t kk, int32_t e,
                          const uint16_t* a_gu, int r, float* a_part, hipStream_t st) {
  const int64_t P = t * kk;
  if (P == 0) return hipSuccess;
  const dim3 g = dim3(unsigned(P), unsigned(lora_kchunks(h))), b = dim3(64);
  return with_rank(r, [&](auto rc) {
    hipLaunchKernelGGL((k_lora_in<decltype(rc)::value>), g, b, 0, st, x, h, ids, kk, e, a_gu, a_part);
    return hipGetLastError();
  });
}

hipError_t launch_lora_mid(const float* base_gu, int64_t t, int64_t h, int64_t inter, const int32_t* ids,
                           const float* w, int32_t kk, int32_t e, int r, const float* a_part, const uint16_t* b_gate,
                           const uint16_t* b_up, const uint16_t* a_down, float* d_part, uint16_t* hw, hipStream_t st) {
  if (t == 0) return hipSuccess;
  const dim3 g = dim3(unsigned(lora_col_blocks(inter)), unsigned(t)), b = dim3(256);
  const int nks = lora_kchunks(h);
  return with_rank(r, [&](auto rc) {
    hipLaunchKernelGGL((k_lora_mid<decltype(rc)::value>), g, b, 0, st, base_gu, inter, ids, w, kk, e, nks, a_part,
                       b_gate, b_up, a_down, d_part, hw);
    return hipGetLastError();
  });
}

hipError_t launch_lora_out(const float* y, int64_t t, int64_t hidden, int64_t inter, const int32_t* ids,
                           const float* w, int32_t kk, int32_t e, int r, const float* d_part, const uint16_t* b_down,
                           uint16_t* out, hipStream_t st, int ncb) {
  if (t == 0) return hipSuccess;
  const dim3 g = dim3(unsigned((hidden + 255) / 256), unsigned(t));
  if (ncb <= 0) ncb = lora_col_blocks(inter);
  return with_rank(r, [&](auto rc) {
    hipLaunchKernelGGL((k_lora_out<decltype(rc)::value>), g, dim3(256), size_t(kk) * (r + 2) * sizeof(float), st, y,
                       hidden, ids, w, kk, e, ncb, d_part, b_down, out);
    return hipGetLastError();
  });
}

bool lora_grouped_rank(int r) { return r == 16 || r == 32; }
int lora_grp_col_blocks(int64_t inter) { return int((inter + kGrpCols - 1) / kGrpCols); }

hipError_t launch_lora_mid_grp(const float* base_gu, int64_t inter, const int32_t* perm, const TileDesc* tiles,
                               const int32_t* num_tiles, int32_t max_tiles, int32_t kk, int64_t h, int r,
                               const float* a_part, const uint16_t* b_gate, const uint16_t* b_up,
                               const uint16_t* a_down, float* d_part, float* h_slot, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 g = dim3(unsigned(lora_grp_col_blocks(inter)), unsigned(max_tiles));
  const int nks = lora_kchunks(h);
  if (r == 16)
    hipLaunchKernelGGL((k_lora_mid_grp<16>), g, dim3(256), 0, st, base_gu, inter, perm, tiles, num_tiles, kk, nks,
                       a_part, b_gate, b_up, a_down, d_part, h_slot);
  else if (r == 32)
    hipLaunchKernelGGL((k_lora_mid_grp<32>), g, dim3(256), 0, st, base_gu, inter, perm, tiles, num_tiles, kk, nks,
                       a_part, b_gate, b_up, a_down, d_part, h_slot);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lora_hsum(const float* h_slot, const float* w, int64_t t, int32_t kk, int64_t inter, uint16_t* hw,
                            float* rs, hipStream_t st) {
  const int64_t n = t * (inter / 4);
  if (n == 0) return hipSuccess;
  if (inter % 128 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_lora_hsum, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, h_slot, w, t, kk, inter, hw, rs);
  return hipGetLastError();
}

}  // namespace q4
