// A6 per-token INT8 activation quantisation, A7/A8/A10/A11 grouped INT4 GEMM
// (W4A16 and W4A8, SwiGLU epilogue), A9 weighted combine.
//
// Method: page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" §2.3 (INT4 widened
// to INT8, INT8 x INT8 -> INT32, rescale by scale_w * scale_a), §3.1 (per-token
// activation scale amax / 127, round, clamp), §5.4 (dequantisation must be fused into
// the matrix product); page "高效大语言模型推理实践：INT4量化与MoE架构的融合探索"
// (SwiGLU FFN experts); page "大模型之Dense、MoE与量化", MoE section (outputs combined
// in proportion to the router scores, a shared expert used by every token).
//
// GEMM structure (gfx950):
//  - a workgroup of 4 waves computes 16*MB rows x 64 device columns (4 column blocks of
//    16); the 4 waves split the K groups into contiguous ranges and are reduced through
//    LDS at the end;
//  - each lane streams its 16-byte share of each 1 KB weight tile (one column block x
//    one group), widens the nibbles in registers and feeds the matrix core;
//  - W4A16 (bf16): the widened value is magic + d (exact in bf16); per group
//    gacc = sum x * (magic + d) over 4 MFMA 16x16x32 and the row sums xs = sum x over
//    4 MFMA with B = 1.0, then acc += s * (gacc - (magic + z) * xs) in fp32;
//  - fp16 activations: magic + d - (magic + z) = d - z is formed exactly with a packed
//    fp16 add, so gacc = sum x * (d - z) directly and acc += s * gacc;
//  - the loads of group g + 1 are issued before group g is computed (two stages);
//  - W4A8: 16 * (d - 8) as int8, two MFMA i32 16x16x64 per group, the INT32 group
//    accumulator is gacc / 16 (- (z - 8) * sum q_x for asymmetric weights), then
//    acc += s_w * acc_g in fp32 and the row scale s_x at the end.
#include "common.h"
#include "internal.h"

namespace q4 {

// ------------------------------------------------------------------ A6 act quant
// One workgroup (256 threads) per row; 8 consecutive elements per thread per step.
template <bool F32IN>
__global__ void __launch_bounds__(256) k_act_quant(const void* __restrict__ x, int64_t cols,
                                                   int8_t* __restrict__ q, float* __restrict__ s_out) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  auto load8v = [&](int64_t c, float v[8]) {
    if constexpr (F32IN) {
      const float* p = static_cast<const float*>(x) + row * cols + c;
      const float4 a = *reinterpret_cast<const float4*>(p);
      const float4 b = *reinterpret_cast<const float4*>(p + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 a = load16(static_cast<const uint16_t*>(x) + row * cols + c);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(uint16_t(w[i] & 0xffff));
        v[2 * i + 1] = bf16_to_f32(uint16_t(w[i] >> 16));
      }
    }
  };
  float amax = 0.f;
  for (int64_t c = int64_t(tid) * 8; c < cols; c += 256 * 8) {
    float v[8];
    load8v(c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) s_out[row] = s;
  for (int64_t c = int64_t(tid) * 8; c < cols; c += 256 * 8) {
    float v[8];
    load8v(c, v);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float qv = 0.f;
      if (s > 0.f) qv = fminf(fmaxf(rintf(__fdiv_rn(v[i], s)), -128.f), 127.f);
      packed[i >> 2] |= (uint32_t(int(qv)) & 0xffu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(q + row * cols + c) = make_uint2(packed[0], packed[1]);
  }
}

hipError_t launch_act_quant(const void* x, int x_is_f32, int64_t rows, int64_t cols, int8_t* q, float* s,
                            int32_t* /*qsum*/, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (x_is_f32)
    hipLaunchKernelGGL(k_act_quant<true>, dim3(unsigned(rows)), dim3(256), 0, st, x, cols, q, s);
  else
    hipLaunchKernelGGL(k_act_quant<false>, dim3(unsigned(rows)), dim3(256), 0, st, x, cols, q, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------ grouped GEMM
constexpr int kNB = 4;       // 16-column blocks per workgroup
constexpr int kWaves = 4;    // K split across the waves of a workgroup

struct RowInfo {
  int64_t src;   // activation row
  int64_t pos;   // output row
  bool valid;
};

template <Act A, int KIND, int MB>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs args) {
  extern __shared__ float red_lds[];  // [kWaves][MB][kNB][64][4]
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t N = args.N, K = args.K, G = K / kGroup;
  const int64_t nblk = N / (16 * kNB);
  const int64_t tile_rows = 16 * MB;
  const int64_t ntiles = args.tiles ? int64_t(*args.num_tiles) : (args.dense_rows + tile_rows - 1) / tile_rows;
  const int64_t items = ntiles * nblk;
  const int64_t w_scale_off = align256(N * K / 2);
  const int64_t w_zero_off = w_scale_off + align256(2 * N * G);
  // contiguous group range of this wave
  const int64_t gper = (G + kWaves - 1) / kWaves;
  const int64_t g_beg = std::min<int64_t>(G, wid * gper), g_end = std::min<int64_t>(G, g_beg + gper);

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t tile = item / nblk;
    const int64_t cb0 = (item % nblk) * kNB;
    int32_t expert = 0;
    int64_t row_start, rows;
    if (args.tiles) {
      const TileDesc d = args.tiles[tile];
      expert = d.expert;
      row_start = d.row_start;
      rows = d.rows;
    } else {
      row_start = tile * tile_rows;
      rows = std::min<int64_t>(tile_rows, args.dense_rows - row_start);
    }
    const uint8_t* wbase = expert < args.num_experts ? args.w + int64_t(expert) * args.w_stride : args.w_shared;
    const uint16_t* wscale = reinterpret_cast<const uint16_t*>(wbase + w_scale_off);
    const uint8_t* wzero = wbase + w_zero_off;

    // rows of the A fragments (lane row = col index in the A layout)
    RowInfo ri[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t r = mb * 16 + col;
      ri[mb].valid = r < rows;
      ri[mb].pos = row_start + r;
      int64_t src = ri[mb].pos;
      if (ri[mb].valid && args.perm) src = args.perm[ri[mb].pos] / args.slots_per_token;
      ri[mb].src = ri[mb].valid ? src : 0;
    }

    f32x4_t acc[MB][kNB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One group's operands: 16 bytes of each of the 4 weight tiles, the lane column's
    // scale / zero point, and the A fragments of the MB row blocks.
    struct Stage {
      uint32_t wv[kNB][4];
      uint16_t sc[kNB];
      uint8_t zp[kNB];
      uint32_t av[MB][4][4];
    };
    auto load_stage = [&](Stage& st, int64_t g) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const uint4 v = load16_stream(wbase + ((cb0 + nb) * G + g) * kTileBytes + lane * 16);
        st.wv[nb][0] = v.x; st.wv[nb][1] = v.y; st.wv[nb][2] = v.z; st.wv[nb][3] = v.w;
        const int64_t mi = ((cb0 + nb) * G + g) * 16 + col;
        st.sc[nb] = wscale[mi];
        st.zp[nb] = args.asym ? wzero[mi] : uint8_t(8);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (A != Act::I8) {
          const uint16_t* xa = static_cast<const uint16_t*>(args.a) + ri[mb].src * K + g * kGroup + 8 * kq;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (ri[mb].valid) v = load16(xa + 32 * s);
            st.av[mb][s][0] = v.x; st.av[mb][s][1] = v.y; st.av[mb][s][2] = v.z; st.av[mb][s][3] = v.w;
          }
        } else {
          const int8_t* qa = static_cast<const int8_t*>(args.a) + ri[mb].src * K + g * kGroup + 8 * kq;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
            if (ri[mb].valid) {
              lo = load8(qa + 64 * i);
              hi = load8(qa + 64 * i + 32);
            }
            st.av[mb][i][0] = lo.x; st.av[mb][i][1] = lo.y; st.av[mb][i][2] = hi.x; st.av[mb][i][3] = hi.y;
          }
        }
      }
    };
    auto compute_stage = [&](const Stage& st, int64_t g) {
      float sc[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) sc[nb] = f16_bits_to_f32(st.sc[nb]);
      if constexpr (A == Act::BF16) {
        // exact row sums of the group through the matrix core (B = 1.0)
        const uint32_t ones[4] = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
        f32x4_t xs[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          xs[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) xs[mb] = mfma16x16x32<A>(st.av[mb][s], ones, xs[mb]);
        }
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          uint32_t b[4][4];
#pragma unroll
          for (int s = 0; s < 4; ++s) widen_word_fp<A>(st.wv[nb][s], b[s]);
          const float negz = -(magic_offset<A>() + float(st.zp[nb]));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            f32x4_t gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) gacc = mfma16x16x32<A>(st.av[mb][s], b[s], gacc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb], fmaf(negz, xs[mb][i], gacc[i]), acc[mb][nb][i]);
          }
        }
      } else if constexpr (A == Act::F16) {
        // magic + d - (magic + z) = d - z, exact in fp16: no correction term
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const _Float16 nz = _Float16(-(magic_offset<A>() + float(st.zp[nb])));
          const f16x2_t negz = {nz, nz};
          uint32_t b[4][4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            widen_word_fp<A>(st.wv[nb][s], b[s]);
#pragma unroll
            for (int r = 0; r < 4; ++r) b[s][r] = bitcast<uint32_t>(bitcast<f16x2_t>(b[s][r]) + negz);
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            f32x4_t gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) gacc = mfma16x16x32<A>(st.av[mb][s], b[s], gacc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb], gacc[i], acc[mb][nb][i]);
          }
        }
      } else {
        int32_t qs[MB];
        if (args.asym) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            qs[mb] = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) qs[mb] = __builtin_amdgcn_sdot4(int32_t(st.av[mb][i][j]), 0x01010101, qs[mb], false);
            // row sum over the 4 quarters (every lane of a row then holds it)
            qs[mb] += __shfl_xor(qs[mb], 16, 64);
            qs[mb] += __shfl_xor(qs[mb], 32, 64);
          }
        }
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          uint32_t b[2][4];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            widen_word_i8(st.wv[nb][2 * i], b[i][0], b[i][1]);
            widen_word_i8(st.wv[nb][2 * i + 1], b[i][2], b[i][3]);
          }
          const int32_t zoff = int32_t(st.zp[nb]) - 8;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            i32x4_t gacc = {0, 0, 0, 0};
            gacc = mfma_i8_16x16x64(st.av[mb][0], b[0], gacc);
            gacc = mfma_i8_16x16x64(st.av[mb][1], b[1], gacc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              int32_t a32 = gacc[i] >> 4;                    // exact: gacc = 16 * sum q (d - 8)
              if (args.asym) a32 -= zoff * __shfl(qs[mb], 4 * kq + i, 64);
              if constexpr (KIND == GEMM_GROUP_ACC) {
                const int64_t r = mb * 16 + 4 * kq + i;
                if (r < rows)
                  args.acc_out[((row_start + r) * N + (cb0 + nb) * 16 + col) * G + g] = a32;
              } else {
                acc[mb][nb][i] = fmaf(sc[nb], float(a32), acc[mb][nb][i]);
              }
            }
          }
        }
      }
    };

    // two-stage software pipeline over this wave's groups: the loads of group g + 1
    // are in flight while group g is computed
    if (g_beg < g_end) {
      Stage s0, s1;
      load_stage(s0, g_beg);
      for (int64_t g = g_beg; g < g_end; g += 2) {
        if (g + 1 < g_end) load_stage(s1, g + 1);
        compute_stage(s0, g);
        if (g + 1 >= g_end) break;
        if (g + 2 < g_end) load_stage(s0, g + 2);
        compute_stage(s1, g + 1);
      }
    }
    if constexpr (KIND == GEMM_GROUP_ACC) continue;

    // ---------------- cross-wave reduction and epilogue
    float* mine = red_lds + wid * (MB * kNB * 64 * 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        *reinterpret_cast<f32x4_t*>(mine + ((mb * kNB + nb) * 64 + lane) * 4) = acc[mb][nb];
    __syncthreads();
    auto reduced = [&](int mb, int nb) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        s += *reinterpret_cast<const f32x4_t*>(red_lds + w * (MB * kNB * 64 * 4) + ((mb * kNB + nb) * 64 + lane) * 4);
      return s;
    };
    if constexpr (KIND == GEMM_PLAIN) {
      const int nb = wid;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f32x4_t v = reduced(mb, nb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = mb * 16 + 4 * kq + i;
          if (r < rows) {
            const int64_t pos = row_start + r;
            float y = v[i];
            if constexpr (A == Act::I8) y *= args.a_scale[args.perm ? args.perm[pos] / args.slots_per_token : pos];
            static_cast<float*>(args.out)[pos * N + (cb0 + nb) * 16 + col] = y;
          }
        }
      }
    } else if (wid < 2) {
      // device blocks cb0.. = gate_j, up_j, gate_j+1, up_j+1 ; pair wid -> h columns
      const int64_t I = N / 2;
      const int64_t hcol = (cb0 / 2 + wid) * 16 + col;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f32x4_t gv = reduced(mb, 2 * wid), uv = reduced(mb, 2 * wid + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = mb * 16 + 4 * kq + i;
          if (r < rows) {
            const int64_t pos = row_start + r;
            float gg = gv[i], uu = uv[i];
            if constexpr (A == Act::I8) {
              const float sa = args.a_scale[args.perm ? args.perm[pos] / args.slots_per_token : pos];
              gg *= sa;
              uu *= sa;
            }
            const float hv = gg / (1.0f + expf(-gg)) * uu;
            if constexpr (A == Act::I8)
              static_cast<float*>(args.out)[pos * I + hcol] = hv;
            else
              static_cast<uint16_t*>(args.out)[pos * I + hcol] = f32_to_bf16(hv);
          }
        }
      }
    }
    __syncthreads();
  }
}

template <Act A, int KIND>
static hipError_t launch_gemm_mb(const GemmArgs& g, int mb, hipStream_t st) {
  const int64_t nblk = g.N / (16 * kNB);
  const int64_t trows = 16 * mb;
  const int64_t max_tiles = g.tiles ? g.max_tiles : (g.dense_rows + trows - 1) / trows;
  const int64_t items = max_tiles * nblk;
  if (items == 0) return hipSuccess;
  const unsigned grid = unsigned(std::min<int64_t>(items, 256 * 16));
  const size_t lds = KIND == GEMM_GROUP_ACC ? 0 : size_t(kWaves) * mb * kNB * 64 * 4 * sizeof(float);
  switch (mb) {
    case 1: hipLaunchKernelGGL((k_gemm<A, KIND, 1>), dim3(grid), dim3(256), lds, st, g); break;
    case 2: hipLaunchKernelGGL((k_gemm<A, KIND, 2>), dim3(grid), dim3(256), lds, st, g); break;
    default: hipLaunchKernelGGL((k_gemm<A, KIND, 4>), dim3(grid), dim3(256), lds, st, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, int act, int kind, int row_blocks, hipStream_t st) {
  const int mb = row_blocks <= 1 ? 1 : (row_blocks <= 2 ? 2 : 4);
  if (act == 0) {
    if (kind == GEMM_GATE_UP) return launch_gemm_mb<Act::BF16, GEMM_GATE_UP>(g, mb, st);
    return launch_gemm_mb<Act::BF16, GEMM_PLAIN>(g, mb, st);
  }
  if (act == 1) return launch_gemm_mb<Act::F16, GEMM_PLAIN>(g, mb, st);
  if (kind == GEMM_GATE_UP) return launch_gemm_mb<Act::I8, GEMM_GATE_UP>(g, mb, st);
  if (kind == GEMM_GROUP_ACC) return launch_gemm_mb<Act::I8, GEMM_GROUP_ACC>(g, mb, st);
  return launch_gemm_mb<Act::I8, GEMM_PLAIN>(g, mb, st);
}

// ------------------------------------------------------------------ A9 combine
// out[t][n] = bf16( sum_{j<k, ascending} w[t][j] * y[inv[t S + j]][n] (+ y[inv[t S + k]][n]) )
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, int64_t t, int32_t k, int shared,
                                                 int64_t h, uint16_t* __restrict__ out) {
  const int64_t per_tok = h / 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= t * per_tok) return;
  const int64_t tok = i / per_tok;
  const int64_t c = (i - tok * per_tok) * 4;
  const int S = k + shared;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t pos = inv[tok * S + j];
    const float wj = w[tok * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + pos * h + c);
    a0 = fmaf(wj, v.x, a0);
    a1 = fmaf(wj, v.y, a1);
    a2 = fmaf(wj, v.z, a2);
    a3 = fmaf(wj, v.w, a3);
  }
  if (shared) {
    const int64_t pos = inv[tok * S + k];
    const float4 v = *reinterpret_cast<const float4*>(y + pos * h + c);
    a0 += v.x;
    a1 += v.y;
    a2 += v.z;
    a3 += v.w;
  }
  const uint32_t lo = uint32_t(f32_to_bf16(a0)) | (uint32_t(f32_to_bf16(a1)) << 16);
  const uint32_t hi = uint32_t(f32_to_bf16(a2)) | (uint32_t(f32_to_bf16(a3)) << 16);
  *reinterpret_cast<uint2*>(out + tok * h + c) = make_uint2(lo, hi);
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int64_t t, int32_t k, int shared,
                          int64_t h, uint16_t* out, hipStream_t st) {
  const int64_t n = t * (h / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, y, inv, w, t, k, shared, h, out);
  return hipGetLastError();
}

}  // namespace q4
