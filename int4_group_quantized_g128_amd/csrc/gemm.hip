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
// GEMM structure (gfx950; the template parameters of k_gemm below):
//  - a workgroup of 4 waves computes 16*MB rows x (4 / KW) * NBW column blocks of 16;
//    KW waves split the K groups into contiguous ranges (reduced through LDS at the
//    end) and each wave covers NBW column blocks;
//  - each lane streams its 16-byte share of each 1 KB weight tile (one column block x
//    one group), widens the nibbles in registers and feeds the matrix core; the loads
//    of the next D - 1 groups are in flight while a group is computed (a register
//    pipeline of depth D);
//  - W4A16 (bf16): the widened value is magic + d (exact in bf16); per group
//    gacc = sum x * (magic + d) over 4 MFMA 16x16x32 and the row sums xs = sum x over
//    4 MFMA with B = 1.0, then acc += s * (gacc - (magic + z) * xs) in fp32;
//  - fp16 activations: magic + d - (magic + z) = d - z is formed exactly with a packed
//    fp16 add, so gacc = sum x * (d - z) directly and acc += s * gacc;
//  - W4A8: 16 * (d - 8) as int8, two MFMA i32 16x16x64 per group, the INT32 group
//    accumulator is gacc / 16 (- (z - 8) * sum q_x for asymmetric weights), then
//    acc += s_w * acc_g in fp32 and the row scale s_x at the end; 8-bit weights go to
//    the matrix core as stored and 2-bit ones are widened to 64 q per byte.
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
  // The first kHeld chunks of 8 per thread (rows of up to 8192 columns) stay in
  // registers between the two passes, so such a row is read once, with all of its loads
  // in flight together; the rest of a longer row is read again for the second pass.
  constexpr int kHeld = 4;
  float held[kHeld][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kHeld; ++j) {
    const int64_t c = (int64_t(j) * 256 + tid) * 8;
    if (c < cols) {
      load8v(c, held[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(held[j][i]));
    }
  }
  for (int64_t c = (int64_t(kHeld) * 256 + tid) * 8; c < cols; c += 256 * 8) {
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
  auto store8 = [&](int64_t c, const float* v) {
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float qv = 0.f;
      if (s > 0.f) qv = fminf(fmaxf(rintf(__fdiv_rn(v[i], s)), -128.f), 127.f);
      packed[i >> 2] |= (uint32_t(int(qv)) & 0xffu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(q + row * cols + c) = make_uint2(packed[0], packed[1]);
  };
#pragma unroll
  for (int j = 0; j < kHeld; ++j) {
    const int64_t c = (int64_t(j) * 256 + tid) * 8;
    if (c < cols) store8(c, held[j]);
  }
  for (int64_t c = (int64_t(kHeld) * 256 + tid) * 8; c < cols; c += 256 * 8) {
    float v[8];
    load8v(c, v);
    store8(c, v);
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
struct RowInfo {
  int64_t src;   // activation row
  int64_t pos;   // output row
  bool valid;
};

// Copies n16 16-byte chunks from global memory to LDS with the workgroup's 256 threads;
// each thread issues up to 4 loads before its stores, so they share one memory latency.
Q4_DEVICE void stage16_to_lds(uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t n16) {
  constexpr int U = 4;
  for (int64_t i0 = threadIdx.x; i0 < n16; i0 += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = i0 + 256 * u < n16 ? src[i0 + 256 * u] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + 256 * u < n16) dst[i0 + 256 * u] = v[u];
  }
}

// Grouped INT4 GEMM.  Template parameters:
//  MB  16-row blocks per tile (rows of one expert, gathered through perm),
//  KW  waves of the workgroup that split the K groups (reduced through LDS),
//  NBW 16-column blocks per wave (the workgroup covers (4 / KW) * NBW blocks),
//  D   depth of the register pipeline (groups whose loads are in flight),
//  WB  weight bits: 4 (1 KB tiles of nibbles), 8 (2 KB tiles of INT8 codes, int8
//      activations, no widening) or 2 (512-byte tiles of 2-bit codes, int8
//      activations: each field widened to 64 q in a byte).
// Tiles are TS = 16 MB rows; a launch over tiles built taller (the prefill tiles of a
// layer whose 2-bit experts run on this kernel) walks each in TS-row sub-tiles.
// The workgroup's scales (and zero points) are staged in LDS once per work item.
template <Act A, int KIND, bool ASYM, int MB, int KW, int NBW, int D, int WB, int SGT>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs args) {
  constexpr bool W8 = WB == 8, W2 = WB == 2;
  static_assert(WB == 2 || WB == 4 || WB == 8, "weight bits");
  static_assert(!W8 || (A == Act::I8 && !ASYM), "8-bit weights: symmetric, int8 activations");
  static_assert(!W2 || (A == Act::I8 && !ASYM && SGT == 1), "2-bit weights: symmetric, int8 activations, g128");
  // SGT scale entries per 1 KB tile (groups of 128 / SGT elements; 0: per item, from the
  // expert's group size): symmetric 4-bit only
  static_assert(SGT == 1 || (!ASYM && !W8 && KIND != GEMM_GROUP_ACC && (SGT == 0 || SGT == 2 || SGT == 4)),
                "scale groups");
  constexpr int64_t TB = W8 ? 2 * kTileBytes : W2 ? kTileBytes / 2 : kTileBytes;   // bytes per (column block, group) tile
  constexpr int kColGroups = 4 / KW;
  constexpr int kCBWG = kColGroups * NBW;  // column blocks per workgroup
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int kw = wid % KW, cgrp = wid / KW;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t N = args.N, K = args.K, G = K / kGroup;
  const int64_t nblk = N / (16 * kCBWG);
  const int64_t tile_rows = 16 * MB;
  int64_t t_first = 0;   // layers with several weight formats: this launch's tile range
  int64_t ntiles = args.tiles      ? int64_t(*args.num_tiles)
                   : args.slot_ids ? args.dense_rows
                                   : (args.dense_rows + tile_rows - 1) / tile_rows;
  if (args.fmt_tiles) {
    t_first = args.fmt_tiles[args.fmt];
    ntiles = args.fmt_tiles[args.fmt_end] - t_first;
  }
  // plain GEMM with few work items (the few-items configuration only): ksplit K slices per
  // (tile, column blocks), each a work item of its own writing its partial sums to its own
  // output slice; every other configuration compiles with ksplit = 1
  constexpr bool kCanSplit = KIND == GEMM_PLAIN && MB == 1 && KW == 4 && NBW == 2;
  const int ksplit = (kCanSplit && args.ksplit > 1) ? args.ksplit : 1;
  // tiles built taller than TS rows (a prefill tile list): nsub sub-tiles each
  const int64_t nsub = (args.tiles && args.built_rows > tile_rows) ? (args.built_rows + tile_rows - 1) / tile_rows : 1;
  const int64_t base_items = ntiles * nsub * nblk;
  const int64_t items = base_items * ksplit;
  const int64_t gslice = (G + ksplit - 1) / ksplit;
  const int64_t w_scale_off = align256(W8 ? N * K : W2 ? N * K / 4 : N * K / 2);
  const int64_t w_zero_off = w_scale_off + align256(2 * N * G);   // zero points: one scale entry per tile
  // LDS: scales [kCBWG][G][16] fp16 (one entry per tile; with SG > 1 entries per tile
  // each lane loads its column's entries with the weights instead), zero points
  // [kCBWG][G][16] u8, reduction buffer
  const int64_t scale_lds = (SGT == 0 || SGT == 1) ? align256(int64_t(kCBWG) * G * 32) : 0;
  uint16_t* s_scale = reinterpret_cast<uint16_t*>(smem);
  uint8_t* s_zero = smem + scale_lds;
  float* s_red = reinterpret_cast<float*>(smem + scale_lds + (ASYM ? align256(int64_t(kCBWG) * G * 16) : 0));

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    int64_t it = item, ks = 0;
    if (ksplit > 1) {
      ks = it / base_items;
      it -= ks * base_items;
    }
    const int64_t tile = t_first + it / (nblk * nsub);
    const int64_t sub = (it / nblk) % nsub;
    const int64_t cb0 = (it % nblk) * kCBWG;     // first column block of the workgroup
    // this item's groups [kg0, kg1), shared out over the KW waves of a column group
    const int64_t kg0 = std::min<int64_t>(G, ks * gslice), kg1 = std::min<int64_t>(G, kg0 + gslice);
    const int64_t gper = (kg1 - kg0 + KW - 1) / KW;
    const int64_t g_beg = std::min<int64_t>(kg1, kg0 + kw * gper), g_end = std::min<int64_t>(kg1, g_beg + gper);
    int32_t expert = 0;
    int64_t row_start, rows;
    if (args.tiles) {
      const TileDesc d = args.tiles[tile];
      expert = d.expert;
      row_start = d.row_start + sub * tile_rows;
      rows = std::min<int64_t>(tile_rows, int64_t(d.rows) - sub * tile_rows);
    } else if (args.slot_ids) {   // one row per slot, its expert straight from the routed ids
      const int64_t tok = tile / args.slots_per_token;
      const int j = int(tile - tok * args.slots_per_token);
      expert = j < args.slot_k ? min(max(args.slot_ids[tok * args.slot_k + j], 0), args.num_experts - 1)
                               : args.num_experts;
      row_start = tile;
      rows = 1;
    } else {
      row_start = tile * tile_rows;
      rows = std::min<int64_t>(tile_rows, args.dense_rows - row_start);
    }
    if (rows <= 0) continue;   // an empty sub-tile (the whole workgroup skips it)
    const uint8_t* wbase = expert >= args.num_experts ? args.w_shared
                           : args.woffs                 ? args.w + args.woffs[expert]
                                                        : args.w + int64_t(expert) * args.w_stride;

    // the rest of the item, for SG scale entries per tile
    auto body = [&](auto sgc) {
    constexpr int SG = decltype(sgc)::value;
    // Rows past the tile end read the tile's first row: every MFMA output row depends on
    // its own A row only, and those rows are never stored, so no zero fill is needed.
    RowInfo ri[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t r = mb * 16 + col;
      ri[mb].valid = r < rows;
      ri[mb].pos = row_start + (ri[mb].valid ? r : 0);
      ri[mb].src = args.perm ? args.perm[ri[mb].pos] / args.slots_per_token
                   : args.src_div > 1 ? ri[mb].pos / args.src_div
                                      : ri[mb].pos;
    }

    const int lcb = cgrp * NBW;                       // wave's first block inside the workgroup
    // per-item base pointers; each group then only adds a constant stride
    const uint8_t* wp[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) wp[nb] = wbase + ((cb0 + lcb + nb) * G) * TB + lane * (W2 ? 8 : 16);
    const uint8_t* ap[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      ap[mb] = static_cast<const uint8_t*>(args.a) + (ri[mb].src * K + 8 * kq) * (A == Act::I8 ? 1 : 2);
    const int sbase = (lcb * int(G)) * 16 + col;

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    struct Stage {
      uint32_t wv[NBW][W8 ? 8 : W2 ? 2 : 4];
      uint32_t av[MB][4][4];
      uint32_t sv[NBW][SG > 1 ? SG / 2 : 1];   // SG > 1: the column's SG binary16 scales
    };
    // SG > 1: this lane's column's scale entries of group g, column block nb
    const uint8_t* sp = wbase + w_scale_off + (int64_t(cb0 + lcb) * G * 16 + col) * 2 * SG;
    auto load_stage = [&](Stage& st, int g) {
      if constexpr (SG == 2) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          st.sv[nb][0] = *reinterpret_cast<const uint32_t*>(sp + (int64_t(nb) * G + g) * 16 * 2 * SG);
      } else if constexpr (SG == 4) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const uint2 v = load8(sp + (int64_t(nb) * G + g) * 16 * 2 * SG);
          st.sv[nb][0] = v.x;
          st.sv[nb][1] = v.y;
        }
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        if constexpr (W2) {
          const uint2 v = load8_stream(wp[nb] + g * TB);
          st.wv[nb][0] = v.x; st.wv[nb][1] = v.y;
          continue;
        }
        const uint4 v = load16_stream(wp[nb] + g * TB);
        st.wv[nb][0] = v.x; st.wv[nb][1] = v.y; st.wv[nb][2] = v.z; st.wv[nb][3] = v.w;
        if constexpr (W8) {
          const uint4 v2 = load16_stream(wp[nb] + g * TB + kTileBytes);
          st.wv[nb][4] = v2.x; st.wv[nb][5] = v2.y; st.wv[nb][6] = v2.z; st.wv[nb][7] = v2.w;
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (A != Act::I8) {
          const uint8_t* xa = ap[mb] + g * (kGroup * 2);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint4 v = load16(xa + 64 * s);
            st.av[mb][s][0] = v.x; st.av[mb][s][1] = v.y; st.av[mb][s][2] = v.z; st.av[mb][s][3] = v.w;
          }
        } else {
          const uint8_t* qa = ap[mb] + g * kGroup;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint2 lo = load8(qa + 64 * i);
            const uint2 hi = load8(qa + 64 * i + 32);
            st.av[mb][i][0] = lo.x; st.av[mb][i][1] = lo.y; st.av[mb][i][2] = hi.x; st.av[mb][i][3] = hi.y;
          }
        }
      }
    };
    constexpr int SPS = 4 / SG;   // 32-element K steps per scale group
    auto compute_stage = [&](const Stage& st, int g) {
      float sc[NBW][SG], zp[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int li = sbase + (nb * int(G) + g) * 16;
        if constexpr (SG == 1) {
          sc[nb][0] = f16_bits_to_f32(s_scale[li]);
        } else {
#pragma unroll
          for (int j = 0; j < SG; ++j) sc[nb][j] = f16_bits_to_f32(uint16_t(st.sv[nb][j / 2] >> (16 * (j & 1))));
        }
        zp[nb] = ASYM ? float(s_zero[li]) : 8.0f;   // SG == 1 with zero points
      }
      if constexpr (A == Act::BF16) {
        // The correction -(magic + z) * sum x enters as the initial accumulator.  Its row
        // sums come from the matrix core: B = -(128 + 8) for symmetric weights (one
        // product serves every column), B = 1 then a per-column multiply otherwise.
        // (per scale group: the sums run over its own K steps)
        f32x4_t ini[MB][SG];
        const uint32_t cb = ASYM ? 0x3f803f80u : 0xc308c308u;   // bf16 1.0 / -136.0
        const uint32_t cvec[4] = {cb, cb, cb, cb};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < SG; ++j) {
            ini[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = j * SPS; s < (j + 1) * SPS; ++s) ini[mb][j] = mfma16x16x32<A>(st.av[mb][s], cvec, ini[mb][j]);
          }
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          uint32_t b[4][4];
#pragma unroll
          for (int s = 0; s < 4; ++s) widen_word_fp<A>(st.wv[nb][s], b[s]);
          const float negz = -(magic_offset<A>() + zp[nb]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int j = 0; j < SG; ++j) {
              f32x4_t gacc = ini[mb][j];
              if constexpr (ASYM) gacc *= negz;
#pragma unroll
              for (int s = j * SPS; s < (j + 1) * SPS; ++s) gacc = mfma16x16x32<A>(st.av[mb][s], b[s], gacc);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb][j], gacc[i], acc[mb][nb][i]);
            }
          }
        }
      } else if constexpr (A == Act::F16) {
        // magic + d - (magic + z) = d - z, exact in fp16: no correction term
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const _Float16 nz = _Float16(-(magic_offset<A>() + zp[nb]));
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
#pragma unroll
            for (int j = 0; j < SG; ++j) {
              f32x4_t gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = j * SPS; s < (j + 1) * SPS; ++s) gacc = mfma16x16x32<A>(st.av[mb][s], b[s], gacc);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb][j], gacc[i], acc[mb][nb][i]);
            }
          }
        }
      } else {
        int32_t qs[MB];
        if constexpr (ASYM) {
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
        for (int nb = 0; nb < NBW; ++nb) {
          uint32_t b[2][4];
          if constexpr (W8) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) b[i][j] = st.wv[nb][4 * i + j];
          } else if constexpr (W2) {
            // word i holds K steps 2i, 2i + 1; field f of its four bytes is elements
            // 0..3 (f even) or 4..7 (f odd) of step 2i + f / 2, in the operand's k order
#pragma unroll
            for (int i = 0; i < 2; ++i) widen_word_i8_2bit(st.wv[nb][i], b[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              widen_word_i8(st.wv[nb][2 * i], b[i][0], b[i][1]);
              widen_word_i8(st.wv[nb][2 * i + 1], b[i][2], b[i][3]);
            }
          }
          const int32_t zoff = int32_t(zp[nb]) - 8;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            if constexpr (SG > 1) {
              // one accumulator per scale group: a 64-element MFMA per group of 64, the two
              // 32-element halves of each operand per group of 32 (exact, 16 (d - 8) codes)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                if constexpr (SG == 2) {
                  const i32x4_t ga = mfma_i8_16x16x64(st.av[mb][h], b[h], i32x4_t{0, 0, 0, 0});
#pragma unroll
                  for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb][h], float(ga[i] >> 4), acc[mb][nb][i]);
                } else {
#pragma unroll
                  for (int q = 0; q < 2; ++q) {
                    const i32x4_t ga = mfma_i8_16x16x32(st.av[mb][h][2 * q], st.av[mb][h][2 * q + 1], b[h][2 * q],
                                                        b[h][2 * q + 1], i32x4_t{0, 0, 0, 0});
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                      acc[mb][nb][i] = fmaf(sc[nb][2 * h + q], float(ga[i] >> 4), acc[mb][nb][i]);
                  }
                }
              }
              continue;
            }
            i32x4_t gacc = {0, 0, 0, 0};
            gacc = mfma_i8_16x16x64(st.av[mb][0], b[0], gacc);
            gacc = mfma_i8_16x16x64(st.av[mb][1], b[1], gacc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // 4-bit: exact, gacc = 16 * sum q (d - 8); 2-bit: 64 * sum q (d - 2); 8-bit: the
              // group sum itself
              int32_t a32 = W8 ? gacc[i] : W2 ? (gacc[i] >> 6) : (gacc[i] >> 4);
              if constexpr (ASYM) a32 -= zoff * __shfl(qs[mb], 4 * kq + i, 64);
              if constexpr (KIND == GEMM_GROUP_ACC) {
                const int64_t r = mb * 16 + 4 * kq + i;
                if (r < rows)
                  args.acc_out[((row_start + r) * N + (cb0 + lcb + nb) * 16 + col) * G + g] = a32;
              } else {
                acc[mb][nb][i] = fmaf(sc[nb][0], float(a32), acc[mb][nb][i]);
              }
            }
          }
        }
      }
    };

    // stage the workgroup's scales / zero points (contiguous in the device layout)
    if constexpr (SG == 1) {
      stage16_to_lds(reinterpret_cast<uint4*>(s_scale),
                     reinterpret_cast<const uint4*>(wbase + w_scale_off + cb0 * G * 32), int64_t(kCBWG) * G * 2);
      if constexpr (ASYM)
        stage16_to_lds(reinterpret_cast<uint4*>(s_zero), reinterpret_cast<const uint4*>(wbase + w_zero_off + cb0 * G * 16),
                       int64_t(kCBWG) * G);
    }
    __syncthreads();

    // D-stage register pipeline over this wave's groups: while group g is computed the
    // loads of groups g + 1 .. g + D - 1 are in flight
    if (g_beg < g_end) {
      Stage st[D];
      const int gb = int(g_beg), ge = int(g_end);
#pragma unroll
      for (int j = 0; j < D - 1; ++j)
        if (gb + j < ge) load_stage(st[j], gb + j);
      for (int g = gb; g < ge; g += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
          if (g + j >= ge) break;
          if (g + j + D - 1 < ge) load_stage(st[(j + D - 1) % D], g + j + D - 1);
          compute_stage(st[j], g + j);
        }
      }
    }

    if constexpr (KIND != GEMM_GROUP_ACC) {
      // ---------------- reduction over the KW waves of a column group, then epilogue
      if constexpr (KW > 1) {
        float* mine = s_red + wid * (MB * NBW * 64 * 4);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            *reinterpret_cast<f32x4_t*>(mine + ((mb * NBW + nb) * 64 + lane) * 4) = acc[mb][nb];
        __syncthreads();
        if (kw == 0) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
              for (int w = 1; w < KW; ++w)
                acc[mb][nb] += *reinterpret_cast<const f32x4_t*>(s_red + (wid + w) * (MB * NBW * 64 * 4) +
                                                                 ((mb * NBW + nb) * 64 + lane) * 4);
        }
      }
      if (kw == 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t r = mb * 16 + 4 * kq + i;
            if (r >= rows) continue;
            const int64_t pos = row_start + r;
            float sa = 1.0f;
            if constexpr (A == Act::I8)
              sa = args.a_scale[args.perm ? args.perm[pos] / args.slots_per_token
                                : args.src_div > 1 ? pos / args.src_div
                                                   : pos];
            if constexpr (KIND == GEMM_PLAIN) {
              if (args.combine_w) {
                // the combine of a one-expert layer: its arithmetic exactly (fp32 w * y, then bf16)
                const float wt = args.combine_w[pos];
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                  args.out_bf16[pos * N + (cb0 + lcb + nb) * 16 + col] = f32_to_bf16(fmaf(wt, acc[mb][nb][i] * sa, 0.f));
              } else {
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                  static_cast<float*>(args.out)[ks * args.out_slice + pos * N + (cb0 + lcb + nb) * 16 + col] =
                      acc[mb][nb][i] * sa;
              }
            } else {
              // device blocks alternate gate_j, up_j: pair p -> h columns of block (cb0 + lcb) / 2 + p
              const int64_t I = N / 2;
#pragma unroll
              for (int p = 0; p < NBW / 2; ++p) {
                const float gg = acc[mb][2 * p][i] * sa, uu = acc[mb][2 * p + 1][i] * sa;
                const float hv = swiglu(gg, uu);
                const int64_t hcol = ((cb0 + lcb) / 2 + p) * 16 + col;
                if constexpr (A == Act::I8)
                  static_cast<float*>(args.out)[pos * I + hcol] = hv;
                else
                  static_cast<uint16_t*>(args.out)[pos * I + hcol] = f32_to_bf16(hv);
              }
            }
          }
        }
      }
    }
    __syncthreads();
    };
    if constexpr (SGT == 0) {   // the expert's own scale entries per tile (wave-uniform)
      const int sge = __builtin_amdgcn_readfirstlane(args.egroups ? sg_of_code(args.egroups[expert]) : 1);
      if (sge == 4)
        body(std::integral_constant<int, 4>{});
      else if (sge == 2)
        body(std::integral_constant<int, 2>{});
      else
        body(std::integral_constant<int, 1>{});
    } else {
      body(std::integral_constant<int, SGT>{});
    }
  }
}

// LDS bytes of one configuration (scales, zero points, reduction buffer).
static size_t gemm_lds_bytes(int64_t K, int asym, int mb, int kw, int nbw, int sg) {
  const int64_t G = K / kGroup;
  const int64_t cbwg = (4 / kw) * nbw;
  size_t b = (sg == 0 || sg == 1) ? size_t(align256(cbwg * G * 32)) : 0;   // 0: per item
  if (asym) b += size_t(align256(cbwg * G * 16));
  if (kw > 1) b += size_t(4) * mb * nbw * 64 * 4 * sizeof(float);
  return b;
}

template <Act A, int KIND, int MB, int KW, int NBW, int D, int WB = 4, int SG = 1>
static hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  constexpr int cbwg = (4 / KW) * NBW;
  const int64_t nblk = g.N / (16 * cbwg);
  const int64_t trows = 16 * MB;
  const int64_t max_tiles = g.tiles ? g.max_tiles : g.slot_ids ? g.dense_rows : (g.dense_rows + trows - 1) / trows;
  constexpr bool can_split = KIND == GEMM_PLAIN && MB == 1 && KW == 4 && NBW == 2;
  const int64_t nsub = (g.tiles && g.built_rows > trows) ? (g.built_rows + trows - 1) / trows : 1;
  const int64_t items = max_tiles * nsub * nblk * ((can_split && g.ksplit > 1) ? g.ksplit : 1);
  if (items == 0) return hipSuccess;
#ifndef Q4_GRID_CAP
#define Q4_GRID_CAP (256 * 16)
#endif
  const unsigned grid = unsigned(std::min<int64_t>(items, Q4_GRID_CAP));
  const size_t lds = gemm_lds_bytes(g.K, g.asym, MB, KW, NBW, SG);
  if (lds > 160 * 1024) return hipErrorInvalidValue;  // K too large for the staged scales
  if constexpr (SG > 1 || SG == 0) {
    if (g.asym) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm<A, KIND, false, MB, KW, NBW, D, 4, SG>), dim3(grid), dim3(256), lds, st, g);
  } else if constexpr (WB != 4) {
    if (g.asym) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm<A, KIND, false, MB, KW, NBW, D, WB, 1>), dim3(grid), dim3(256), lds, st, g);
  } else if (g.asym) {
    hipLaunchKernelGGL((k_gemm<A, KIND, true, MB, KW, NBW, D, 4, 1>), dim3(grid), dim3(256), lds, st, g);
  } else {
    hipLaunchKernelGGL((k_gemm<A, KIND, false, MB, KW, NBW, D, 4, 1>), dim3(grid), dim3(256), lds, st, g);
  }
  return hipGetLastError();
}

// Decode configuration (16-row tiles, many tiles), by operation and activation type.
// gate/up: two waves per column group split K (KW = 2, 128 columns per workgroup), so a
// work item streams half as long and the launch's closing ramp, where fewer and fewer
// items are in flight, is shorter (256-expert layer T = 64: bf16 354 -> 345 us with a
// three-stage register pipeline, int8 350 -> 330 us); down (K = 2048, shorter items
// already): one wave per column group for bf16 (KW = 2 measured 191 -> 203 us), two for
// int8 (188 -> 184 us).  Layers with other group sizes (SG != 1) keep one wave per column
// group (two would need 250-280 registers), and three stages are used only where the
// registers allow it (bf16, one scale entry per tile: down 194.7 -> 191.9 us at T = 64
// with three stages, 205 registers, the same two waves per SIMD as with two; four
// stages, 255 / 237 registers, measured no faster for gate/up and 1.6 % slower for down).
template <Act A, int KIND, int WB, int SG>
struct DecodeCfg {
  static constexpr bool kPlain = KIND == GEMM_PLAIN;
  static constexpr int KW = (SG == 1 && (!kPlain || A == Act::I8)) ? 2 : 1;
  static constexpr int NBW = 4;
  static constexpr int D = (A == Act::BF16 && SG == 1 && WB == 4) ? 3 : 2;
  static constexpr int CB = (4 / KW) * NBW;   // column blocks per workgroup
};

// Configuration table: (MB, KW, NBW, D) by row blocks and the column count.
template <Act A, int KIND, int WB, int SG>
static hipError_t launch_kind_sg(const GemmArgs& g, int rb, int split, hipStream_t st) {
  if (rb <= 1) {
    using C = DecodeCfg<A, KIND, WB, SG>;
    if (split && g.N % (16 * 2) == 0) return launch_cfg<A, KIND, 1, 4, 2, 2, WB, SG>(g, st);
    if (g.N % (16 * C::CB) == 0) return launch_cfg<A, KIND, 1, C::KW, C::NBW, C::D, WB, SG>(g, st);
    return launch_cfg<A, KIND, 1, 4, 2, 2, WB, SG>(g, st);
  }
  if (rb <= 2) return launch_cfg<A, KIND, 2, 4, 4, 2, WB, SG>(g, st);
  // 64-row tiles: one scale entry per tile only (the forward caps the tiles of layers
  // with other group sizes at 32 rows; four row blocks with per-group accumulators
  // would not fit the registers)
  if constexpr (SG == 1) return launch_cfg<A, KIND, 4, 4, 4, 2, WB, SG>(g, st);
  return hipErrorInvalidValue;
}

// scale entries per tile: 1 (groups of 128 / 256), 2 (64), 4 (32; 4-bit weights only), or
// -1: per item from the expert's group size (one launch for all 4-bit formats)
template <Act A, int KIND, int WB = 4>
static hipError_t launch_kind(const GemmArgs& g, int rb, int split, hipStream_t st) {
  if constexpr (WB == 4 && A != Act::F16) {
    if (g.sg == 2) return launch_kind_sg<A, KIND, false, 2>(g, rb, split, st);
    if (g.sg == 4) return launch_kind_sg<A, KIND, false, 4>(g, rb, split, st);
    if (g.sg == -1) {
      if (g.asym) return hipErrorInvalidValue;
      return launch_kind_sg<A, KIND, 4, 0>(g, rb, split, st);
    }
  }
  if (g.sg > 1 || g.sg < 0) return hipErrorInvalidValue;
  return launch_kind_sg<A, KIND, WB, 1>(g, rb, split, st);
}

hipError_t launch_gemm(const GemmArgs& g, int act, int kind, int row_blocks, hipStream_t st) {
  if (act != 2 && g.wbits != 0 && g.wbits != 4) return hipErrorInvalidValue;   // 2 / 8-bit weights: int8 only
  // K slices: plain GEMM on 16-row tiles only, in the few-items configuration (the one
  // that implements them); each output slice holds the a_rows rows
  if (g.ksplit > 1) {
    if (kind != GEMM_PLAIN || row_blocks != 1 || g.N % 32 != 0 || g.out_slice < g.a_rows * g.N || g.ebits ||
        g.egroups)
      return hipErrorInvalidValue;
    if (act == 0) return launch_cfg<Act::BF16, GEMM_PLAIN, 1, 4, 2, 2>(g, st);
    if (act == 1) return launch_cfg<Act::F16, GEMM_PLAIN, 1, 4, 2, 2>(g, st);
    if (g.wbits == 8) return launch_cfg<Act::I8, GEMM_PLAIN, 1, 4, 2, 2, 8>(g, st);
    if (g.wbits == 2) return hipErrorInvalidValue;
    return launch_cfg<Act::I8, GEMM_PLAIN, 1, 4, 2, 2>(g, st);
  }
  // few tiles (small batches): split K over the 4 waves for more waves in flight
  const int64_t est_items = (g.tiles ? std::min<int64_t>(g.max_tiles, 64) : 1) * (g.N / 128);
  const int split = est_items < 1024 ? 1 : 0;
  if (act == 0) {
    if (kind == GEMM_GATE_UP) return launch_kind<Act::BF16, GEMM_GATE_UP>(g, row_blocks, split, st);
    return launch_kind<Act::BF16, GEMM_PLAIN>(g, row_blocks, split, st);
  }
  if (act == 1) return launch_kind<Act::F16, GEMM_PLAIN>(g, row_blocks, split, st);
  if (g.wbits == 8) {
    if (kind == GEMM_GATE_UP) return launch_kind<Act::I8, GEMM_GATE_UP, 8>(g, row_blocks, split, st);
    if (kind == GEMM_GROUP_ACC) return launch_cfg<Act::I8, GEMM_GROUP_ACC, 1, 4, 1, 2, 8>(g, st);
    return launch_kind<Act::I8, GEMM_PLAIN, 8>(g, row_blocks, split, st);
  }
  if (g.wbits == 2) {
    if (kind == GEMM_GATE_UP) return launch_kind<Act::I8, GEMM_GATE_UP, 2>(g, row_blocks, split, st);
    if (kind == GEMM_GROUP_ACC) return launch_cfg<Act::I8, GEMM_GROUP_ACC, 1, 4, 1, 2, 2>(g, st);
    return launch_kind<Act::I8, GEMM_PLAIN, 2>(g, row_blocks, split, st);
  }
  if (kind == GEMM_GATE_UP) return launch_kind<Act::I8, GEMM_GATE_UP>(g, row_blocks, split, st);
  if (kind == GEMM_GROUP_ACC) return launch_cfg<Act::I8, GEMM_GROUP_ACC, 1, 4, 1, 2>(g, st);
  return launch_kind<Act::I8, GEMM_PLAIN>(g, row_blocks, split, st);
}

// ------------------------------------------------------------------ A9 combine
// out[t][n] = bf16( sum_{j<k, ascending} w[t][j] * y[inv[t S + j]][n] (+ y[inv[t S + k]][n]) ),
// inv == NULL: positions in slot order (a one-expert layer's rows are its tokens),
// with y = the sum of the ksplit slices y + s * slice in slice order when the down
// projection split K (SPLIT); NT reads y with non-temporal loads (each value is read
// once; used when y is larger than the 256 MB last-level cache)
template <bool SPLIT, bool NT>
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, int64_t t, int32_t k, int shared,
                                                 int64_t h, uint16_t* __restrict__ out, int ksplit, int64_t slice) {
  const int64_t per_tok = h / 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= t * per_tok) return;
  const int64_t tok = i / per_tok;
  const int64_t c = (i - tok * per_tok) * 4;
  const int S = k + shared;
  auto row = [&](int64_t pos) {
    float4 v;
    if constexpr (NT) {
      const uint4 u = load16_stream(y + pos * h + c);
      v = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    } else {
      v = *reinterpret_cast<const float4*>(y + pos * h + c);
    }
    if constexpr (SPLIT) {
      for (int s = 1; s < ksplit; ++s) {
        const float4 u = *reinterpret_cast<const float4*>(y + s * slice + pos * h + c);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
    }
    return v;
  };
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  // eight slots at a time: all index / weight loads, then all row loads, then the sums
  // in slot order
  constexpr int U = 8;
  for (int j0 = 0; j0 < k; j0 += U) {
    int64_t pos[U];
    float wj[U];
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = j0 + u < k;
      pos[u] = ok ? (inv ? inv[tok * S + j0 + u] : tok * S + j0 + u) : 0;
      wj[u] = ok ? w[tok * k + j0 + u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = j0 + u < k ? row(pos[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < k) {
        a0 = fmaf(wj[u], v[u].x, a0);
        a1 = fmaf(wj[u], v[u].y, a1);
        a2 = fmaf(wj[u], v[u].z, a2);
        a3 = fmaf(wj[u], v[u].w, a3);
      }
    }
  }
  if (shared) {
    const float4 v = row(inv ? inv[tok * S + k] : tok * S + k);
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
                          int64_t h, uint16_t* out, hipStream_t st, int ksplit, int64_t slice) {
  const int64_t n = t * (h / 4);
  if (n == 0) return hipSuccess;
  const dim3 grid(unsigned((n + 255) / 256));
  const bool nt = double(t) * (k + shared) * h * 4 > 256.0 * 1024 * 1024;
  if (ksplit > 1)
    hipLaunchKernelGGL((k_combine<true, false>), grid, dim3(256), 0, st, y, inv, w, t, k, shared, h, out, ksplit,
                       slice);
  else if (nt)
    hipLaunchKernelGGL((k_combine<false, true>), grid, dim3(256), 0, st, y, inv, w, t, k, shared, h, out, 1,
                       int64_t(0));
  else
    hipLaunchKernelGGL((k_combine<false, false>), grid, dim3(256), 0, st, y, inv, w, t, k, shared, h, out, 1,
                       int64_t(0));
  return hipGetLastError();
}

}  // namespace q4
