// Prefill grouped INT4 GEMM (A7/A8/A10/A11 at large row counts): LDS-staged activation
// tiles, in-register nibble widening, bf16 or INT8 matrix core, per-group scaling.
//
// Method: page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" §2.3 (INT4 widened to
// INT8, INT8 x INT8 -> INT32, rescale by scale_w * scale_a) and §5.4 (the dequantisation
// is fused into the matrix product); page "从FP32到INT4：大语言模型量化压缩实战指南" §1.3
// (one scale per group of 128 along K).
//
// Structure (gfx950):
//  - one workgroup (4 waves) computes a 128-row x 128-column tile of one expert; the
//    waves form a 2 x 2 grid of 64 x 64 sub-tiles (4 x 4 MFMA 16x16 blocks each);
//  - K advances one group (128) at a time.  The 128 x 128 activation tile of group g + 1
//    is copied global -> LDS with 16-byte direct-to-LDS loads while group g is computed
//    (two LDS buffers, one barrier per group); 16-byte chunks are XOR-swizzled by row so
//    that the MFMA fragment reads hit distinct banks;
//  - each wave streams its 4 weight tiles (16 bytes per lane) for group g + 1 into
//    registers during group g and widens them there (the same nibble layout as decode);
//  - bf16: acc += s * (sum_k x (magic + d) - (magic + z) * sum_k x), the row sums coming
//    precomputed per (row, group); INT8: acc += s * (acc_i32 / 16 [- (z - 8) sum q]).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace q4 {

constexpr int kPfRows = 128;   // rows per tile
constexpr int kPfCB = 8;       // 16-column blocks per workgroup

// Row sums per group of 128 (bf16 -> fp32, int8 -> int32), in element order.
__global__ void __launch_bounds__(256) k_rowsum_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                                     float* __restrict__ out) {
  const int64_t G = K / kGroup;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * G) return;
  const uint16_t* p = x + i / G * K + (i % G) * kGroup;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint4 v = load16(p + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s += bf16_to_f32(uint16_t(w[j] & 0xffff));
      s += bf16_to_f32(uint16_t(w[j] >> 16));
    }
  }
  out[i] = s;
}

__global__ void __launch_bounds__(256) k_rowsum_i8(const int8_t* __restrict__ q, int64_t rows, int64_t K,
                                                   int32_t* __restrict__ out) {
  const int64_t G = K / kGroup;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * G) return;
  const int8_t* p = q + i / G * K + (i % G) * kGroup;
  int32_t s = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 v = load16(p + 16 * c);
    s = __builtin_amdgcn_sdot4(int32_t(v.x), 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(int32_t(v.y), 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(int32_t(v.z), 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(int32_t(v.w), 0x01010101, s, false);
  }
  out[i] = s;
}

hipError_t launch_rowsum(const void* a, int is_i8, int64_t rows, int64_t K, void* out, hipStream_t st) {
  const int64_t n = rows * (K / kGroup);
  if (n == 0) return hipSuccess;
  const unsigned blocks = unsigned((n + 255) / 256);
  if (is_i8)
    hipLaunchKernelGGL(k_rowsum_i8, dim3(blocks), dim3(256), 0, st, static_cast<const int8_t*>(a), rows, K,
                       static_cast<int32_t*>(out));
  else
    hipLaunchKernelGGL(k_rowsum_bf16, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t*>(a), rows, K,
                       static_cast<float*>(out));
  return hipGetLastError();
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt that waits until at most n vector-memory operations are outstanding
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in [15:14]).
template <int N>
Q4_DEVICE void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Per-stage LDS image of one group (K = 128) of one work item:
//   A tile  [128 rows][ROWB]  (16-byte chunks XOR-swizzled by row)
//   W tiles [8 column blocks][64 lanes][16 B]  (the device tiles as stored)
//   scales  [8][16] fp16, zero points [8][16] u8 (asymmetric)
//   rsum    [128] fp32 row sums (bf16) / int32 code sums (int8, asymmetric)
template <Act A>
struct PfStage {
  static constexpr int ESZ = (A == Act::I8) ? 1 : 2;
  static constexpr int ROWB = kGroup * ESZ;
  static constexpr int A_BYTES = kPfRows * ROWB;
  static constexpr int W_OFF = A_BYTES;
  static constexpr int S_OFF = W_OFF + kPfCB * kTileBytes;
  static constexpr int Z_OFF = S_OFF + kPfCB * 32;
  static constexpr int R_OFF = S_OFF + 512;
  static constexpr int BYTES = R_OFF + kPfRows * 4;
};
constexpr int kPfStages = 3;

template <Act A, int KIND, bool ASYM>
__global__ void __launch_bounds__(256, 1) k_gemm_pf(GemmArgs args) {
  using St = PfStage<A>;
  constexpr int ROWB = St::ROWB;
  constexpr int CHUNKS = ROWB / 16;                   // 16-byte chunks per row
  constexpr int ROWS_PER_INST = 64 / CHUNKS;          // rows one direct-to-LDS load covers
  constexpr int A_INSTS = 32 / ROWS_PER_INST;         // A loads per wave per stage (32 rows)
  constexpr bool RSUM = (A != Act::I8) || ASYM;
  // three distinct LDS objects, so the compiler can tell which in-flight copies a read
  // depends on (the loop below is unrolled by three to keep each slot compile-time)
  __shared__ __align__(16) uint8_t slot0[St::BYTES];
  __shared__ __align__(16) uint8_t slot1[St::BYTES];
  __shared__ __align__(16) uint8_t slot2[St::BYTES];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid & 1, wn = wid >> 1;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t N = args.N, K = args.K;
  const int G = int(K / kGroup);
  const int64_t nblk = N / (16 * kPfCB);
  const int64_t ntiles = *args.num_tiles;
  const int64_t items = ntiles * nblk;
  const int64_t w_scale_off = align256(N * K / 2);
  const int64_t w_zero_off = w_scale_off + align256(2 * N * int64_t(G));

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t tile = item / nblk;
    const int64_t cb0 = (item % nblk) * kPfCB;
    const TileDesc d = args.tiles[tile];
    const int64_t row_start = d.row_start, rows = d.rows;
    const uint8_t* wbase = d.expert < args.num_experts ? args.w + int64_t(d.expert) * args.w_stride : args.w_shared;
    auto src_of = [&](int64_t r) -> int64_t {   // activation row of tile row r (clamped)
      const int64_t pos = row_start + (r < rows ? r : 0);
      return args.perm ? args.perm[pos] / args.slots_per_token : pos;
    };
    // global sources of this lane's direct-to-LDS copies
    const uint8_t* arow[A_INSTS];
#pragma unroll
    for (int j = 0; j < A_INSTS; ++j) {
      const int r = 32 * wid + ROWS_PER_INST * j + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ (r % CHUNKS);   // global chunk that lands in this slot
      arow[j] = static_cast<const uint8_t*>(args.a) + src_of(r) * K * St::ESZ + c * 16;
    }
    const uint8_t* wsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) wsrc[j] = wbase + (cb0 + 2 * wid + j) * G * kTileBytes + lane * 16;
    // wave 0: scales (lanes 0..15) and zero points (lanes 16..23) of the 8 blocks
    const uint8_t* msrc = nullptr;
    if (lane < 16) msrc = wbase + w_scale_off + ((cb0 + lane / 2) * G) * 32 + (lane & 1) * 16;
    else if (lane < 24) msrc = wbase + w_zero_off + ((cb0 + lane - 16) * G) * 16;
    // waves 1 and 2: the row sums of rows (wid - 1) * 64 + lane
    const void* rsrc = nullptr;
    if constexpr (RSUM) {
      if (wid == 1 || wid == 2) {
        const int64_t sr = src_of((wid - 1) * 64 + lane);
        if constexpr (A == Act::I8) rsrc = args.a_qsum + sr * G;
        else rsrc = args.a_gsum + sr * G;
      }
    }
    auto slot_of = [&](auto sl) -> uint8_t* {
      if constexpr (decltype(sl)::value == 0) return slot0;
      else if constexpr (decltype(sl)::value == 1) return slot1;
      else return slot2;
    };
    auto issue = [&](int g, auto sl) {
      uint8_t* base = slot_of(sl);
#pragma unroll
      for (int j = 0; j < A_INSTS; ++j)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(arow[j] + int64_t(g) * ROWB),
                                         (lds_ptr_t)(base + (32 * wid + ROWS_PER_INST * j) * ROWB), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(wsrc[j] + int64_t(g) * kTileBytes),
                                         (lds_ptr_t)(base + St::W_OFF + (2 * wid + j) * kTileBytes), 16, 0, 0);
      if (wid == 0 && (lane < 16 || (ASYM && lane < 24)))
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(msrc + (lane < 16 ? g * 32 : g * 16)),
                                         (lds_ptr_t)(base + St::S_OFF), 16, 0, 0);
      if constexpr (RSUM) {
        if (wid == 1 || wid == 2)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(static_cast<const int32_t*>(rsrc) + g),
                                           (lds_ptr_t)(base + St::R_OFF + (wid - 1) * 256), 4, 0, 0);
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // compute(sl, after_reads): after the LDS fragments of the stage are in registers,
    // after_reads() issues the copies of a later stage, then the math runs.
    auto compute = [&](auto sl, auto&& after_reads) {
      const uint8_t* base = slot_of(sl);
      const uint16_t* s_sc = reinterpret_cast<const uint16_t*>(base + St::S_OFF);
      const uint8_t* s_z = base + St::Z_OFF;
      const float* s_rs = reinterpret_cast<const float*>(base + St::R_OFF);
      float sc[4], zp[4];
      uint32_t wv[4][4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int cbl = wn * 4 + nb;
        sc[nb] = f16_bits_to_f32(s_sc[cbl * 16 + col]);
        zp[nb] = ASYM ? float(s_z[cbl * 16 + col]) : 8.0f;
        const uint4 v = *reinterpret_cast<const uint4*>(base + St::W_OFF + cbl * kTileBytes + lane * 16);
        wv[nb][0] = v.x; wv[nb][1] = v.y; wv[nb][2] = v.z; wv[nb][3] = v.w;
      }
      if constexpr (A == Act::BF16) {
        uint32_t af[4][4][4];
        f32x4_t xv[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int r = wm * 64 + mb * 16 + col;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int c = (4 * s + kq) ^ col;          // r % 16 == col
            const uint4 v = *reinterpret_cast<const uint4*>(base + r * ROWB + c * 16);
            af[mb][s][0] = v.x; af[mb][s][1] = v.y; af[mb][s][2] = v.z; af[mb][s][3] = v.w;
          }
          xv[mb] = *reinterpret_cast<const f32x4_t*>(s_rs + wm * 64 + mb * 16 + 4 * kq);
        }
        after_reads();
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          uint32_t b[4][4];
#pragma unroll
          for (int s = 0; s < 4; ++s) widen_word_fp<A>(wv[nb][s], b[s]);
          const float negz = -(magic_offset<A>() + zp[nb]);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            f32x4_t gacc = xv[mb] * negz;
#pragma unroll
            for (int s = 0; s < 4; ++s) gacc = mfma16x16x32<A>(af[mb][s], b[s], gacc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb], gacc[i], acc[mb][nb][i]);
          }
        }
      } else {
        uint32_t af[4][2][4];
        int32_t qv[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int r = wm * 64 + mb * 16 + col;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int c1 = (4 * i + (kq >> 1)) ^ (col & 7), c2 = (4 * i + 2 + (kq >> 1)) ^ (col & 7);
            const uint2 lo = *reinterpret_cast<const uint2*>(base + r * ROWB + c1 * 16 + 8 * (kq & 1));
            const uint2 hi = *reinterpret_cast<const uint2*>(base + r * ROWB + c2 * 16 + 8 * (kq & 1));
            af[mb][i][0] = lo.x; af[mb][i][1] = lo.y; af[mb][i][2] = hi.x; af[mb][i][3] = hi.y;
          }
          if constexpr (ASYM) {
            const i32x4_t q4 = *reinterpret_cast<const i32x4_t*>(s_rs + wm * 64 + mb * 16 + 4 * kq);
#pragma unroll
            for (int i = 0; i < 4; ++i) qv[mb][i] = q4[i];
          }
        }
        after_reads();
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          uint32_t b[2][4];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            widen_word_i8(wv[nb][2 * i], b[i][0], b[i][1]);
            widen_word_i8(wv[nb][2 * i + 1], b[i][2], b[i][3]);
          }
          const int32_t zoff = int32_t(zp[nb]) - 8;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            i32x4_t gacc = {0, 0, 0, 0};
            gacc = mfma_i8_16x16x64(af[mb][0], b[0], gacc);
            gacc = mfma_i8_16x16x64(af[mb][1], b[1], gacc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              int32_t a32 = gacc[i] >> 4;
              if constexpr (ASYM) a32 -= zoff * qv[mb][i];
              acc[mb][nb][i] = fmaf(sc[nb], float(a32), acc[mb][nb][i]);
            }
          }
        }
      }
    };

    // 3-slot ring: stages g + 1 and g + 2 are in flight while stage g is computed.  Each
    // wave issues at least A_INSTS + 2 copies per stage, so waiting until that many are
    // outstanding leaves only the newest stage in flight; then a barrier publishes every
    // wave's completed copies.  (The raw barrier carries no wait of its own; the empty
    // asm statements keep the compiler from moving memory accesses across it.)
    auto sync = [&](bool newest_in_flight) {
      if (newest_in_flight) wait_vmcnt<A_INSTS + 2>();
      else wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    issue(0, S0{});
    if (G > 1) issue(1, S1{});
    sync(G > 1);
    for (int g = 0; g < G; g += 3) {
      compute(S0{}, [&] { if (g + 2 < G) issue(g + 2, S2{}); });
      sync(g + 2 < G);
      if (g + 1 >= G) break;
      compute(S1{}, [&] { if (g + 3 < G) issue(g + 3, S0{}); });
      sync(g + 3 < G);
      if (g + 2 >= G) break;
      compute(S2{}, [&] { if (g + 4 < G) issue(g + 4, S1{}); });
      sync(g + 4 < G);
    }

    // epilogue
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = wm * 64 + mb * 16 + 4 * kq + i;
        if (r >= rows) continue;
        const int64_t pos = row_start + r;
        float sa = 1.0f;
        if constexpr (A == Act::I8) sa = args.a_scale[args.perm ? args.perm[pos] / args.slots_per_token : pos];
        if constexpr (KIND == GEMM_PLAIN) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            static_cast<float*>(args.out)[pos * N + (cb0 + wn * 4 + nb) * 16 + col] = acc[mb][nb][i] * sa;
        } else {
          const int64_t I = N / 2;
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float gg = acc[mb][2 * p][i] * sa, uu = acc[mb][2 * p + 1][i] * sa;
            const float hv = gg / (1.0f + expf(-gg)) * uu;
            const int64_t hcol = ((cb0 + wn * 4) / 2 + p) * 16 + col;
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

size_t prefill_lds_bytes(int act) {
  return size_t(kPfStages) * (act == 2 ? PfStage<Act::I8>::BYTES : PfStage<Act::BF16>::BYTES);
}


template <Act A, int KIND>
static hipError_t launch_pf_kind(const GemmArgs& g, hipStream_t st) {
  const int64_t nblk = g.N / (16 * kPfCB);
  const int64_t items = int64_t(g.max_tiles) * nblk;
  if (items == 0) return hipSuccess;
  const unsigned grid = unsigned(std::min<int64_t>(items, 256));
  if (g.asym)
    hipLaunchKernelGGL((k_gemm_pf<A, KIND, true>), dim3(grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemm_pf<A, KIND, false>), dim3(grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_gemm_prefill(const GemmArgs& g, int act, int kind, hipStream_t st) {
  if (g.N % (16 * kPfCB) != 0 || !g.tiles) return hipErrorInvalidValue;
  if (act == 0) {
    if (kind == GEMM_GATE_UP) return launch_pf_kind<Act::BF16, GEMM_GATE_UP>(g, st);
    return launch_pf_kind<Act::BF16, GEMM_PLAIN>(g, st);
  }
  if (act == 2) {
    if (kind == GEMM_GATE_UP) return launch_pf_kind<Act::I8, GEMM_GATE_UP>(g, st);
    return launch_pf_kind<Act::I8, GEMM_PLAIN>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace q4
