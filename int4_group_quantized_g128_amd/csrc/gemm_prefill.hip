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
#include <utility>

#include "common.h"
#include "internal.h"

namespace q4 {

constexpr int kPfRows = 128;   // rows per tile
constexpr int kPfCB = 8;       // 16-column blocks per workgroup

// Row sums per scale group (bf16 -> fp32 over C chunks of 8: groups of 128, 64 or 32;
// int8 -> int32 over groups of 128), in element order.
template <int C>
__global__ void __launch_bounds__(256) k_rowsum_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                                     float* __restrict__ out) {
  const int64_t G = K / (8 * C);
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * G) return;
  const uint16_t* p = x + i / G * K + (i % G) * (8 * C);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
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

hipError_t launch_rowsum(const void* a, int is_i8, int64_t rows, int64_t K, void* out, hipStream_t st, int sg) {
  if (is_i8 && sg > 1) return hipErrorInvalidValue;
  const int64_t n = rows * (K / kGroup) * sg;
  if (n == 0) return hipSuccess;
  const unsigned blocks = unsigned((n + 255) / 256);
  const uint16_t* x = static_cast<const uint16_t*>(a);
  float* o = static_cast<float*>(out);
  if (is_i8)
    hipLaunchKernelGGL(k_rowsum_i8, dim3(blocks), dim3(256), 0, st, static_cast<const int8_t*>(a), rows, K,
                       static_cast<int32_t*>(out));
  else if (sg == 4)
    hipLaunchKernelGGL(k_rowsum_bf16<4>, dim3(blocks), dim3(256), 0, st, x, rows, K, o);
  else if (sg == 2)
    hipLaunchKernelGGL(k_rowsum_bf16<8>, dim3(blocks), dim3(256), 0, st, x, rows, K, o);
  else
    hipLaunchKernelGGL(k_rowsum_bf16<16>, dim3(blocks), dim3(256), 0, st, x, rows, K, o);
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

// Raw buffer resource (V#) over [base, base + bytes), bytes < 2^31: copies address it with
// a per-lane 32-bit offset plus a wave-uniform scalar offset, so advancing K costs no VALU.
Q4_DEVICE u32x4_t buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{uint32_t(a), uint32_t(a >> 32) & 0xffffu, uint32_t(bytes), 0x00020000u};
}

// LDS byte address of a generic pointer into LDS: the low half of a flat LDS address is
// the LDS offset (the high half is the shared aperture), so no address-space cast (and
// its null check) is needed.
Q4_DEVICE uint32_t lds_addr(const void* p) { return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)); }

// Direct-to-LDS copy of SIZE (16 or 4) bytes per lane: lane L's bytes land at
// lds + L * SIZE.  Written as inline asm with no register outputs other than a scratch
// SGPR: the compiler then does not see an LDS write whose target it cannot tell apart
// from the ring slot being read, and would otherwise wait for every copy in flight
// before each LDS read.  The kernel orders copies and reads itself (vmcnt waits +
// barriers).  M0 (the LDS base of the copy) is saved and restored around it; the
// leading s_nop covers the wait states between SGPR/M0 writes and their use.
template <int SIZE>
Q4_DEVICE void copy_to_lds(const u32x4_t& rsrc, uint32_t lds_in, uint32_t voff, uint32_t soff_in) {
  static_assert(SIZE == 16 || SIZE == 4, "copy size");
  // wave-uniform by construction; readfirstlane makes that visible (scalar operands)
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  const uint32_t soff = __builtin_amdgcn_readfirstlane(soff_in);
  uint32_t saved;
  if constexpr (SIZE == 16)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
  (void)saved;
}

// Per-stage LDS image of one group (K = 128) of one work item:
//   A tile  [128 rows][ROWB]  (16-byte chunks XOR-swizzled by row)
//   W tiles [8 column blocks][TB]  (the device tiles as stored: 1 KB 4-bit, 2 KB 8-bit)
//   scales  [8][16][SG] fp16, zero points [8][16] u8 (asymmetric, SG == 1)
//   rsum    [SG][128] fp32 row sums (bf16) / int32 code sums (int8, asymmetric)
// (SG scale entries per tile: groups of 128 / SG elements)
// int8 activations: two workgroups per CU (a two-slot ring: 51 KB of LDS with 4-bit
// weights, 67 KB with 8-bit ones, and at most 256 registers per lane) so the waves of one
// hide the barrier and LDS latencies of the other
#ifndef Q4_PF_GRID_I8
#define Q4_PF_GRID_I8 512
#endif
#ifndef Q4_PF_SLOTS_I8
#define Q4_PF_SLOTS_I8 2
#endif

template <Act A, bool W8 = false, int SG = 1>
struct PfStage {
  static constexpr int ESZ = (A == Act::I8) ? 1 : 2;
  static constexpr int ROWB = kGroup * ESZ;
  static constexpr int A_BYTES = kPfRows * ROWB;
  static constexpr int TB = W8 ? 2 * kTileBytes : kTileBytes;
  static constexpr int W_OFF = A_BYTES;
  static constexpr int S_OFF = W_OFF + kPfCB * TB;
  static constexpr int Z_OFF = S_OFF + kPfCB * 32 * SG;
  static constexpr int R_OFF = S_OFF + (SG == 1 ? 512 : kPfCB * 32 * SG);
  static constexpr int BYTES = R_OFF + kPfRows * 4 * SG;
  // LDS ring depth (3 x 41 KB bf16; int8: Q4_PF_SLOTS_I8 x 25.6 KB, x 33.4 KB with 8-bit
  // weights)
  static constexpr int SLOTS = (A != Act::I8) ? 3 : (W8 && Q4_PF_SLOTS_I8 > 4) ? 4 : Q4_PF_SLOTS_I8;
};

// f(integral_constant<int, i>) for i = 0 .. N - 1, in order.
template <typename F, int... I>
Q4_DEVICE void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
Q4_DEVICE void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Work items (row tile, 128-column block) in tile-major order.  Workgroups are dispatched
// round-robin over the 8 XCDs (workgroup x runs on XCD x % 8); with a grid that is a
// multiple of 8, each XCD walks one contiguous range of items, so the column blocks that
// share an activation tile are computed under the same L2.
struct ItemRange {
  int64_t first, last, step;
};
Q4_DEVICE ItemRange item_range(int64_t items) {
  const int64_t nwg = gridDim.x;
  if (nwg % 8 != 0) return {int64_t(blockIdx.x), items, nwg};
  const int64_t chunk = (items + 7) / 8, xcd = blockIdx.x % 8;
  const int64_t last = std::min<int64_t>(items, (xcd + 1) * chunk);
  return {xcd * chunk + blockIdx.x / 8, last, nwg / 8};
}

template <Act A, int KIND, bool ASYM, bool W8, int SG>
__global__ void __launch_bounds__(256, (A == Act::I8) ? 2 : 1) k_gemm_pf(GemmArgs args) {
  static_assert(!W8 || (A == Act::I8 && !ASYM), "8-bit weights: symmetric, int8 activations");
  static_assert(SG == 1 || (!ASYM && !W8 && (SG == 2 || SG == 4)), "scale groups: symmetric 4-bit only");
  using St = PfStage<A, W8, SG>;
  constexpr int TB = St::TB;
  constexpr int WCOPIES = W8 ? 4 : 2;                 // 1 KB weight copies per wave per stage
  constexpr int ROWB = St::ROWB;
  constexpr int CHUNKS = ROWB / 16;                   // 16-byte chunks per row
  constexpr int ROWS_PER_INST = 64 / CHUNKS;          // rows one copy instruction covers
  constexpr int A_INSTS = 32 / ROWS_PER_INST;         // A copies per wave per stage (32 rows)
  constexpr bool RSUM = (A != Act::I8) || ASYM;
  // LDS slot of 16-byte chunk c of tile row r: c ^ swz(r).  A fragment read touches 16
  // rows (r % 16 = 0..15) at one chunk index: bf16 rows are 256 B (one bank period), so
  // XOR by r % 16 spreads them; int8 rows are 128 B, two rows per period, so rows of
  // equal parity are spread by (r / 2) % 8.
  auto swz = [](int r) -> int { return CHUNKS == 16 ? (r & 15) : ((r >> 1) & 7); };
  // ring of NS stage slots (the loop below is unrolled by NS so every slot offset is a
  // compile-time constant)
  constexpr int NS = St::SLOTS;
  __shared__ __align__(16) uint8_t ring[NS * St::BYTES];
  __shared__ float s_sa[kPfRows];   // int8: per-row activation scales of the item

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  // wave (wm, wn): row blocks {wm, wm + 2, wm + 4, wm + 6} (interleaved, so that a short
  // tile leaves both wave rows with work) and column blocks 4 wn .. 4 wn + 3
  const int wm = wid & 1, wn = wid >> 1;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t N = args.N, K = args.K;
  const int G = int(K / kGroup);
  const int64_t nblk = N / (16 * kPfCB);
  int64_t t_first = 0, ntiles = *args.num_tiles;   // several weight formats: this launch's tiles
  if (args.fmt_tiles) {
    t_first = args.fmt_tiles[args.fmt];
    ntiles = args.fmt_tiles[args.fmt_end] - t_first;
  }
  const int64_t items = ntiles * nblk;
  const int64_t w_scale_off = align256(W8 ? N * K : N * K / 2);
  const int64_t w_zero_off = w_scale_off + align256(2 * N * int64_t(G) * SG);
  const auto a_rsrc = buffer_rsrc(args.a, args.a_rows * K * St::ESZ);
  const void* rs_base = (A == Act::I8) ? static_cast<const void*>(args.a_qsum) : static_cast<const void*>(args.a_gsum);
  const auto r_rsrc = buffer_rsrc(rs_base, RSUM ? args.a_rows * G * SG * 4 : 0);

  const ItemRange ir = item_range(items);
  for (int64_t item = ir.first; item < ir.last; item += ir.step) {
    const int64_t tile = t_first + item / nblk;
    const int64_t cb0 = (item % nblk) * kPfCB;
    const TileDesc d = args.tiles[tile];
    if constexpr (A == Act::I8) __syncthreads();   // previous item's epilogue is done with s_sa
    const int64_t row_start = d.row_start;
    const int rows = d.rows;
    const bool shared = d.expert >= args.num_experts;
    typedef __attribute__((address_space(1))) const int64_t* gptr_i64;   // global (not flat) load
    int64_t woff = shared ? 0 : args.woffs ? ((gptr_i64)args.woffs)[d.expert] : int64_t(d.expert) * args.w_stride;
    woff = int64_t(uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(uint64_t(woff) >> 32)))) << 32 |
                   uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(woff))));   // wave-uniform
    const uint8_t* wbase = (shared ? args.w_shared : args.w) + woff;
    // bytes of one expert matrix in this kernel's format
    const int64_t w_bytes = w_scale_off + align256(2 * N * int64_t(G) * SG) + (ASYM ? align256(N * int64_t(G)) : 0);
    const auto w_rsrc = buffer_rsrc(wbase, w_bytes);
    auto src_of = [&](int r) -> int64_t {   // activation row of tile row r (clamped)
      const int64_t pos = row_start + (r < rows ? r : 0);
      return args.perm ? args.perm[pos] / args.slots_per_token : pos;
    };
    // per-lane byte offsets of this lane's copies (the stage adds a scalar offset)
    uint32_t a_off[A_INSTS];
#pragma unroll
    for (int j = 0; j < A_INSTS; ++j) {
      const int r = 32 * wid + ROWS_PER_INST * j + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ swz(r);         // global chunk that lands in this slot
      a_off[j] = uint32_t(src_of(r) * K * St::ESZ + c * 16);
    }
    // weight copies: column blocks 2 wid + (j / (WCOPIES / 2)), 1 KB part j % (WCOPIES / 2)
    uint32_t w_off[WCOPIES];
#pragma unroll
    for (int j = 0; j < WCOPIES; ++j)
      w_off[j] = uint32_t((cb0 + 2 * wid + j / (WCOPIES / 2)) * G * TB + (j % (WCOPIES / 2)) * kTileBytes + lane * 16);
    // wave 0: scales of the 8 blocks (lanes 0 .. 16 SG - 1, 32 SG bytes per block and
    // group) and zero points (lanes 16..23, 16 B per block and group; SG == 1)
    uint32_t m_off = 0, m_step = 0;
    if (lane < 16 * SG) {
      m_off = uint32_t(w_scale_off + (cb0 + lane / (2 * SG)) * G * 32 * SG + (lane % (2 * SG)) * 16);
      m_step = 32 * SG;
    } else if (SG == 1 && lane < 24) {
      m_off = uint32_t(w_zero_off + (cb0 + lane - 16) * G * 16);
      m_step = 16;
    }
    // waves 1 and 2: the row sums of tile rows (wid - 1) * 64 + lane
    uint32_t r_off = 0;
    if (RSUM && (wid == 1 || wid == 2)) r_off = uint32_t(src_of((wid - 1) * 64 + lane) * G * SG * 4);

    auto slot_of = [&](auto sl) -> uint8_t* { return ring + decltype(sl)::value * St::BYTES; };
    auto issue = [&](int g, auto sl) {
      const uint32_t base = lds_addr(slot_of(sl));
#pragma unroll
      for (int j = 0; j < A_INSTS; ++j)
        copy_to_lds<16>(a_rsrc, base + (32 * wid + ROWS_PER_INST * j) * ROWB, a_off[j], uint32_t(g * ROWB));
#pragma unroll
      for (int j = 0; j < WCOPIES; ++j)
        copy_to_lds<16>(w_rsrc, base + St::W_OFF + (2 * wid + j / (WCOPIES / 2)) * TB + (j % (WCOPIES / 2)) * kTileBytes,
                        w_off[j], uint32_t(g * TB));
      if (wid == 0 && (lane < 16 * SG || (ASYM && lane < 24)))
        copy_to_lds<16>(w_rsrc, base + St::S_OFF, m_off + uint32_t(g) * m_step, 0u);
      if constexpr (RSUM) {
        if (wid == 1 || wid == 2) {
#pragma unroll
          for (int j = 0; j < SG; ++j)
            copy_to_lds<4>(r_rsrc, base + St::R_OFF + j * 512 + (wid - 1) * 256, r_off + 4 * j, uint32_t(g * 4 * SG));
        }
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One group of one stage: the widened weight fragments of the wave's 4 column blocks
    // stay in registers; the activation fragments are read per row block.  Only the
    // wave's first NMB row blocks hold valid rows (NMB is fixed per work item, so the
    // step has no branches and the MFMAs of one row block overlap the scaling of another).
    auto compute = [&](auto sl, auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      const uint8_t* base = slot_of(sl);
      const uint16_t* s_sc = reinterpret_cast<const uint16_t*>(base + St::S_OFF);
      const uint8_t* s_z = base + St::Z_OFF;
      // Software pipeline over the (row block, column block) tiles of the stage: chunk
      // (mb, nb) issues the MFMAs of its tile, then the VALU work of the previous tile
      // (its rescale into the fp32 accumulators) and widens the next column block's
      // weights, so the matrix core and the VALU work at the same time.  A scheduling
      // fence closes every chunk (the compiler would otherwise hoist all MFMAs first).
      // pin(v): v is computed before this point; pass(x): x is (re)defined here, so
      // users of x cannot move above it.  Empty asm statements, no instructions.
      auto pin = [](const f32x4_t& v) { asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])); };
      auto pass = [](u32x4_t& x) { asm volatile("" : "+v"(x)); };
      auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
      uint4 wraw[4][W8 ? 2 : 1];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int hh = 0; hh < (W8 ? 2 : 1); ++hh)
          wraw[nb][hh] =
              *reinterpret_cast<const uint4*>(base + St::W_OFF + (wn * 4 + nb) * TB + hh * kTileBytes + lane * 16);
      if constexpr (SG > 1) {
        // Groups of 64 or 32 (SG scale entries per tile): one accumulator per scale group,
        // rescaled after its own MFMAs (a plain loop; groups of 128 take the pipelined
        // path below).
        const float* s_rs = reinterpret_cast<const float*>(base + St::R_OFF);
        if constexpr (A == Act::BF16) {
          constexpr int SPS = 4 / SG;
          u32x4_t b[4][4];
          float sc[4][SG];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const uint32_t w4[4] = {wraw[nb][0].x, wraw[nb][0].y, wraw[nb][0].z, wraw[nb][0].w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              uint32_t o[4];
              widen_word_fp<A>(w4[s], o);
              b[nb][s] = u32x4_t{o[0], o[1], o[2], o[3]};
            }
#pragma unroll
            for (int j = 0; j < SG; ++j) sc[nb][j] = f16_bits_to_f32(s_sc[((wn * 4 + nb) * 16 + col) * SG + j]);
          }
          const float negz = -(magic_offset<A>() + 8.0f);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const int rb = 2 * mb + wm;
            const int r = rb * 16 + col;
            u32x4_t af[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int c = (4 * s + kq) ^ swz(r);
              af[s] = *reinterpret_cast<const u32x4_t*>(base + r * ROWB + c * 16);
            }
            f32x4_t xv[SG];
#pragma unroll
            for (int j = 0; j < SG; ++j) xv[j] = *reinterpret_cast<const f32x4_t*>(s_rs + j * 128 + rb * 16 + 4 * kq);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
              for (int j = 0; j < SG; ++j) {
                f32x4_t g = xv[j] * negz;
#pragma unroll
                for (int s = j * SPS; s < (j + 1) * SPS; ++s) g = mfma16x16x32<A>(af[s], b[nb][s], g);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc[nb][j], g[i], acc[mb][nb][i]);
              }
          }
        } else {
          u32x4_t b[4][2];
          float sc16[4][SG];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            uint32_t o[8];
            widen_word_i8(wraw[nb][0].x, o[0], o[1]);
            widen_word_i8(wraw[nb][0].y, o[2], o[3]);
            widen_word_i8(wraw[nb][0].z, o[4], o[5]);
            widen_word_i8(wraw[nb][0].w, o[6], o[7]);
            b[nb][0] = u32x4_t{o[0], o[1], o[2], o[3]};
            b[nb][1] = u32x4_t{o[4], o[5], o[6], o[7]};
#pragma unroll
            for (int j = 0; j < SG; ++j)
              sc16[nb][j] = f16_bits_to_f32(s_sc[((wn * 4 + nb) * 16 + col) * SG + j]) * 0.0625f;
          }
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const int rb = 2 * mb + wm;
            const int r = rb * 16 + col;
            u32x4_t af[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int c1 = (4 * i + (kq >> 1)) ^ swz(r), c2 = (4 * i + 2 + (kq >> 1)) ^ swz(r);
              const uint2 lo = *reinterpret_cast<const uint2*>(base + r * ROWB + c1 * 16 + 8 * (kq & 1));
              const uint2 hi = *reinterpret_cast<const uint2*>(base + r * ROWB + c2 * 16 + 8 * (kq & 1));
              af[i] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                if constexpr (SG == 2) {
                  const i32x4_t ga = mfma_i8_16x16x64(af[h], b[nb][h], i32x4_t{0, 0, 0, 0});
#pragma unroll
                  for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc16[nb][h], float(ga[i]), acc[mb][nb][i]);
                } else {
#pragma unroll
                  for (int q = 0; q < 2; ++q) {
                    const i32x4_t ga = mfma_i8_16x16x32(af[h][2 * q], af[h][2 * q + 1], b[nb][h][2 * q],
                                                        b[nb][h][2 * q + 1], i32x4_t{0, 0, 0, 0});
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                      acc[mb][nb][i] = fmaf(sc16[nb][2 * h + q], float(ga[i]), acc[mb][nb][i]);
                  }
                }
              }
          }
        }
      } else if constexpr (A == Act::BF16) {
        float sc[4], negz[4];
        u32x4_t b[4][4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int cbl = wn * 4 + nb;
          sc[nb] = f16_bits_to_f32(s_sc[cbl * 16 + col]);
          negz[nb] = -(magic_offset<A>() + (ASYM ? float(s_z[cbl * 16 + col]) : 8.0f));
        }
        auto widen = [&](int nb) {
          const uint32_t w4[4] = {wraw[nb][0].x, wraw[nb][0].y, wraw[nb][0].z, wraw[nb][0].w};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint32_t o[4];
            widen_word_fp<A>(w4[s], o);
            b[nb][s] = u32x4_t{o[0], o[1], o[2], o[3]};
          }
        };
        const float* s_rs = reinterpret_cast<const float*>(base + St::R_OFF);
        auto read_a = [&](int mb, u32x4_t (&af)[4], f32x4_t& xv) {
          const int rb = 2 * mb + wm;
          const int r = rb * 16 + col;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int c = (4 * s + kq) ^ swz(r);
            af[s] = *reinterpret_cast<const u32x4_t*>(base + r * ROWB + c * 16);
          }
          xv = *reinterpret_cast<const f32x4_t*>(s_rs + rb * 16 + 4 * kq);
        };
        if constexpr (NMB > 0) {
          u32x4_t afc[4], afn[4];
          f32x4_t xvc, xvn;
          read_a(0, afc, xvc);
          widen(0);
          f32x4_t gt[4], gl;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
              for (int s = 0; s < 4; ++s) pass(b[nb][s]);
              f32x4_t g = xvc * negz[nb];
#pragma unroll
              for (int s = 0; s < 4; ++s) g = mfma16x16x32<A>(afc[s], b[nb][s], g);
              gt[nb] = g;
              if (mb == 0 && nb < 3) widen(nb + 1);
              if (nb == 0 && mb + 1 < NMB) read_a(mb + 1, afn, xvn);
              if (nb > 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb][nb - 1][i] = fmaf(sc[nb - 1], gt[nb - 1][i], acc[mb][nb - 1][i]);
                pin(acc[mb][nb - 1]);
              } else if (mb > 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb - 1][3][i] = fmaf(sc[3], gl[i], acc[mb - 1][3][i]);
                pin(acc[mb - 1][3]);
              }
              fence();
            }
            gl = gt[3];
#pragma unroll
            for (int s = 0; s < 4; ++s) afc[s] = afn[s];
            xvc = xvn;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[NMB - 1][3][i] = fmaf(sc[3], gl[i], acc[NMB - 1][3][i]);
        }
      } else {
        // 4-bit: widened codes are 16 (d - 8); s / 16 is exact in fp32, so scaling the
        // raw accumulator by s / 16 equals scaling the group sum by s.  8-bit: the codes
        // go to the matrix core as stored, the scale is s.
        float sc16[4];
        int32_t zoff16[4];
        u32x4_t b[4][2];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int cbl = wn * 4 + nb;
          sc16[nb] = f16_bits_to_f32(s_sc[cbl * 16 + col]) * (W8 ? 1.0f : 0.0625f);
          zoff16[nb] = ASYM ? 16 * (int32_t(s_z[cbl * 16 + col]) - 8) : 0;
        }
        auto widen = [&](int nb) {
          if constexpr (W8) {
            b[nb][0] = u32x4_t{wraw[nb][0].x, wraw[nb][0].y, wraw[nb][0].z, wraw[nb][0].w};
            b[nb][1] = u32x4_t{wraw[nb][1].x, wraw[nb][1].y, wraw[nb][1].z, wraw[nb][1].w};
          } else {
            uint32_t o[8];
            widen_word_i8(wraw[nb][0].x, o[0], o[1]);
            widen_word_i8(wraw[nb][0].y, o[2], o[3]);
            widen_word_i8(wraw[nb][0].z, o[4], o[5]);
            widen_word_i8(wraw[nb][0].w, o[6], o[7]);
            b[nb][0] = u32x4_t{o[0], o[1], o[2], o[3]};
            b[nb][1] = u32x4_t{o[4], o[5], o[6], o[7]};
          }
        };
        const int32_t* s_qs = reinterpret_cast<const int32_t*>(base + St::R_OFF);
        auto read_a = [&](int mb, u32x4_t (&af)[2], i32x4_t& qv) {
          const int rb = 2 * mb + wm;
          const int r = rb * 16 + col;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int c1 = (4 * i + (kq >> 1)) ^ swz(r), c2 = (4 * i + 2 + (kq >> 1)) ^ swz(r);
            const uint2 lo = *reinterpret_cast<const uint2*>(base + r * ROWB + c1 * 16 + 8 * (kq & 1));
            const uint2 hi = *reinterpret_cast<const uint2*>(base + r * ROWB + c2 * 16 + 8 * (kq & 1));
            af[i] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
          }
          if constexpr (ASYM) qv = *reinterpret_cast<const i32x4_t*>(s_qs + rb * 16 + 4 * kq);
        };
        auto rescale = [&](int mb, int nb, const i32x4_t& g_in, const i32x4_t& qv) {
          // the group sums enter the rescale through an empty asm statement: the
          // conversions cannot then be hoisted up to the MFMAs that produce them (which
          // made every rescale wait for its own tile's MFMA latency)
          i32x4_t g = g_in;
          asm volatile("" : "+v"(g));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int32_t a32 = g[i];
            if constexpr (ASYM) a32 -= zoff16[nb] * qv[i];
            acc[mb][nb][i] = fmaf(sc16[nb], float(a32), acc[mb][nb][i]);
          }
        };
        if constexpr (NMB > 0) {
          // Tiles t = 4 mb + nb in order; step t issues tile t's two MFMAs and rescales
          // tile t - 2, whose sums were ready a whole tile earlier, so the VALU work of a
          // step never waits for the matrix core (a ring of three pending sums).
          constexpr int NT = 4 * NMB;
          u32x4_t afc[2], afn[2];
          i32x4_t qvc = {0, 0, 0, 0}, qvn = {0, 0, 0, 0}, qvl = {0, 0, 0, 0};
          read_a(0, afc, qvc);
          widen(0);
          i32x4_t gq[3];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int mb = t / 4, nb = t % 4;
            pass(b[nb][0]);
            pass(b[nb][1]);
            i32x4_t g = {0, 0, 0, 0};
            g = mfma_i8_16x16x64(afc[0], b[nb][0], g);
            g = mfma_i8_16x16x64(afc[1], b[nb][1], g);
            gq[t % 3] = g;
            if (mb == 0 && nb < 3) widen(nb + 1);
            if (nb == 0 && mb + 1 < NMB) read_a(mb + 1, afn, qvn);
            if (t >= 2) {
              const int tp = t - 2, mp = tp / 4, np = tp % 4;
              rescale(mp, np, gq[tp % 3], mp == mb ? qvc : qvl);
              pin(acc[mp][np]);
            }
            // issue order inside the step: MFMA, VALU, MFMA, the rest
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
            fence();
            if (nb == 3) {
              qvl = qvc;
              afc[0] = afn[0];
              afc[1] = afn[1];
              qvc = qvn;
            }
          }
          // the last two tiles (qvl: the last row block's sums after the final swap)
          if constexpr (NT >= 2) rescale((NT - 2) / 4, (NT - 2) % 4, gq[(NT - 2) % 3], qvl);
          rescale((NT - 1) / 4, (NT - 1) % 4, gq[(NT - 1) % 3], qvl);
        }
      }
    };

    // NS-slot ring: while stage g is computed, stages g + 1 .. g + NS - 1 are in flight.
    // The copies of stage g + NS - 1 go to the slot that stage g - 1 used, which every
    // wave has finished reading (barrier at the end of the previous step).  Each wave
    // issues at least PER = A_INSTS + WCOPIES copies per stage and copies complete in order,
    // so after step g waiting until n * PER are outstanding (n = stages issued after
    // stage g + 1) leaves stage g + 1 complete; the barrier then publishes every wave's
    // copies.  (The raw barrier carries no wait of its own; the empty asm statements
    // keep the compiler from moving memory accesses across it.)
    constexpr int PER = A_INSTS + WCOPIES;
    auto sync = [&](int newer) {
      static_assert((NS - 2) * PER < 64, "vmcnt range");
      static_for<NS - 1>([&](auto u) {   // newer in 0 .. NS - 2 (wave-uniform)
        if (newer == decltype(u)::value) wait_vmcnt<decltype(u)::value * PER>();
      });
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    auto kloop = [&](auto nmb_c) {
      static_for<NS - 1>([&](auto u) {
        if (decltype(u)::value < G) issue(decltype(u)::value, u);
      });
      if constexpr (A == Act::I8) {
        // row scales for the epilogue (published by the barrier of the first sync)
        if (threadIdx.x < kPfRows) {
          const int r = int(threadIdx.x);
          s_sa[r] = r < rows ? args.a_scale[src_of(r)] : 0.f;
        }
      }
      sync(std::min(NS - 2, G - 1));
      for (int g0 = 0; g0 < G; g0 += NS) {
        bool done = false;
        static_for<NS>([&](auto u) {
          constexpr int U = decltype(u)::value;
          const int g = g0 + U;
          if (done || g >= G) {
            done = true;
            return;
          }
          if (g + NS - 1 < G) issue(g + NS - 1, std::integral_constant<int, (U + NS - 1) % NS>{});
          compute(u, nmb_c);
          sync(std::max(0, std::min(NS - 2, G - 2 - g)));
        });
      }
    };
    // row blocks 2 mb + wm (mb < nmb) hold valid rows; nmb is uniform within the wave
    const int nrb = (rows + 15) / 16;
    const int nmb = std::min(4, std::max(0, (nrb - wm + 1) / 2));
    switch (nmb) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // epilogue: row (2 mb + wm) * 16 + 4 kq + i, columns of blocks 4 wn + nb
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (2 * mb + wm) * 16 + 4 * kq + i;
        if (r >= rows) continue;
        const int64_t pos = row_start + r;
        float sa = 1.0f;
        if constexpr (A == Act::I8) sa = s_sa[r];
        if constexpr (KIND == GEMM_PLAIN) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            static_cast<float*>(args.out)[pos * N + (cb0 + wn * 4 + nb) * 16 + col] = acc[mb][nb][i] * sa;
        } else {
          const int64_t I = N / 2;
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float gg = acc[mb][2 * p][i] * sa, uu = acc[mb][2 * p + 1][i] * sa;
            const float hv = swiglu(gg, uu);
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

// bf16 prefill with wide tiles: 64 RG rows x 256 columns (16 column blocks) per
// workgroup of 4 RG waves (RG x 4 waves of 64 x 64).  RG = 2: 8 waves, a three-slot LDS
// ring of 49 KB stages (A 32 KB, W 16 KB, scales, zero points, row sums), one workgroup
// per CU; RG = 1: 4 waves on 64-row halves of the 128-row tiles, a two-slot ring of
// 33 KB stages, two workgroups per CU (the waves of one run while the other's wait at
// its per-group barrier).  Each wave walks the four 32-element K steps
// of a group outermost: only one K step's widened weights (16 registers) and the
// per-tile group accumulators are live, which keeps the kernel within 256 registers so
// two waves share each SIMD, and every activation byte copied to LDS feeds 256 columns.
// SG scale entries per tile (groups of 128 / SG): a scale group's accumulators are
// rescaled after its own K steps, so the register count does not depend on SG.
constexpr int kPfwCB = 16;

template <int KIND, bool ASYM, int SG, int RG>
__global__ void __launch_bounds__(256 * RG, RG == 1 ? 2 : 1) k_gemm_pf16w(GemmArgs args) {
  static_assert(RG == 1 || RG == 2, "row groups");
  static_assert(SG == 1 || (!ASYM && (SG == 2 || SG == 4)), "scale groups: symmetric weights only");
  constexpr int SPS = 4 / SG;                           // 32-element K steps per scale group
  constexpr int ROWB = kGroup * 2;                      // bf16 bytes of one row of a group
  constexpr int ROWS = 64 * RG;                         // rows per work item
  constexpr int NSUB = kPfRows / ROWS;                  // work items per 128-row tile
  constexpr int W_OFF = ROWS * ROWB;                    // 32 (16) KB of activations
  constexpr int S_OFF = W_OFF + kPfwCB * kTileBytes;    // 16 KB of weight tiles
  constexpr int Z_OFF = S_OFF + kPfwCB * 32 * SG;       // scales [16][16][SG] fp16
  constexpr int R_OFF = Z_OFF + (SG == 1 ? kPfwCB * 16 : 0);   // zero points [16][16] u8
  constexpr int BYTES = R_OFF + ROWS * 4 * SG;          // row sums [SG][ROWS] fp32
  constexpr int NS = RG == 1 ? 2 : 3;
  constexpr int A_INSTS = 4;                            // 16 rows per wave, 4 rows per copy
  constexpr int WCOPIES = 4 / RG;                       // 1 KB weight tiles per wave
  constexpr int PER = A_INSTS + WCOPIES;
  __shared__ __align__(16) uint8_t ring[NS * BYTES];
  auto swz = [](int r) -> int { return r & 15; };      // 256-byte rows: chunk c at c ^ (r % 16)

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  // row blocks RG mb + wm, column blocks 4 wn ..
  const int wm = RG == 1 ? 0 : (wid & 1), wn = RG == 1 ? wid : (wid >> 1);
  const int col = lane & 15, kq = lane >> 4;
  const int64_t N = args.N, K = args.K;
  const int G = int(K / kGroup);
  const int64_t nblk = N / (16 * kPfwCB);
  int64_t t_first = 0, ntiles = *args.num_tiles;
  if (args.fmt_tiles) {
    t_first = args.fmt_tiles[args.fmt];
    ntiles = args.fmt_tiles[args.fmt_end] - t_first;
  }
  const int64_t items = ntiles * NSUB * nblk;
  const int64_t w_scale_off = align256(N * K / 2);
  const int64_t w_zero_off = w_scale_off + align256(2 * N * int64_t(G));
  const auto a_rsrc = buffer_rsrc(args.a, args.a_rows * K * 2);
  const auto r_rsrc = buffer_rsrc(args.a_gsum, args.a_rows * G * SG * 4);

  const ItemRange ir = item_range(items);
  for (int64_t item = ir.first; item < ir.last; item += ir.step) {
    const int64_t tile = t_first + item / (NSUB * nblk);
    const int sub = int((item / nblk) % NSUB);
    const int64_t cb0 = (item % nblk) * kPfwCB;
    const TileDesc d = args.tiles[tile];
    const int64_t row_start = d.row_start + int64_t(sub) * ROWS;
    const int rows = std::min(ROWS, int(d.rows) - sub * ROWS);
    if (rows <= 0) continue;   // an empty second half (the whole workgroup skips it)
    const bool shared = d.expert >= args.num_experts;
    typedef __attribute__((address_space(1))) const int64_t* gptr_i64;
    int64_t woff = shared ? 0 : args.woffs ? ((gptr_i64)args.woffs)[d.expert] : int64_t(d.expert) * args.w_stride;
    woff = int64_t(uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(uint64_t(woff) >> 32)))) << 32 |
                   uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(woff))));
    const uint8_t* wbase = (shared ? args.w_shared : args.w) + woff;
    const int64_t w_bytes = w_scale_off + align256(2 * N * int64_t(G) * SG) + (ASYM ? align256(N * int64_t(G)) : 0);
    const auto w_rsrc = buffer_rsrc(wbase, w_bytes);
    auto src_of = [&](int r) -> int64_t {
      const int64_t pos = row_start + (r < rows ? r : 0);
      return args.perm ? args.perm[pos] / args.slots_per_token : pos;
    };
    // copies: activation rows 16 wid + 4 j + lane / 16 (chunk slot lane % 16), weight
    // tiles of column blocks WCOPIES wid + j
    uint32_t a_off[A_INSTS];
#pragma unroll
    for (int j = 0; j < A_INSTS; ++j) {
      const int r = 16 * wid + 4 * j + lane / 16;
      const int c = (lane % 16) ^ swz(r);
      a_off[j] = uint32_t(src_of(r) * K * 2 + c * 16);
    }
    uint32_t w_off[WCOPIES];
#pragma unroll
    for (int j = 0; j < WCOPIES; ++j) w_off[j] = uint32_t((cb0 + WCOPIES * wid + j) * G * kTileBytes + lane * 16);
    // scales, 32 SG bytes per block and group: wave 0 (16 B per lane; with four entries
    // per tile waves 0 and 3 copy 1 KB each); zero points: wave 0 lanes 32..47
    const int sidx = lane + (wid == 3 ? 64 : 0);
    const bool scale_lane = (wid == 0 && sidx < 32 * SG) || (SG == 4 && wid == 3);
    uint32_t m_off = 0, m_step = 0;
    if (scale_lane) {
      m_off = uint32_t(w_scale_off + (cb0 + sidx / (2 * SG)) * G * 32 * SG + (sidx % (2 * SG)) * 16);
      m_step = 32 * SG;
    } else if (SG == 1 && wid == 0 && lane >= 32 && lane < 48) {
      m_off = uint32_t(w_zero_off + (cb0 + lane - 32) * G * 16);
      m_step = 16;
    }
    // waves 1 .. RG: the row sums (one per scale group) of tile rows (wid - 1) * 64 + lane
    uint32_t r_off = 0;
    if (wid >= 1 && wid <= RG) r_off = uint32_t(src_of((wid - 1) * 64 + lane) * G * SG * 4);

    auto slot_of = [&](auto sl) -> uint8_t* { return ring + decltype(sl)::value * BYTES; };
    auto issue = [&](int g, auto sl) {
      const uint32_t base = lds_addr(slot_of(sl));
#pragma unroll
      for (int j = 0; j < A_INSTS; ++j) copy_to_lds<16>(a_rsrc, base + (16 * wid + 4 * j) * ROWB, a_off[j], uint32_t(g * ROWB));
#pragma unroll
      for (int j = 0; j < WCOPIES; ++j)
        copy_to_lds<16>(w_rsrc, base + W_OFF + (WCOPIES * wid + j) * kTileBytes, w_off[j],
                        uint32_t(g * kTileBytes));
      if (scale_lane || (ASYM && wid == 0 && lane < 48))
        copy_to_lds<16>(w_rsrc, base + S_OFF + (wid == 3 ? 1024 : 0), m_off + uint32_t(g) * m_step, 0u);
      if (wid >= 1 && wid <= RG) {
#pragma unroll
        for (int j = 0; j < SG; ++j)
          copy_to_lds<4>(r_rsrc, base + R_OFF + j * (ROWS * 4) + (wid - 1) * 256, r_off + 4 * j, uint32_t(g * 4 * SG));
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](auto sl, auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      if constexpr (NMB > 0) {
        const uint8_t* base = slot_of(sl);
        const uint16_t* s_sc = reinterpret_cast<const uint16_t*>(base + S_OFF);
        const uint8_t* s_z = base + Z_OFF;
        const float* s_rs = reinterpret_cast<const float*>(base + R_OFF);
        // scale j of column block 4 wn + nb (read when scale group j is rescaled)
        auto scale = [&](int nb, int j) -> float { return f16_bits_to_f32(s_sc[((wn * 4 + nb) * 16 + col) * SG + j]); };
        float negz[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          negz[nb] = -(magic_offset<Act::BF16>() + (ASYM ? float(s_z[(wn * 4 + nb) * 16 + col]) : 8.0f));
        const uint8_t* wl = base + W_OFF + wn * 4 * kTileBytes + lane * 16;   // word w of block nb at + nb KB + 4 w
        f32x4_t g[NMB][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s % SPS == 0) {
            // a scale group's accumulators start at -(magic + z) * (its row sum)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
              const f32x4_t xv =
                  *reinterpret_cast<const f32x4_t*>(s_rs + (s / SPS) * ROWS + (RG * mb + wm) * 16 + 4 * kq);
#pragma unroll
              for (int nb = 0; nb < 4; ++nb) g[mb][nb] = xv * negz[nb];
            }
          }
          // One scale entry per tile: lane quarter kq takes K step ws = (s + kq) % 4 at
          // step s (each quarter still covers the four steps once, and its A and B
          // fragments come from the same step), so the 64 lanes' 4-byte weight reads,
          // 16 bytes apart, fall in 64 distinct LDS banks; with several scale entries the
          // steps of a scale group must stay together, so every quarter takes step s.
          const int ws = SG == 1 ? ((s + kq) & 3) : s;
          // the step's activation fragments, then the weight blocks one at a time: block
          // nb + 1 is widened (VALU) while block nb's MFMAs run
          u32x4_t a[NMB];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const int r = (RG * mb + wm) * 16 + col;
            const int c = (4 * ws + kq) ^ swz(r);
            a[mb] = *reinterpret_cast<const u32x4_t*>(base + r * ROWB + c * 16);
          }
          auto widen_block = [&](int nb) -> u32x4_t {
            const uint32_t wd = *reinterpret_cast<const uint32_t*>(wl + nb * kTileBytes + 4 * ws);
            uint32_t o[4];
            widen_word_fp<Act::BF16>(wd, o);
            return u32x4_t{o[0], o[1], o[2], o[3]};
          };
          u32x4_t bc = widen_block(0);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const u32x4_t bn = nb < 3 ? widen_block(nb + 1) : bc;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) g[mb][nb] = mfma16x16x32<Act::BF16>(a[mb], bc, g[mb][nb]);
            // issue order: each MFMA followed by two VALU instructions (the next block's
            // widening), so the vector ALU works while the matrix core is busy
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
            bc = bn;
          }
          if (s % SPS == SPS - 1) {   // the scale group is complete: rescale into the totals
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const float sc = scale(nb, s / SPS);
#pragma unroll
              for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc, g[mb][nb][i], acc[mb][nb][i]);
            }
            // make the rescale happen here: otherwise the compiler sinks it past the
            // following scale groups and keeps all of their accumulators live
            if constexpr (SG > 1) {
#pragma unroll
              for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) asm volatile("" : "+v"(acc[mb][nb]));
            }
          }
        }
      }
    };

    auto sync = [&](int newer) {
      static_for<NS - 1>([&](auto u) {
        if (newer == decltype(u)::value) wait_vmcnt<decltype(u)::value * PER>();
      });
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    auto kloop = [&](auto nmb_c) {
      static_for<NS - 1>([&](auto u) {
        if (decltype(u)::value < G) issue(decltype(u)::value, u);
      });
      sync(std::min(NS - 2, G - 1));
      for (int g0 = 0; g0 < G; g0 += NS) {
        bool done = false;
        static_for<NS>([&](auto u) {
          constexpr int U = decltype(u)::value;
          const int g = g0 + U;
          if (done || g >= G) {
            done = true;
            return;
          }
          if (g + NS - 1 < G) issue(g + NS - 1, std::integral_constant<int, (U + NS - 1) % NS>{});
          compute(u, nmb_c);
          sync(std::max(0, std::min(NS - 2, G - 2 - g)));
        });
      }
    };
    const int nrb = (rows + 15) / 16;
    const int nmb = std::min(4, std::max(0, (nrb - wm + RG - 1) / RG));
    switch (nmb) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // epilogue: row (RG mb + wm) * 16 + 4 kq + i, columns of blocks cb0 + 4 wn + nb
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (RG * mb + wm) * 16 + 4 * kq + i;
        if (r >= rows) continue;
        const int64_t pos = row_start + r;
        if constexpr (KIND == GEMM_PLAIN) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            static_cast<float*>(args.out)[pos * N + (cb0 + wn * 4 + nb) * 16 + col] = acc[mb][nb][i];
        } else {
          const int64_t I = N / 2;
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float hv = swiglu(acc[mb][2 * p][i], acc[mb][2 * p + 1][i]);
            const int64_t hcol = ((cb0 + wn * 4) / 2 + p) * 16 + col;
            static_cast<uint16_t*>(args.out)[pos * I + hcol] = f32_to_bf16(hv);
          }
        }
      }
    }
  }
}

template <Act A, int KIND>
static hipError_t launch_pf_kind(const GemmArgs& g, hipStream_t st) {
  const int64_t nblk = g.N / (16 * kPfCB);
  const int64_t items = int64_t(g.max_tiles) * nblk;
  if (items == 0) return hipSuccess;
  const int64_t cap = (A == Act::I8) ? Q4_PF_GRID_I8 : 256;
  const unsigned grid = unsigned(std::min<int64_t>(items, cap));
  if (g.sg > 1 && (g.asym || g.wbits == 8)) return hipErrorInvalidValue;
  if constexpr (A == Act::BF16) {
    // wide tiles (8 waves, 128 x 256) when they still give every CU a work item
    const int64_t wblk = g.N / (16 * kPfwCB);
    if (g.N % (16 * kPfwCB) == 0 && int64_t(g.max_tiles) * wblk >= 256) {
      // gate/up (long K): 8-wave workgroups, each weight tile feeding 128 rows; the plain
      // (down) projection: two 4-wave workgroups per CU (256-expert T = 4096: gate/up
      // 3.08 -> 3.20 ms with 4-wave workgroups, down 1.63 -> 1.56 ms)
      constexpr int RG = KIND == GEMM_PLAIN ? 1 : 2;
      const unsigned wgrid = unsigned(std::min<int64_t>(int64_t(g.max_tiles) * (kPfRows / (64 * RG)) * wblk, 512 / RG));
      const dim3 blk(256 * RG);
      if (g.sg == 4)
        hipLaunchKernelGGL((k_gemm_pf16w<KIND, false, 4, RG>), dim3(wgrid), blk, 0, st, g);
      else if (g.sg == 2)
        hipLaunchKernelGGL((k_gemm_pf16w<KIND, false, 2, RG>), dim3(wgrid), blk, 0, st, g);
      else if (g.asym)
        hipLaunchKernelGGL((k_gemm_pf16w<KIND, true, 1, RG>), dim3(wgrid), blk, 0, st, g);
      else
        hipLaunchKernelGGL((k_gemm_pf16w<KIND, false, 1, RG>), dim3(wgrid), blk, 0, st, g);
      return hipGetLastError();
    }
  }
  if constexpr (A == Act::I8) {
    if (g.wbits == 8) {
      hipLaunchKernelGGL((k_gemm_pf<A, KIND, false, true, 1>), dim3(grid), dim3(256), 0, st, g);
      return hipGetLastError();
    }
  }
  if (g.sg == 4)
    hipLaunchKernelGGL((k_gemm_pf<A, KIND, false, false, 4>), dim3(grid), dim3(256), 0, st, g);
  else if (g.sg == 2)
    hipLaunchKernelGGL((k_gemm_pf<A, KIND, false, false, 2>), dim3(grid), dim3(256), 0, st, g);
  else if (g.asym)
    hipLaunchKernelGGL((k_gemm_pf<A, KIND, true, false, 1>), dim3(grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemm_pf<A, KIND, false, false, 1>), dim3(grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

bool prefill_fits(int64_t a_rows, int64_t K, int act, int64_t w_stride) {
  const int64_t esz = act == 2 ? 1 : 2;
  const int64_t lim = int64_t(1) << 31;
  return a_rows * K * esz < lim && a_rows * (K / kGroup) * 4 < lim && w_stride < lim;
}

hipError_t launch_gemm_prefill(const GemmArgs& g, int act, int kind, hipStream_t st) {
  if (g.N % (16 * kPfCB) != 0 || !g.tiles || !prefill_fits(g.a_rows, g.K, act, g.w_stride))
    return hipErrorInvalidValue;
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
