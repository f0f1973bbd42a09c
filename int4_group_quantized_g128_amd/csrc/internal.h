// Internal launcher declarations of the q4moe HIP library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>

namespace q4 {

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Row tile of the grouped GEMM: one 16-row MFMA block per row block.
struct TileDesc {
  int32_t expert;
  int32_t row_start;  // first position of the tile (index into perm / the row buffers)
  int32_t rows;       // valid rows in the tile
  int32_t pad;
};

hipError_t launch_quantize(const void* w, int dtype, int64_t n, int64_t k, int asym, uint8_t* packed,
                           uint16_t* scales, uint8_t* zeros, int32_t* flags, hipStream_t st);
hipError_t launch_repack(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros, int64_t n,
                         int64_t k, int asym, int gate_up, void* out, hipStream_t st, int group = 128);
// Groups of 32, 64 or 256 along K (128 goes to launch_quantize).
hipError_t launch_quantize_grouped(const void* w, int dtype, int64_t n, int64_t k, int group, int asym,
                                   uint8_t* packed, uint16_t* scales, uint8_t* zeros, int32_t* flags,
                                   hipStream_t st);

// INT8 g128 weights (W8A8): quantisation and device tiles (2 KB per (16-column block, group)).
hipError_t launch_quantize8(const void* w, int dtype, int64_t n, int64_t k, int8_t* q, uint16_t* scales,
                            int32_t* flags, hipStream_t st);
hipError_t launch_repack8(const int8_t* q, const uint16_t* scales, int64_t n, int64_t k, int gate_up, void* out,
                          hipStream_t st);

// 2-bit g128 weights (cold experts): quantisation and device tiles (512 B per
// (16-column block, group)).
hipError_t launch_quantize2(const void* w, int dtype, int64_t n, int64_t k, uint8_t* packed, uint16_t* scales,
                            int32_t* flags, hipStream_t st);
hipError_t launch_repack2(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int gate_up, void* out,
                          hipStream_t st);

// Router: fp32 logits split over kslices partial sums, then reduction + top-k; the
// workspace holds the partial sums (and for large batches the split weights).
int route_kslices(int64_t t, int64_t h, int32_t e);
size_t route_workspace_bytes(int64_t t, int64_t h, int32_t e);
hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int64_t t, int64_t h,
                        int32_t e, int32_t k, float* logits, int32_t* ids, float* w, float* partial,
                        hipStream_t st);

// Weight formats a layer may mix (tile order of the permutation): 4-bit with 1 / 2 / 4
// scale entries per tile, 8-bit, 2-bit.
constexpr int kNumFormats = 5;

// Permutation.  Slots s = t * S + j with S = k + shared; expert(s) = ids[t][j] for
// j < k, num_experts for the shared slot.  Optionally builds the row-tile list.
// scratch: permute_scratch_ints(t * (k + shared), e + shared) ints lets large batches use
// many workgroups (NULL: one workgroup at every size).
int64_t permute_scratch_ints(int64_t slots, int ee);
hipError_t launch_permute(const int32_t* ids, int64_t t, int32_t k, int32_t e, int shared, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, TileDesc* tiles, int32_t* num_tiles,
                          int tile_rows, hipStream_t st, const uint8_t* ebits = nullptr,
                          const uint8_t* egroups = nullptr, int32_t* fmt_tiles = nullptr, int32_t* scratch = nullptr,
                          int64_t scratch_ints = 0);

// Per-row INT8 activation quantisation (x: bf16 or fp32 rows).
hipError_t launch_act_quant(const void* x, int x_is_f32, int64_t rows, int64_t cols, int8_t* q, float* s,
                            int32_t* qsum, hipStream_t st);

// Grouped GEMM over INT4 device-layout weights.
struct GemmArgs {
  // activations
  const void* a;          // bf16 / f16 [rows][K] or int8 [rows][K]
  const float* a_scale;   // int8 mode: per-row scale
  const int32_t* a_qsum;  // int8 asymmetric prefill: per (row, group) code sums [rows][G]
  const float* a_gsum;    // bf16 prefill: per (row, group) activation sums [rows][G]
  int64_t a_rows;         // rows of the activation buffer(s) a / a_scale / a_qsum / a_gsum
  const int32_t* perm;    // position -> slot (gather rows), or NULL = identity
  int32_t slots_per_token;  // row = perm[p] / slots_per_token when perm != NULL
  // weights
  const uint8_t* w;       // routed experts: num_experts blocks of w_stride bytes
  int64_t w_stride;
  const uint8_t* w_shared;  // shared expert block (expert index == num_experts) or NULL
  int32_t num_experts;
  int32_t asym;
  int32_t wbits;          // 4 (INT4 tiles), 8 (INT8 tiles) or 2 (2-bit tiles); 8 and 2: int8 activations only
  const uint8_t* ebits;   // mixed layers: bits per expert (tiles of other experts are skipped), or NULL
  const int64_t* woffs;   // mixed layers: byte offset of each routed expert's block in w, or NULL
  const uint8_t* egroups; // per-expert group size / 32, or NULL
  int32_t sg;             // scale entries per 128-element tile of this launch (1, 2, 4; -1: per item)
  const int32_t* fmt_tiles;  // layers with several weight formats: tile range of each format [kNumFormats + 1], or NULL
  int32_t fmt, fmt_end;   // this launch's formats: tiles fmt_tiles[fmt] .. fmt_tiles[fmt_end]
                          //   (0..2: 4-bit with 1 / 2 / 4 scale entries per tile, 3: 8-bit, 4: 2-bit)
  int64_t N;              // device columns (2I for gate/up)
  int64_t K;
  // tiles
  const TileDesc* tiles;  // NULL = dense rows [0, dense_rows), or the slot tiles below
  const int32_t* slot_ids;  // tiles == NULL: tile i is slot i (one row) of expert slot_ids[i / S * slot_k + i % S]
                            //   (i % S == slot_k: the shared expert), S = slots_per_token, dense_rows slots; or NULL
  int32_t slot_k;
  int32_t src_div;        // perm == NULL: activation row = position / src_div (0 / 1: the position)
  int32_t built_rows;     // rows per tile as the permutation built them (0: the kernel's own);
                          //   taller tiles are walked in sub-tiles (streaming kernel only)
  const int32_t* num_tiles;
  int32_t max_tiles;
  int64_t dense_rows;
  // outputs
  void* out;              // gate/up: h [rows][N/2] (bf16, or fp32 in int8 mode); else fp32 [rows][N]
  int32_t ksplit;         // plain decode GEMM: K split over this many workgroups (0 / 1: none);
  int64_t out_slice;      //   slice s (groups [s G/ksplit, (s+1) G/ksplit)) writes out + s * out_slice
  int32_t* acc_out;       // debug: int32 [rows][N][G] group accumulators (int8 mode, plain)
  // plain streaming GEMM of a one-expert, one-choice layer without K slices: the
  // weighted combine in the epilogue, out_bf16[r][n] = bf16(combine_w[r] * y[r][n])
  const float* combine_w;
  uint16_t* out_bf16;
};

enum GemmKind { GEMM_PLAIN = 0, GEMM_GATE_UP = 1, GEMM_GROUP_ACC = 2 };

hipError_t launch_gemm(const GemmArgs& g, int act /*0 bf16, 1 f16, 2 i8*/, int kind, int row_blocks,
                       hipStream_t st);

// Prefill (128-row tiles, LDS-staged activations); tiles must be built with 128 rows.
// prefill_fits: the buffers stay within the kernel's 32-bit buffer offsets.
bool prefill_fits(int64_t a_rows, int64_t K, int act, int64_t w_stride);
hipError_t launch_gemm_prefill(const GemmArgs& g, int act /*0 bf16, 2 i8*/, int kind, hipStream_t st);
// Per-(row, group of 128 / sg) sums: bf16 -> fp32 (sg 1, 2, 4), or int8 -> int32 (sg 1).
hipError_t launch_rowsum(const void* a, int is_i8, int64_t rows, int64_t K, void* out, hipStream_t st, int sg = 1);

// Scale entries per 1 KB tile of an expert with the given group-size code (group / 32):
// 4 for groups of 32, 2 for 64, 1 for 128 and 256 (the 256-group's scale on both tiles).
__host__ __device__ inline int sg_of_code(int code) { return code == 1 ? 4 : code == 2 ? 2 : 1; }

// LoRA-mode experts (lora.hip).
hipError_t launch_dense_tiles(int64_t t, int tile_rows, TileDesc* tiles, int32_t* num_tiles, hipStream_t st);
hipError_t launch_lora_in(const uint16_t* x, int64_t t, int64_t h, const int32_t* ids, int32_t kk, int32_t e,
                          const uint16_t* a_gu, int r, float* a_part, hipStream_t st);
hipError_t launch_lora_mid(const float* base_gu, int64_t t, int64_t h, int64_t inter, const int32_t* ids,
                           const float* w, int32_t kk, int32_t e, int r, const float* a_part, const uint16_t* b_gate,
                           const uint16_t* b_up, const uint16_t* a_down, float* d_part, uint16_t* hw, hipStream_t st);
hipError_t launch_lora_out(const float* y, int64_t t, int64_t hidden, int64_t inter, const int32_t* ids,
                           const float* w, int32_t kk, int32_t e, int r, const float* d_part, const uint16_t* b_down,
                           uint16_t* out, hipStream_t st, int ncb = 0);
// Large batches, slots grouped by expert (tiles of the permutation, at most 64 slots
// each): h per slot and the down-adapter projections per 256-column block, then hw.
bool lora_grouped_rank(int r);
int lora_grp_col_blocks(int64_t inter);
hipError_t launch_lora_mid_grp(const float* base_gu, int64_t inter, const int32_t* perm, const TileDesc* tiles,
                               const int32_t* num_tiles, int32_t max_tiles, int32_t kk, int64_t h, int r,
                               const float* a_part, const uint16_t* b_gate, const uint16_t* b_up,
                               const uint16_t* a_down, float* d_part, float* h_slot, hipStream_t st);
hipError_t launch_lora_hsum(const float* h_slot, const float* w, int64_t t, int32_t kk, int64_t inter, uint16_t* hw,
                            float* rs, hipStream_t st);
int lora_kchunks(int64_t h);       // K chunks (512 wide) of the adapter input projections
int lora_col_blocks(int64_t inter);  // column blocks of the SwiGLU / down-projection kernel

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int64_t t, int32_t k, int shared,
                          int64_t h, uint16_t* out, hipStream_t st, int ksplit = 1, int64_t slice = 0);

}  // namespace q4
