/*
 * q4moe.h -- C ABI of the INT4 group-128 top-k MoE SwiGLU FFN forward for
 * AMD Instinct MI355X (gfx950).
 *
 * Method (pages cited by title and section):
 *  - "从FP32到INT4：大语言模型量化压缩实战指南" §1.3 (group-wise quantisation:
 *    group 128 along K, a per-group scale from the group's min/max, a zero point
 *    only in the asymmetric variant);
 *  - "高效大语言模型推理实践：INT4量化与MoE架构的融合探索", INT4量化实现 and
 *    MoE架构设计 (4-bit integers with an independent per-group scale; a MoE layer
 *    of small FFN experts chosen per input by a router; slice mode);
 *  - "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" §2.3 (W4A8: 4-bit
 *    storage widened to INT8, INT8 x INT8 -> INT32, rescale by
 *    scale_w * scale_a), §3.1 (per-token activation scale amax / 127, round,
 *    clamp to [-128, 127]), §3.2 (the router stays in floating point; the shared
 *    expert sees every token);
 *  - "大模型之Dense、MoE与量化", MoE section (a Linear router scores the
 *    experts, a few are chosen, outputs combined in proportion to the scores).
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev or documented as device pointers point to device
 *    memory of the current HIP device; the caller owns every buffer and the
 *    stream.  The library allocates no device memory and keeps no pointer after
 *    a call returns.  Work is enqueued on `stream` (may be NULL = default
 *    stream); no call synchronises the device unless stated.
 *  - Device pointers must be 16-byte aligned (128-bit loads), else
 *    Q4_ERR_ALIGN.  All validation happens on the host before any launch; a
 *    failed validation enqueues nothing.
 *  - Return value: Q4_OK or one of the error codes below; q4_last_error()
 *    gives a thread-local message for the last failing call.  No C++
 *    exception crosses this boundary.
 *  - Binary16 values travel as their uint16_t bit patterns, bf16 as uint16_t
 *    bit patterns.
 */
#ifndef Q4MOE_H
#define Q4MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* exported symbols (the library is built with hidden default visibility) */
#if defined(__GNUC__)
#define Q4_API __attribute__((visibility("default")))
#else
#define Q4_API
#endif

/* status codes */
#define Q4_OK 0
#define Q4_ERR_NULL 1        /* a required pointer is NULL                       */
#define Q4_ERR_SHAPE 2       /* K % 128 != 0, k > E, t < 0, unsupported sizes... */
#define Q4_ERR_ALIGN 3       /* a device pointer is not 16-byte aligned          */
#define Q4_ERR_DTYPE 4       /* unsupported dtype / mode value                   */
#define Q4_ERR_WORKSPACE 5   /* workspace or output buffer too small             */
#define Q4_ERR_UNSUPPORTED 6 /* a case this build does not implement             */
#define Q4_ERR_HIP 7         /* a HIP runtime / launch error                     */

/* dtypes */
#define Q4_F32 0
#define Q4_F16 1
#define Q4_BF16 2

/* forward modes */
#define Q4_W4A16 0 /* weights dequantised in-kernel, bf16 activations, fp32 accumulate */
#define Q4_W4A8 1  /* per-token INT8 activations x INT4->INT8 weights, INT32 per group   */
#define Q4_W8A8 2  /* per-token INT8 activations x INT8 weights (weight_bits == 8)        */

/* repack flags */
#define Q4_REPACK_PLAIN 0
#define Q4_REPACK_GATE_UP 1 /* input is [gate; up] stacked (2I rows); 16-column blocks interleaved */

/* quantize_int4_g128 status flags written to *flags_dev (bitwise OR) */
#define Q4_QFLAG_NONFINITE 1      /* a non-finite weight was seen (its group's codes are unspecified) */
#define Q4_QFLAG_SCALE_OVERFLOW 2 /* a group scale exceeds binary16 range                           */

/* Text of a status code; never NULL. */
Q4_API const char* q4_status_string(int status);

/* Thread-local message of the last failing call on this thread ("" if none). */
Q4_API const char* q4_last_error(void);

/* Library version, e.g. "q4moe 0.1 gfx950". */
Q4_API const char* q4_version(void);

/*
 * quantize_int4_g128 -- A1: INT4 group-128 quantisation into the canonical layout.
 * (FP32->INT4 guide §1.3; INT4量化实现 of the Efficient-LLM-Inference summary.)
 *
 *  w        device [n][k] weights of dtype w_dtype (Q4_F32, Q4_F16, Q4_BF16), row-major.
 *  n, k     rows (output channels) and reduction length; k % 128 == 0, n >= 1.
 *  asymmetric 0: scale s = fp16_rne(fp32(amax) / 7), q = clamp(rint(w / s), -8, 7),
 *              two's-complement nibbles;
 *             1: mn = min(min w, 0), mx = max(max w, 0), s = fp16 rounded up of
 *              fp32(mx - mn) / 15, z = clamp(rint(-mn / s), 0, 15),
 *              q = clamp(rint(w / s) + z, 0, 15).
 *             Divisions are IEEE fp32 divisions by the stored scale; rint is
 *             round-half-to-even; a zero scale gives codes (and zero point) 0.
 *  packed   device [n][k/2] bytes; byte j of a row holds k = 2j (low nibble) and 2j + 1.
 *  scales   device [n][k/128] binary16 bit patterns.
 *  zeros    device [n][ceil((k/128)/2)] bytes, two zero points per byte, even group in
 *           the low nibble, pad nibble 0; must be NULL iff asymmetric == 0.
 *  flags_dev optional device int32 (may be NULL): Q4_QFLAG_* bits are OR-ed in; the
 *           caller clears it beforehand.
 */
Q4_API int quantize_int4_g128(const void* w, int w_dtype, int64_t n, int64_t k, int asymmetric,
                       uint8_t* packed, uint16_t* scales, uint8_t* zeros, int32_t* flags_dev,
                       hipStream_t stream);

/*
 * q4_device_bytes / q4_repack_device -- A2: canonical layout -> device tile layout.
 * The pages fix only the canonical format (quantize_int4_g128); the device layout is
 * this library's own specification, made for the gfx950 kernels: 128-bit coalesced
 * loads, one 1 KB tile per wave load, nibble order matched to the register widening.
 * It is a fixed permutation of the canonical bytes (plus one byte per (column,
 * group) for asymmetric zero points):
 *  - columns: PLAIN keeps order; GATE_UP takes [gate; up] (n = 2I rows) and places
 *    gate rows [16b, 16b+16) in device block 2b, up rows [I+16b, I+16b+16) in 2b+1;
 *  - nibble value d = q + 8 (symmetric) or q (asymmetric);
 *  - weights: one 1024-byte tile per (16-column block cb, group g), cb-major;
 *    lane L in [0, 64) of a tile owns 16 bytes: column L % 16, quarter kq = L / 16;
 *    its 32-bit little-endian word s in [0, 4) holds k = 128 g + 32 s + 8 kq + e,
 *    e in [0, 8), element e at nibble position [0,2,4,6,1,3,5,7][e] (byte j of the
 *    word: element j in the low nibble, element j + 4 in the high nibble);
 *  - scales: binary16 [n/16][k/128][16] at byte align256(n k / 2);
 *  - zeros (asymmetric): one byte z per (column, group), [n/16][k/128][16], after the
 *    scales at the next 256-byte boundary.
 * Requirements: k % 128 == 0; n % 16 == 0 (PLAIN) or n % 32 == 0 (GATE_UP).
 * q4_device_bytes returns 0 for an unsupported shape.
 * dev_out: device buffer of at least q4_device_bytes(n, k, asymmetric) bytes
 * (Q4_ERR_WORKSPACE otherwise).
 */
Q4_API size_t q4_device_bytes(int64_t n, int64_t k, int asymmetric);
Q4_API int q4_repack_device(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                     int64_t n, int64_t k, int asymmetric, int flags, void* dev_out,
                     size_t dev_bytes, hipStream_t stream);

/*
 * quantize_int4_grouped / q4_device_bytes_grouped / q4_repack_device_grouped -- INT4
 * weights with groups of 32, 64, 128 or 256 along K (page "MoE推理优化实战：4bit存储+
 * INT8计算的W4A8路线解析", §5.3: the group size chosen per expert by how often it is
 * hit -- 32 for the hottest, 64 for ordinary, 128 or 256 for rarely used experts).
 * The same definitions as quantize_int4_g128 over groups of `group` elements; group
 * 128 gives exactly quantize_int4_g128 / q4_device_bytes / q4_repack_device.
 *  scales   device [n][k/group] binary16; zeros [n][ceil((k/group)/2)] (asymmetric).
 *  Requires group in {32, 64, 128, 256}, k % 128 == 0 and k % group == 0; zero points
 *  (asymmetric) only with groups of 128 or 256 (Q4_ERR_UNSUPPORTED otherwise).
 * Device layout: the weight tiles of q4_repack_device (they do not depend on the
 * group); scales binary16 [n/16][k/128][16][SG] (a column's entries of one tile
 * adjacent) with SG = 128 / group scale entries per 1 KB tile for groups of 32 or 64
 * (entry j covers k in [128 g + j 128/SG, 128 g + (j + 1) 128/SG)) and SG = 1
 * otherwise, a 256-group's
 * scale repeated on both of its tiles; zeros (asymmetric) one byte per (column,
 * tile), [n/16][k/128][16], the tile's group's zero point.
 */
Q4_API int quantize_int4_grouped(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group,
                                 int asymmetric, uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                                 int32_t* flags_dev, hipStream_t stream);
Q4_API size_t q4_device_bytes_grouped(int64_t n, int64_t k, int asymmetric, int32_t group);
Q4_API int q4_repack_device_grouped(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                                    int64_t n, int64_t k, int asymmetric, int32_t group, int flags,
                                    void* dev_out, size_t dev_bytes, hipStream_t stream);

/*
 * quantize_int8_g128 / q8_device_bytes / q8_repack_device -- INT8 g128 weights for the
 * W8A8 comparison route (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析":
 * W8A8 = INT8 weights and INT8 compute, the accuracy-safe route to set up first).
 * The same group structure as the INT4 format: per row and group of 128,
 * s = binary16 rounded up of fp32(amax) / 127, q = clamp(rint(w / s), -127, 127)
 * (IEEE fp32 division by the stored scale, half-to-even); a zero scale gives codes 0.
 *  q       device [n][k] int8 codes (canonical), scales device [n][k/128] binary16 bits.
 *  flags_dev as for quantize_int4_g128.
 * Device layout: one 2048-byte tile per (16-column block cb, group g), cb-major; the
 * tile is two 1024-byte halves (k in [128 g + 64 i, 128 g + 64 i + 64)), and inside a
 * half lane L (column L % 16, quarter kq = L / 16) owns 16 bytes: bytes 0..7 are
 * k = 128 g + 64 i + 8 kq + e, bytes 8..15 the same k + 32 (e in [0, 8)); scales
 * binary16 [n/16][k/128][16] at byte align256(n k).  Column orders as for
 * q4_repack_device (Q4_REPACK_PLAIN / Q4_REPACK_GATE_UP).
 */
Q4_API int quantize_int8_g128(const void* w, int w_dtype, int64_t n, int64_t k, int8_t* q,
                       uint16_t* scales, int32_t* flags_dev, hipStream_t stream);
Q4_API size_t q8_device_bytes(int64_t n, int64_t k);
Q4_API int q8_repack_device(const int8_t* q, const uint16_t* scales, int64_t n, int64_t k, int flags,
                     void* dev_out, size_t dev_bytes, hipStream_t stream);

/*
 * quantize_int2_g128 / q2_device_bytes / q2_repack_device -- 2-bit g128 weights for
 * rarely used ("cold") experts (page "大模型之Dense、MoE与量化", APEX section: experts
 * get precision by importance, commonly used ones 4 bits, cold ones 2 bits).  The INT4
 * format's structure with two bits: per row and group of 128, s = binary16 rounded up
 * of fp32(amax) (so |w / s| <= 1), q = clamp(rint(w / s), -2, 1) (IEEE fp32 division
 * by the stored scale, half-to-even; -2 is never produced); a zero scale gives codes 0.
 *  packed  device [n][k/4] bytes, four two's-complement codes per byte, k = 4 j + i in
 *          bits 2 i, 2 i + 1 of byte j.   scales device [n][k/128] binary16 bits.
 *  flags_dev as for quantize_int4_g128.
 * Device layout (this library's own): one 512-byte tile per (16-column block cb,
 * group g), cb-major; lane L (column L % 16, quarter kq = L / 16) owns 8 bytes, two
 * little-endian words; element k = 128 g + 32 s + 8 kq + e sits in word s / 2, byte
 * e % 4, bit field 2 (s % 2) + e / 4 (bits 2 f, 2 f + 1 of the byte) as d = q + 2.
 * Scales binary16 [n/16][k/128][16] at byte align256(n k / 4).  Column orders as for
 * q4_repack_device.
 */
Q4_API int quantize_int2_g128(const void* w, int w_dtype, int64_t n, int64_t k, uint8_t* packed, uint16_t* scales,
                              int32_t* flags_dev, hipStream_t stream);
Q4_API size_t q2_device_bytes(int64_t n, int64_t k);
Q4_API int q2_repack_device(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int flags,
                            void* dev_out, size_t dev_bytes, hipStream_t stream);

/*
 * moe_route_topk -- A3 + A4: fp32 router logits, top-k and renormalised weights.
 * (Dense/MoE page, MoE section: a Linear router; W4A8 page §3.2: router kept in float.)
 *
 *  x_bf16    device [t][h] bf16 tokens.
 *  w_router  device [e][h] fp32 router weight; bias: device [e] fp32 or NULL.
 *  logits_out device [t][e] fp32 (required): L = x W_r^T + b with exact products
 *            and fp32 sums.  From 512 tokens and 64 experts the sums run on the bf16
 *            matrix cores: each fp32 weight is split exactly into three bf16 parts
 *            (hi + mid + lo), and x is bf16, so every product stays exact.
 *  topk_ids  device [t][k] int32: experts by descending L, equal L -> lower index.
 *  topk_w    device [t][k] fp32: exp(L_j - L_max) / sum over the selected k
 *            (softmax over e, then renormalised over the selected k).
 *  workspace device buffer of moe_route_workspace_bytes(t, h, e) bytes (may be 0),
 *            16-byte aligned (Q4_ERR_ALIGN otherwise): K-slice partial sums and, for
 *            the large batches above, the three bf16 parts of w_router.
 *  Requires 1 <= k <= e <= 1024, h % 16 == 0, h >= 16; t == 0 is a no-op.
 *  NaN logits give unspecified ids.
 */
Q4_API size_t moe_route_workspace_bytes(int64_t t, int64_t h, int32_t e);
Q4_API int moe_route_topk(const uint16_t* x_bf16, const float* w_router, const float* bias, int64_t t,
                   int64_t h, int32_t e, int32_t k, float* logits_out, int32_t* topk_ids,
                   float* topk_w, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * moe_permute -- A5: group the t*k routed slots (slot s = t_idx * k + j) by expert
 * (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析", §1: routing dispatch sends
 * each token to its chosen experts and the results are combined afterwards; page
 * "大模型之Dense、MoE与量化", MoE section: the chosen experts process the token).  The
 * expert-grouped order lets each expert's rows be processed as one GEMM; the stable
 * order within an expert is this library's choice (any order is correct).
 *  ids     device [t][k] int32 in [0, e).
 *  counts  device [e] int32: slots per expert.
 *  offsets device [e + 1] int32: exclusive prefix sum of counts.
 *  perm    device [t*k] int32: position -> slot, sorted by expert, stable in slot order.
 *  inv     device [t*k] int32: slot -> position.
 *  Requires 1 <= k <= e <= 4096 and t*k < 2^31.  Ids outside [0, e) give unspecified
 *  results.
 */
Q4_API int moe_permute(const int32_t* ids, int64_t t, int32_t k, int32_t e, int32_t* counts,
                int32_t* offsets, int32_t* perm, int32_t* inv, hipStream_t stream);

/*
 * act_quant_int8 -- A6: per-row INT8 quantisation (W4A8 page §3.1).
 *  x       device [rows][cols] of dtype x_dtype (Q4_BF16 or Q4_F32).
 *  q       device [rows][cols] int8: clamp(rint(x / s), -128, 127).
 *  s       device [rows] fp32: s = amax / 127 (IEEE fp32 divisions); a zero row
 *          gets s = 0 and q = 0.
 *  Requires cols % 128 == 0.
 */
Q4_API int act_quant_int8(const void* x, int x_dtype, int64_t rows, int64_t cols, int8_t* q, float* s,
                   hipStream_t stream);

/*
 * Layer descriptor (host struct holding device pointers).
 *  num_experts, hidden (H), inter (I), top_k, asymmetric as named.
 *  gate_up: num_experts consecutive blocks of q4_device_bytes(2I, H, asymmetric) bytes,
 *           each repacked with Q4_REPACK_GATE_UP from the expert's [gate; up] rows.
 *  down:    num_experts consecutive blocks of q4_device_bytes(H, I, asymmetric) bytes
 *           (Q4_REPACK_PLAIN).
 *  (weight_bits == 8: the blocks are q8_device_bytes(2I, H) / q8_device_bytes(H, I)
 *           bytes of q8_repack_device output instead.)
 *  shared_inter: 0 = no shared expert; else the shared expert's intermediate size,
 *           which must equal inter in this build; shared_gate_up / shared_down are
 *           one block each, laid out as above.
 */
typedef struct q4_moe_layer_t {
  int32_t num_experts;
  int32_t hidden;
  int32_t inter;
  int32_t top_k;
  int32_t asymmetric;
  int32_t shared_inter;
  const void* gate_up;
  const void* down;
  const void* shared_gate_up;
  const void* shared_down;
  int32_t weight_bits;   /* 0 or 4: INT4 device layout (modes W4A16 / W4A8); 8: INT8 device
                            layout of q8_repack_device, symmetric, mode Q4_W8A8 only */
  /* Mixed layers (per-expert bit width; page "大模型之Dense、MoE与量化", APEX: experts get
   * different precisions by importance).  When expert_bits != NULL: weight_bits must be
   * 0, asymmetric 0 and mode Q4_W4A8 (INT8 activations for every expert); expert e's
   * gate/up block starts at byte gate_up_offsets[e] of gate_up (down: down_offsets[e]
   * of down) and holds q4_device_bytes(., ., 0), q8_device_bytes(., .) or
   * q2_device_bytes(., .) bytes by its bits; the shared expert's bits are
   * expert_bits[num_experts].  2-bit experts (group 128) run on the streaming GEMM
   * kernel at every batch size. */
  const uint8_t* expert_bits;      /* device [num_experts + shared] values 2, 4 or 8 */
  const int64_t* gate_up_offsets;  /* device [num_experts] */
  const int64_t* down_offsets;     /* device [num_experts] */
  /* Per-expert group size (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析",
   * §5.3: smaller groups for hotter experts).  When expert_groups != NULL: weight_bits
   * 0, asymmetric 0, the block offsets above are required, and expert e's blocks hold
   * q4_repack_device_grouped output for its group (q4_device_bytes_grouped(2I, H, 0,
   * group) and (H, I, 0, group) bytes); modes W4A16 and W4A8 (W4A8 only if expert_bits
   * is also given, in which case 8-bit experts must have group 128).  The values are
   * the group size / 32 (1, 2, 4 or 8); the shared expert's is expert_groups[num_experts].
   * Any value other than 1 or 2 is read as one scale entry per tile (groups of 128 or
   * 256).  The forward orders the row tiles by weight format and runs each GEMM once
   * per format present in the layer's description. */
  const uint8_t* expert_groups;    /* device [num_experts + shared] values 1, 2, 4 or 8 */
} q4_moe_layer_t;

/*
 * moe_int4_ffn_forward -- A5..A11: the MoE SwiGLU FFN forward.
 *   out[t] = sum_j topk_w[t, j] * FFN_{ids[t, j]}(x[t])  (+ FFN_shared(x[t]))
 *   FFN(v) = down(silu(gate v) * up v)
 * W4A16: weights dequantised in registers; products in bf16 MFMA with fp32
 *   accumulation, one fp32 scale step per group; h rounded to bf16.
 * W4A8: x quantised per token and h per (token, choice) row to INT8 (amax / 127);
 *   INT32 accumulation per group of int8(x) * (q - z); y = s_x * sum_g s_w * acc.
 * W8A8 (layer weight_bits == 8): the same with the 8-bit codes q.
 * The combine adds the k routed outputs in ascending j in fp32, then the shared
 * expert, then rounds to bf16.  For narrow layers at small t (touched experts x H / 32
 * under 512 work items) the down projection splits K over up to 8 workgroups and each
 * routed output is the fp32 sum of its slices, in slice order (the workspace holds the
 * slices).  A dense SwiGLU FFN is the case num_experts = 1,
 * top_k = 1, topk_w = 1.
 *
 *  x_bf16   device [t][H] bf16; out_bf16 device [t][H] bf16 (may not alias x).
 *  topk_ids device [t][top_k] int32 in [0, num_experts); topk_w device [t][top_k] fp32.
 *  workspace device buffer of moe_int4_ffn_workspace_bytes(L, t, mode) bytes.
 *  Requires H % 128 == 0, I % 128 == 0, 1 <= top_k <= num_experts <= 4096.
 *  t == 0 is a no-op.  Ids outside range give unspecified results.
 */
Q4_API size_t moe_int4_ffn_workspace_bytes(const q4_moe_layer_t* layer, int64_t t, int mode);
Q4_API int moe_int4_ffn_forward(const q4_moe_layer_t* layer, const uint16_t* x_bf16, int64_t t,
                         const int32_t* topk_ids, const float* topk_w, int mode,
                         uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/*
 * moe_int4_ffn_debug -- moe_int4_ffn_forward (same arguments, the same launches and
 * the same results) that also returns views of its intermediates, for stage-by-stage
 * parity checks: the INT8 codes and scales of x and h (page "MoE推理优化实战：4bit存储+
 * INT8计算的W4A8路线解析" §3, per-token activation quantisation) and the per-position
 * expert outputs before the weighted combine (page "大模型之Dense、MoE与量化", MoE
 * section).
 * On success `views` points into `workspace` (valid once the stream has executed the
 * call, until the workspace is reused); P = t * slots_per_token positions, position
 * p holds slot perm[p] = token * slots_per_token + j (j == top_k: the shared expert):
 *   counts [E + shared] int32, offsets [E + shared + 1] int32, perm / inv [P] int32;
 *   h   [P][I]: silu(gate) * up per position, bf16 (W4A16) or fp32 (W4A8);
 *   y   [y_slices][P][H] fp32: the down projection per position, as y_slices partial
 *       sums over consecutive K ranges of y_slice_groups groups each (y_slices == 1
 *       except where the forward splits the down projection's K, see
 *       moe_int4_ffn_forward); the routed output of a position is the fp32 sum of its
 *       slices in slice order;
 *   q_x [t][H] int8, s_x [t] fp32, q_h [P][I] int8, s_h [P] fp32 (W4A8; NULL in W4A16).
 * For a one-expert layer at decode sizes and for a single token (rows_in_token_order,
 * slot_tiles of moe_int4_ffn_plan) the debug call also runs the permutation, for its
 * views, and (one-expert layer) keeps y in the workspace with the combine as a launch of
 * its own (the same arithmetic, so the same results).
 * The gate and up products before SwiGLU are not stored by the fused kernel; the same
 * GEMM core gives them on the forward's own inputs: int4_linear_forward (W4A16, fp32
 * g and u) and int4_w4a8_group_acc (the INT32 group accumulators of either GEMM) on an
 * expert's gate/up or down block of the layer (a Q4_REPACK_GATE_UP block is read as a
 * PLAIN [2I][H] matrix whose 16-column block 2b holds gate rows 16b.., block 2b + 1
 * up rows 16b..).
 * views == NULL -> Q4_ERR_NULL; on any error *views is zeroed.
 */
typedef struct q4_ffn_views_t {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* inv;
  const void* h;
  int32_t h_is_f32;
  int32_t slots_per_token;
  int64_t positions;
  const float* y;
  const int8_t* q_x;
  const float* s_x;
  const int8_t* q_h;
  const float* s_h;
  int32_t y_slices;        /* K slices of the down projection held in y (1: whole rows) */
  int32_t y_slice_groups;  /* groups of 128 per slice: slice s covers groups
                              [s * y_slice_groups, min(I / 128, (s + 1) * y_slice_groups)) */
  int64_t y_slice_stride;  /* floats between slices (= positions * H) */
} q4_ffn_views_t;
Q4_API int moe_int4_ffn_debug(const q4_moe_layer_t* layer, const uint16_t* x_bf16, int64_t t,
                       const int32_t* topk_ids, const float* topk_w, int mode,
                       uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                       q4_ffn_views_t* views, hipStream_t stream);

/*
 * moe_int4_ffn_forward_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_int4_ffn_forward with the same arguments minus the workspace.  Its workspace is
 * a file-scope device array of Q4_NOALLOC_SCRATCH_BYTES in the library, one per GPU,
 * held until the process ends; the call allocates nothing (no hipMalloc / hipFree,
 * no allocating library routine).  Batches whose workspace
 * (moe_int4_ffn_workspace_bytes) exceeds that size return Q4_ERR_WORKSPACE.  Every
 * call on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  The first call
 * on a device looks up the array's device address (hipGetSymbolAddress).
 * Results equal moe_int4_ffn_forward's bit for bit (same kernels).
 */
#define Q4_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
#define Q4_MAX_DEVICES 64
Q4_API int moe_int4_ffn_forward_noalloc(const q4_moe_layer_t* layer, const uint16_t* x_bf16, int64_t t,
                                        const int32_t* topk_ids, const float* topk_w, int mode,
                                        uint16_t* out_bf16, hipStream_t stream);

/*
 * moe_int4_ffn_plan -- host-only query of the launch plan moe_int4_ffn_forward uses
 * for (layer, t, mode); no device work, no pointer is dereferenced except layer.
 *  kernel         Q4_PLAN_DECODE: the streaming GEMM kernel with 16 / 32 / 64-row tiles
 *                 (tile_rows), or Q4_PLAN_PREFILL: the 128-row matrix-core tiles staged
 *                 through LDS.  The prefill tiles are chosen from 64 routed rows per
 *                 expert on average, or from 17 (9 with INT8 activations) when the
 *                 launch has at least 2048 estimated gate/up work items, but only where
 *                 every activation buffer of the launch is below 2^31 bytes (the
 *                 prefill kernels address activations with 32-bit buffer offsets);
 *                 beyond that the decode kernel (64-bit addressing) runs and
 *                 prefill_addr_limited is 1.
 *  down_ksplit    K slices of the down projection (1: none).
 *  rows_in_token_order 1 for a one-expert, one-choice layer without a shared expert (a
 *                 dense SwiGLU FFN) at decode sizes: no permutation launch, the GEMMs
 *                 read and write rows in token order;
 *  combine_in_down 1 when, in addition, the down projection has no K slices: its
 *                 epilogue applies the weight and rounds to bf16 (no combine launch).
 *  slot_tiles     1 for a single token (t == 1) on any other layer with one weight
 *                 format at decode sizes: its slots have distinct experts, so each
 *                 slot is its own one-row tile taken straight from topk_ids (no
 *                 permutation launch; rows and y stay in slot order).  The results equal
 *                 the permuted path's bit for bit.
 *  workspace_bytes moe_int4_ffn_workspace_bytes(layer, t, mode).
 * Errors as moe_int4_ffn_forward's validation (the layer's device pointers are checked
 * for NULL and alignment only).
 */
#define Q4_PLAN_DECODE 0
#define Q4_PLAN_PREFILL 1
typedef struct q4_ffn_plan_t {
  int32_t kernel;
  int32_t tile_rows;
  int32_t down_ksplit;
  int32_t prefill_addr_limited;
  int32_t rows_in_token_order;
  int32_t combine_in_down;
  int32_t slot_tiles;
  int64_t workspace_bytes;
} q4_ffn_plan_t;
Q4_API int moe_int4_ffn_plan(const q4_moe_layer_t* layer, int64_t t, int mode, q4_ffn_plan_t* plan);

/*
 * moe_expert_bits_by_hotness / moe_expert_groups_by_hotness -- per-expert weight format
 * from routing hit counts (host arrays; counts[e] = routed slots of expert e over a
 * calibration batch, e.g. the counts moe_permute returns).  Page "MoE推理优化实战：4bit存储
 * +INT8计算的W4A8路线解析", §5.3: the most frequently hit experts, its top 5 %, keep more
 * precision (finer groups); ordinary experts groups of 64; experts almost no token
 * reaches 128 or even 256; §6.1: a W8 / W4 choice per expert; page "大模型之Dense、MoE与
 * 量化", APEX: expert precision by importance.  Hit counts stand in for importance.
 *  bits:   the ceil(frac8 * e) most-hit experts (equal counts: lower index first) 8,
 *          the others 4; with shared != 0 one more entry, 8, for the shared expert
 *          (hit by every token).
 *  groups: the ceil(hot_frac * e) most-hit experts 32; of the others, experts with
 *          counts[i] * e < cold_share * sum(counts) 256, the rest 64; shared: 32.
 *  The ceil is of (fraction * e - 1e-9) in double precision.  Output arrays hold
 *  e + (shared != 0) entries.  Requires 1 <= e <= 4096, counts >= 0, fractions in
 *  [0, 1], cold_share >= 0.
 */
Q4_API int moe_expert_bits_by_hotness(const int64_t* counts, int32_t e, double frac8, int shared, int32_t* bits_out);
Q4_API int moe_expert_groups_by_hotness(const int64_t* counts, int32_t e, double hot_frac, double cold_share,
                                        int shared, int32_t* groups_out);
/*  bits (APEX): experts with counts[i] * e < cold_share * sum(counts) 2 bits, the
 *          ceil(frac8 * e) most-hit experts 8 bits (over the cold rule), the others 4;
 *          shared: 8 if frac8 > 0, else 4. */
Q4_API int moe_expert_bits_apex(const int64_t* counts, int32_t e, double frac8, double cold_share, int shared,
                                int32_t* bits_out);

/*
 * q4_lora_layer_t / moe_lora_ffn_forward -- LoRA-mode experts (page
 * "高效大语言模型推理实践：INT4量化与MoE架构的融合探索", 第三阶段: experts built from LoRA
 * adapters on frozen dense weights).  Expert e of matrix m in {gate, up, down} is
 * W_hat_m + B_m,e A_m,e with W_hat_m one shared INT4 g128 dense matrix and rank-r
 * bf16 adapters (any LoRA scaling folded into B);
 *   out[t] = sum_j topk_w[t, j] * FFN_{ids[t, j]}(x[t]),
 *   FFN_e(v) = W_down,e (silu(W_gate,e v) * (W_up,e v)).
 * Computed as: INT4 base gate/up GEMM once per token (fp32); per slot the rank-r
 * updates B (A x) and SwiGLU (fp32); hw = sum_j w_j h_j rounded to bf16; INT4 base
 * down GEMM once per token on hw (fp32); plus sum_j w_j B_down (A_down h_j); the
 * output rounded to bf16.  W4A16 arithmetic (bf16 activations into the base GEMMs).
 *
 *  base_gate_up  device layout (Q4_REPACK_PLAIN) of [gate; up], 2I x H.
 *  base_down     device layout (Q4_REPACK_PLAIN), H x I.
 *  a_gate_up     bf16 [E][2r][H]: rows [0, r) A_gate,e, rows [r, 2r) A_up,e.
 *  b_gate, b_up  bf16 [E][I][r].    a_down  bf16 [E][r][I].    b_down  bf16 [E][H][r].
 *  Requires H % 128 == 0, I % 128 == 0, rank in {8, 16, ..., 64},
 *  1 <= top_k <= num_experts <= 4096; all pointers 16-byte aligned.
 *  x_bf16 [t][H], topk_ids / topk_w [t][top_k], out_bf16 [t][H] (may not alias x);
 *  workspace of moe_lora_ffn_workspace_bytes(layer, t) bytes.  t == 0 is a no-op.
 */
typedef struct q4_lora_layer_t {
  int32_t num_experts;
  int32_t hidden;
  int32_t inter;
  int32_t top_k;
  int32_t rank;
  int32_t asymmetric;
  const void* base_gate_up;
  const void* base_down;
  const uint16_t* a_gate_up;
  const uint16_t* b_gate;
  const uint16_t* b_up;
  const uint16_t* a_down;
  const uint16_t* b_down;
} q4_lora_layer_t;
Q4_API size_t moe_lora_ffn_workspace_bytes(const q4_lora_layer_t* layer, int64_t t);
Q4_API int moe_lora_ffn_forward(const q4_lora_layer_t* layer, const uint16_t* x_bf16, int64_t t,
                         const int32_t* topk_ids, const float* topk_w, uint16_t* out_bf16,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * int4_linear_forward -- one INT4 g128 linear y = x W_hat^T (fp32 output), the
 * W4A16 core on a plain token matrix (page "从FP32到INT4：大语言模型量化压缩实战指南",
 * §1.3: a linear layer's weight quantised in groups of 128 along K, each group
 * dequantised with its own scale and zero point; page "MoE推理优化实战：4bit存储+INT8
 * 计算的W4A8路线解析", §2.1: W4A16 keeps activations in 16 bits and dequantises the
 * 4-bit weights for the product).
 *  x      device [t][k], dtype Q4_F16 or Q4_BF16.
 *  w_dev  device layout (Q4_REPACK_PLAIN) of an [n][k] matrix.
 *  y      device [t][n] fp32.
 *  Requires k % 128 == 0, n % 64 == 0.
 */
Q4_API int int4_linear_forward(const void* x, int x_dtype, int64_t t, int64_t k, const void* w_dev,
                        int64_t n, int asymmetric, float* y, hipStream_t stream);

/*
 * int4_w4a8_group_acc -- A11 debug view: the per-group INT32 accumulators of the
 * W4A8 core, acc[r][c][g] = sum_{k in group g} q[r][k] * (code[c][k] - z[c][g]),
 * computed by the same MFMA core as moe_int4_ffn_forward.
 *  q      device [rows][k] int8 activation codes.
 *  w_dev  device layout (Q4_REPACK_PLAIN) of an [n][k] matrix.
 *  acc    device [rows][n][k/128] int32.
 *  Requires k % 128 == 0, n % 64 == 0.
 */
Q4_API int int4_w4a8_group_acc(const int8_t* q, int64_t rows, int64_t k, const void* w_dev, int64_t n,
                        int asymmetric, int32_t* acc, hipStream_t stream);

/*
 * int2_w2a8_group_acc -- the INT32 group accumulators of the 2-bit core,
 * acc[r][c][g] = sum_{k in group g} q[r][k] * code[c][k], same MFMA core as the forward.
 *  q      device [rows][k] int8 activation codes.
 *  w_dev  q2_repack_device output (Q4_REPACK_PLAIN) of an [n][k] matrix.
 *  acc    device [rows][n][k/128] int32.   Requires k % 128 == 0, n % 64 == 0.
 */
Q4_API int int2_w2a8_group_acc(const int8_t* q, int64_t rows, int64_t k, const void* w_dev, int64_t n,
                               int32_t* acc, hipStream_t stream);

/*
 * int8_w8a8_group_acc -- the INT32 group accumulators of the W8A8 core,
 * acc[r][c][g] = sum_{k in group g} q[r][k] * code[c][k], same MFMA core as the forward.
 *  q      device [rows][k] int8 activation codes.
 *  w_dev  q8_repack_device output (Q4_REPACK_PLAIN) of an [n][k] matrix.
 *  acc    device [rows][n][k/128] int32.   Requires k % 128 == 0, n % 64 == 0.
 */
Q4_API int int8_w8a8_group_acc(const int8_t* q, int64_t rows, int64_t k, const void* w_dev, int64_t n,
                        int32_t* acc, hipStream_t stream);

/*
 * q4_set_stage_events -- optional per-stage timing markers for profiling tools.
 * When set (count >= Q4_NUM_STAGES, non-NULL arrays), every later
 * moe_int4_ffn_forward call on this thread records begin[s] before and end[s] after
 * the launches of stage s on its stream (hipEventRecord), for the stages it runs.
 * The events (hipEvent_t handles) are owned by the caller and must outlive their
 * use.  count == 0 or NULL arrays disable the markers.  Thread-local.
 */
#define Q4_STAGE_PERMUTE 0
#define Q4_STAGE_X_QUANT 1
#define Q4_STAGE_GATE_UP 2
#define Q4_STAGE_H_QUANT 3
#define Q4_STAGE_DOWN 4
#define Q4_STAGE_COMBINE 5
#define Q4_NUM_STAGES 6
Q4_API int q4_set_stage_events(void* const* begin, void* const* end, int count);

#ifdef __cplusplus
}
#endif
#endif /* Q4MOE_H */
