// C ABI of the q4moe library: host-side validation, workspace carving and the
// launch sequence of each entry point.  Declarations and contracts: include/q4moe.h.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/q4moe.h"
#include "internal.h"

using namespace q4;

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_stage_begin[Q4_NUM_STAGES];
thread_local hipEvent_t g_stage_end[Q4_NUM_STAGES];
thread_local bool g_stage_events = false;

void stage_begin(int s, hipStream_t st) {
  if (g_stage_events) (void)hipEventRecord(g_stage_begin[s], st);
}
void stage_end(int s, hipStream_t st) {
  if (g_stage_events) (void)hipEventRecord(g_stage_end[s], st);
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() { return Q4_OK; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define Q4_REQUIRE(cond, code, ...) \
  do {                              \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int64_t a256(int64_t x) { return align256(x); }

// Carves the forward workspace; with base == nullptr only the size is computed.
struct FwdWorkspace {
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* perm = nullptr;
  int32_t* inv = nullptr;
  TileDesc* tiles = nullptr;
  int32_t* num_tiles = nullptr;
  int32_t* fmt_tiles = nullptr;   // [kNumFormats + 1] tile range of each weight format
  int32_t* perm_scratch = nullptr;   // per-range expert counts of the many-workgroup permutation
  int64_t perm_scratch_ints = 0;
  void* h = nullptr;
  float* y = nullptr;
  int8_t* qx = nullptr;
  float* sx = nullptr;
  int8_t* qh = nullptr;
  float* sh = nullptr;
  void* rs_x = nullptr;   // prefill: per (token, group) sums of x (fp32) or of q_x (int32)
  void* rs_h = nullptr;   // prefill: per (position, group) sums of h / q_h
  bool prefill = false;
  int64_t bytes = 0;
  int32_t max_tiles = 0;
  int tile_rows = 16;
  int ksplit = 1;   // K slices of the down projection (y holds ksplit partial slices)
};

bool int8_acts(int mode) { return mode == Q4_W4A8 || mode == Q4_W8A8; }
int wbits_of(const q4_moe_layer_t* L) { return L->weight_bits == 8 ? 8 : 4; }

// Device bytes of one [n][k] expert matrix in the layer's weight format (the larger,
// 8-bit, size for mixed layers).
int64_t mat_bytes(const q4_moe_layer_t* L, int64_t n, int64_t k) {
  if (wbits_of(L) == 8 || L->expert_bits) return int64_t(q8_device_bytes(n, k));
  if (L->expert_groups) return int64_t(q4_device_bytes_grouped(n, k, 0, 32));   // the largest scale table
  return int64_t(q4_device_bytes(n, k, L->asymmetric));
}

// Arithmetic modes a layer supports.
bool mode_ok(const q4_moe_layer_t* L, int mode) {
  if (L->expert_bits) return mode == Q4_W4A8;
  if (wbits_of(L) == 8) return mode == Q4_W8A8;
  return mode == Q4_W4A16 || mode == Q4_W4A8;
}

// Average routed rows per expert decides the GEMM shape: 16-row decode tiles, 32 / 64-row
// mid tiles, or the 128-row prefill kernel.
double avg_rows(const q4_moe_layer_t* L, int64_t t) { return double(t) * L->top_k / L->num_experts; }

int row_blocks_for(const q4_moe_layer_t* L, int64_t t) {
  const double avg = avg_rows(L, t);
  if (avg <= 16) return 1;
  if (avg <= 32) return 2;
  return 4;
}

// The 128-row prefill kernel from 64 rows per expert on average, and from 17 (9 with
// INT8 activations; bf16 measured slower there: T = 512 1.84 -> 2.03 ms) when the
// launch has enough work items for its tiles to fill the chip several times (estimated
// gate/up items >= 2048): 256-expert layer T = 768 / 1024 / 1536 W4A16 2.29 / 2.79 /
// 4.83 -> 2.18 / 2.36 / 2.87 ms, W4A8 T = 1280 4.38 -> 1.88 ms; small layers (the
// 8-expert one at 48 rows per expert) stay faster on the decode kernel's 64-row tiles.
// The row-count rule alone (wants_prefill) and with the prefill kernels' 32-bit buffer
// offsets (use_prefill: every activation buffer of both launches below 2^31 bytes; past
// that the decode kernel, which addresses with 64-bit offsets, runs instead).
bool wants_prefill(const q4_moe_layer_t* L, int64_t t, int mode) {
  const int act = int8_acts(mode) ? 2 : 0;
  const int64_t S = L->top_k + (L->shared_inter > 0 ? 1 : 0);
  const int64_t P = t * S, ee = int64_t(L->num_experts) + (L->shared_inter > 0 ? 1 : 0);
  const int64_t pf_items = (std::min<int64_t>(ee, P) + P / 128) * (2 * int64_t(L->inter) / 128);
  const double avg = avg_rows(L, t);
  const double lo = act == 2 ? 8 : 16;   // INT8 activations: from 9 rows (T = 512: 1.78 -> 1.51 ms)
  // the lower thresholds were measured on layers of one weight format only
  const bool uniform = !L->expert_bits && !L->expert_groups;
  return (avg >= 64 || (uniform && avg > lo && pf_items >= 2048)) && (2 * int64_t(L->inter)) % 128 == 0 &&
         L->hidden % 128 == 0;
}

bool use_prefill(const q4_moe_layer_t* L, int64_t t, int mode) {
  const int act = int8_acts(mode) ? 2 : 0;
  const int64_t S = L->top_k + (L->shared_inter > 0 ? 1 : 0);
  return wants_prefill(L, t, mode) && prefill_fits(t, L->hidden, act, mat_bytes(L, 2 * L->inter, L->hidden)) &&
         prefill_fits(t * S, L->inter, act, mat_bytes(L, L->hidden, L->inter));
}

FwdWorkspace carve(const q4_moe_layer_t* L, int64_t t, int mode, void* base);

// The forward's one-expert decode path (see ffn_forward).
bool one_expert_decode(const q4_moe_layer_t* L, const FwdWorkspace& w) {
  return L->num_experts == 1 && L->top_k == 1 && L->shared_inter == 0 && !L->expert_bits && !L->expert_groups &&
         !w.prefill;
}

// One token on a layer with one weight format (and not the one-expert path): its slots
// have distinct experts, so the permutation is one row per expert; the GEMMs take
// one-row tiles straight from the routed ids instead (see ffn_forward).
bool slot_tile_decode(const q4_moe_layer_t* L, int64_t t, const FwdWorkspace& w) {
  return t == 1 && !w.prefill && !L->expert_bits && !L->expert_groups && !one_expert_decode(L, w);
}

FwdWorkspace carve(const q4_moe_layer_t* L, int64_t t, int mode, void* base) {
  FwdWorkspace w;
  const int shared = L->shared_inter > 0 ? 1 : 0;
  const int64_t ee = int64_t(L->num_experts) + shared;
  const int64_t S = L->top_k + shared;
  const int64_t P = t * S;
  const int64_t H = L->hidden, I = L->inter;
  w.prefill = use_prefill(L, t, mode);
  // (layers with groups of 32 / 64 use at most 32-row decode tiles)
  w.tile_rows = w.prefill ? 128 : 16 * (L->expert_groups ? std::min(2, row_blocks_for(L, t)) : row_blocks_for(L, t));
  w.max_tiles = int32_t(P / w.tile_rows + std::min<int64_t>(ee, P) + 1);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off += a256(bytes);
    return base ? static_cast<uint8_t*>(base) + at : nullptr;
  };
  w.counts = reinterpret_cast<int32_t*>(take((ee + 1) * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((ee + 2) * 4));
  w.perm = reinterpret_cast<int32_t*>(take(P * 4));
  w.inv = reinterpret_cast<int32_t*>(take(P * 4));
  w.tiles = reinterpret_cast<TileDesc*>(take(int64_t(w.max_tiles) * sizeof(TileDesc)));
  w.num_tiles = reinterpret_cast<int32_t*>(take(4));
  w.fmt_tiles = reinterpret_cast<int32_t*>(take((kNumFormats + 1) * 4));
  w.perm_scratch_ints = permute_scratch_ints(P, int(ee));
  w.perm_scratch = reinterpret_cast<int32_t*>(take(w.perm_scratch_ints * 4));
  w.h = take(P * I * (int8_acts(mode) ? 4 : 2));
  // Decode down projections with few work items (narrow layers: the dense FFN, a few
  // touched experts) split K over workgroups, aiming at about 512 items; the combine sums
  // the partial slices in order.  Layers of one weight format only.
  if (!w.prefill && w.tile_rows == 16 && !L->expert_bits && !L->expert_groups) {
    const int64_t est = std::min<int64_t>(ee, P) * (H / 32);   // items of two column blocks, one tile per expert
    const int64_t G = I / 128;
    if (est > 0 && est < 512) {
      const int64_t ks = std::min<int64_t>({(512 + est - 1) / est, 8, std::max<int64_t>(1, G / 2)});
      // as many slices as the ceil(G / ks)-group slices need: none is left empty
      const int64_t per = (G + ks - 1) / ks;
      w.ksplit = int((G + per - 1) / per);
    }
  }
  w.y = reinterpret_cast<float*>(take(w.ksplit * P * H * 4));
  if (int8_acts(mode)) {
    w.qx = reinterpret_cast<int8_t*>(take(t * H));
    w.sx = reinterpret_cast<float*>(take(t * 4));
    w.qh = reinterpret_cast<int8_t*>(take(P * I));
    w.sh = reinterpret_cast<float*>(take(P * 4));
  }
  if (w.prefill && (mode == Q4_W4A16 || L->asymmetric)) {
    const int64_t sg = L->expert_groups ? 4 : 1;   // sums per 128-element group (finest: groups of 32)
    w.rs_x = take(t * (H / 128) * sg * 4);
    w.rs_h = take(P * (I / 128) * sg * 4);
  }
  w.bytes = off;
  return w;
}

int validate_layer(const q4_moe_layer_t* L) {
  Q4_REQUIRE(L, Q4_ERR_NULL, "layer descriptor is NULL");
  Q4_REQUIRE(L->num_experts >= 1 && L->num_experts <= 4096, Q4_ERR_SHAPE, "num_experts %d not in [1, 4096]",
             L->num_experts);
  Q4_REQUIRE(L->top_k >= 1 && L->top_k <= L->num_experts, Q4_ERR_SHAPE, "top_k %d not in [1, num_experts]",
             L->top_k);
  Q4_REQUIRE(L->hidden > 0 && L->hidden % 128 == 0, Q4_ERR_SHAPE, "hidden %d must be a positive multiple of 128",
             L->hidden);
  Q4_REQUIRE(L->inter > 0 && L->inter % 128 == 0, Q4_ERR_SHAPE, "inter %d must be a positive multiple of 128",
             L->inter);
  Q4_REQUIRE(L->asymmetric == 0 || L->asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  Q4_REQUIRE(L->gate_up && L->down, Q4_ERR_NULL, "expert weight pointers are NULL");
  Q4_REQUIRE(!misaligned(L->gate_up) && !misaligned(L->down), Q4_ERR_ALIGN, "expert weights not 16-byte aligned");
  Q4_REQUIRE(L->weight_bits == 0 || L->weight_bits == 4 || L->weight_bits == 8, Q4_ERR_SHAPE,
             "weight_bits %d not in {0, 4, 8}", L->weight_bits);
  Q4_REQUIRE(L->weight_bits != 8 || L->asymmetric == 0, Q4_ERR_UNSUPPORTED, "8-bit weights are symmetric only");
  if (L->expert_bits) {
    Q4_REQUIRE(L->weight_bits == 0 && L->asymmetric == 0, Q4_ERR_UNSUPPORTED,
               "mixed layers: weight_bits 0 and symmetric weights");
    Q4_REQUIRE(L->gate_up_offsets && L->down_offsets, Q4_ERR_NULL, "mixed layers need the block offsets");
  }
  if (L->expert_groups) {
    Q4_REQUIRE(L->weight_bits == 0 && L->asymmetric == 0, Q4_ERR_UNSUPPORTED,
               "per-expert group sizes: weight_bits 0 and symmetric weights");
    Q4_REQUIRE(L->gate_up_offsets && L->down_offsets, Q4_ERR_NULL, "per-expert group sizes need the block offsets");
  }
  if (L->shared_inter != 0) {
    Q4_REQUIRE(L->shared_inter == L->inter, Q4_ERR_UNSUPPORTED,
               "shared_inter %d must equal inter %d in this build", L->shared_inter, L->inter);
    Q4_REQUIRE(L->shared_gate_up && L->shared_down, Q4_ERR_NULL, "shared expert weight pointers are NULL");
    Q4_REQUIRE(!misaligned(L->shared_gate_up) && !misaligned(L->shared_down), Q4_ERR_ALIGN,
               "shared expert weights not 16-byte aligned");
  }
  return ok();
}

}  // namespace

extern "C" {

const char* q4_status_string(int s) {
  switch (s) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "null pointer";
    case Q4_ERR_SHAPE: return "invalid shape";
    case Q4_ERR_ALIGN: return "misaligned pointer";
    case Q4_ERR_DTYPE: return "unsupported dtype or mode";
    case Q4_ERR_WORKSPACE: return "workspace or buffer too small";
    case Q4_ERR_UNSUPPORTED: return "unsupported case";
    case Q4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* q4_last_error(void) { return g_last_error.c_str(); }

const char* q4_version(void) { return "q4moe 0.1 gfx950"; }

int q4_set_stage_events(void* const* begin, void* const* end, int count) {
  g_last_error.clear();
  if (count == 0 || !begin || !end) {
    g_stage_events = false;
    return ok();
  }
  Q4_REQUIRE(count >= Q4_NUM_STAGES, Q4_ERR_SHAPE, "need %d events per array", Q4_NUM_STAGES);
  for (int i = 0; i < Q4_NUM_STAGES; ++i) {
    Q4_REQUIRE(begin[i] && end[i], Q4_ERR_NULL, "event %d is NULL", i);
    g_stage_begin[i] = static_cast<hipEvent_t>(begin[i]);
    g_stage_end[i] = static_cast<hipEvent_t>(end[i]);
  }
  g_stage_events = true;
  return ok();
}

int quantize_int4_g128(const void* w, int w_dtype, int64_t n, int64_t k, int asymmetric, uint8_t* packed,
                       uint16_t* scales, uint8_t* zeros, int32_t* flags_dev, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(w_dtype == Q4_F32 || w_dtype == Q4_F16 || w_dtype == Q4_BF16, Q4_ERR_DTYPE, "w_dtype %d", w_dtype);
  Q4_REQUIRE(asymmetric == 0 || asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  Q4_REQUIRE(n >= 1 && k >= 128 && k % 128 == 0, Q4_ERR_SHAPE, "need n >= 1 and k a positive multiple of 128");
  Q4_REQUIRE(n * (k / 256 + 1) < (int64_t(1) << 31), Q4_ERR_SHAPE, "matrix too large");
  Q4_REQUIRE(w && packed && scales, Q4_ERR_NULL, "w, packed and scales are required");
  Q4_REQUIRE(asymmetric ? zeros != nullptr : zeros == nullptr, Q4_ERR_NULL,
             "zeros must be given iff asymmetric");
  Q4_REQUIRE(!misaligned(w) && !misaligned(packed) && !misaligned(scales) && !(zeros && misaligned(zeros)),
             Q4_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return check_hip(launch_quantize(w, w_dtype, n, k, asymmetric, packed, scales, zeros, flags_dev, stream),
                   "quantize launch");
}

size_t q4_device_bytes(int64_t n, int64_t k, int asymmetric) {
  if (n < 16 || n % 16 || k < 128 || k % 128) return 0;
  const int64_t g = k / 128;
  int64_t b = a256(n * k / 2) + a256(2 * n * g);
  if (asymmetric) b += a256(n * g);
  return size_t(b);
}

static bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }

int quantize_int4_grouped(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group, int asymmetric,
                          uint8_t* packed, uint16_t* scales, uint8_t* zeros, int32_t* flags_dev, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(valid_group(group), Q4_ERR_SHAPE, "group %d not in {32, 64, 128, 256}", group);
  Q4_REQUIRE(!asymmetric || group >= 128, Q4_ERR_UNSUPPORTED, "zero points need groups of 128 or 256");
  Q4_REQUIRE(k % 128 == 0 && k % group == 0, Q4_ERR_SHAPE, "k must be a multiple of 128 and of the group");
  if (group == 128) return quantize_int4_g128(w, w_dtype, n, k, asymmetric, packed, scales, zeros, flags_dev, stream);
  Q4_REQUIRE(w_dtype == Q4_F32 || w_dtype == Q4_F16 || w_dtype == Q4_BF16, Q4_ERR_DTYPE, "w_dtype %d", w_dtype);
  Q4_REQUIRE(asymmetric == 0 || asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  Q4_REQUIRE(n >= 1 && k >= 128, Q4_ERR_SHAPE, "need n >= 1 and k >= 128");
  Q4_REQUIRE(n * (k / 512 + 1) < (int64_t(1) << 31), Q4_ERR_SHAPE, "matrix too large");
  Q4_REQUIRE(w && packed && scales, Q4_ERR_NULL, "w, packed and scales are required");
  Q4_REQUIRE(asymmetric ? zeros != nullptr : zeros == nullptr, Q4_ERR_NULL,
             "zeros must be given iff asymmetric");
  Q4_REQUIRE(!misaligned(w) && !misaligned(packed) && !misaligned(scales) && !(zeros && misaligned(zeros)),
             Q4_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return check_hip(launch_quantize_grouped(w, w_dtype, n, k, group, asymmetric, packed, scales, zeros, flags_dev,
                                           stream),
                   "grouped quantize launch");
}

size_t q4_device_bytes_grouped(int64_t n, int64_t k, int asymmetric, int32_t group) {
  if (!valid_group(group) || (asymmetric && group < 128) || k % group) return 0;
  if (n < 16 || n % 16 || k < 128 || k % 128) return 0;
  const int64_t g = k / 128, sg = group < 128 ? 128 / group : 1;
  int64_t b = a256(n * k / 2) + a256(2 * n * g * sg);
  if (asymmetric) b += a256(n * g);
  return size_t(b);
}

int q4_repack_device_grouped(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros, int64_t n,
                             int64_t k, int asymmetric, int32_t group, int flags, void* dev_out, size_t dev_bytes,
                             hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(valid_group(group), Q4_ERR_SHAPE, "group %d not in {32, 64, 128, 256}", group);
  Q4_REQUIRE(!asymmetric || group >= 128, Q4_ERR_UNSUPPORTED, "zero points need groups of 128 or 256");
  Q4_REQUIRE(k % group == 0, Q4_ERR_SHAPE, "k must be a multiple of the group");
  Q4_REQUIRE(flags == Q4_REPACK_PLAIN || flags == Q4_REPACK_GATE_UP, Q4_ERR_DTYPE, "flags %d", flags);
  Q4_REQUIRE(asymmetric == 0 || asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  Q4_REQUIRE(k >= 128 && k % 128 == 0 && n >= 16 && n % (flags == Q4_REPACK_GATE_UP ? 32 : 16) == 0,
             Q4_ERR_SHAPE, "need k %% 128 == 0 and n %% %d == 0", flags == Q4_REPACK_GATE_UP ? 32 : 16);
  Q4_REQUIRE(packed && scales && dev_out, Q4_ERR_NULL, "packed, scales and dev_out are required");
  Q4_REQUIRE(!asymmetric || zeros, Q4_ERR_NULL, "zeros required for the asymmetric format");
  Q4_REQUIRE(!misaligned(packed) && !misaligned(dev_out), Q4_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = q4_device_bytes_grouped(n, k, asymmetric, group);
  Q4_REQUIRE(dev_bytes >= need, Q4_ERR_WORKSPACE, "dev_out holds %zu bytes, need %zu", dev_bytes, need);
  return check_hip(launch_repack(packed, scales, zeros, n, k, asymmetric, flags == Q4_REPACK_GATE_UP, dev_out, stream,
                                 group),
                   "repack launch");
}

int q4_repack_device(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros, int64_t n, int64_t k,
                     int asymmetric, int flags, void* dev_out, size_t dev_bytes, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(flags == Q4_REPACK_PLAIN || flags == Q4_REPACK_GATE_UP, Q4_ERR_DTYPE, "flags %d", flags);
  Q4_REQUIRE(asymmetric == 0 || asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  Q4_REQUIRE(k >= 128 && k % 128 == 0 && n >= 16 && n % (flags == Q4_REPACK_GATE_UP ? 32 : 16) == 0,
             Q4_ERR_SHAPE, "need k %% 128 == 0 and n %% %d == 0", flags == Q4_REPACK_GATE_UP ? 32 : 16);
  Q4_REQUIRE(packed && scales && dev_out, Q4_ERR_NULL, "packed, scales and dev_out are required");
  Q4_REQUIRE(!asymmetric || zeros, Q4_ERR_NULL, "zeros required for the asymmetric format");
  Q4_REQUIRE(!misaligned(packed) && !misaligned(dev_out), Q4_ERR_ALIGN, "device pointers must be 16-byte aligned");
  Q4_REQUIRE(dev_bytes >= q4_device_bytes(n, k, asymmetric), Q4_ERR_WORKSPACE, "dev_out holds %zu bytes, need %zu",
             dev_bytes, q4_device_bytes(n, k, asymmetric));
  return check_hip(launch_repack(packed, scales, zeros, n, k, asymmetric, flags == Q4_REPACK_GATE_UP, dev_out, stream),
                   "repack launch");
}

int quantize_int8_g128(const void* w, int w_dtype, int64_t n, int64_t k, int8_t* q, uint16_t* scales,
                       int32_t* flags_dev, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(w_dtype == Q4_F32 || w_dtype == Q4_F16 || w_dtype == Q4_BF16, Q4_ERR_DTYPE, "w_dtype %d", w_dtype);
  Q4_REQUIRE(n >= 1 && k >= 128 && k % 128 == 0, Q4_ERR_SHAPE, "need n >= 1 and k a positive multiple of 128");
  Q4_REQUIRE(n * (k / 128) < (int64_t(1) << 31), Q4_ERR_SHAPE, "matrix too large");
  Q4_REQUIRE(w && q && scales, Q4_ERR_NULL, "w, q and scales are required");
  Q4_REQUIRE(!misaligned(w) && !misaligned(q) && !misaligned(scales), Q4_ERR_ALIGN,
             "device pointers must be 16-byte aligned");
  return check_hip(launch_quantize8(w, w_dtype, n, k, q, scales, flags_dev, stream), "quantize8 launch");
}

size_t q8_device_bytes(int64_t n, int64_t k) {
  if (n < 16 || n % 16 || k < 128 || k % 128) return 0;
  return size_t(a256(n * k) + a256(2 * n * (k / 128)));
}

int q8_repack_device(const int8_t* q, const uint16_t* scales, int64_t n, int64_t k, int flags, void* dev_out,
                     size_t dev_bytes, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(flags == Q4_REPACK_PLAIN || flags == Q4_REPACK_GATE_UP, Q4_ERR_DTYPE, "flags %d", flags);
  Q4_REQUIRE(k >= 128 && k % 128 == 0 && n >= 16 && n % (flags == Q4_REPACK_GATE_UP ? 32 : 16) == 0,
             Q4_ERR_SHAPE, "need k %% 128 == 0 and n %% %d == 0", flags == Q4_REPACK_GATE_UP ? 32 : 16);
  Q4_REQUIRE(q && scales && dev_out, Q4_ERR_NULL, "q, scales and dev_out are required");
  Q4_REQUIRE(!misaligned(q) && !misaligned(dev_out), Q4_ERR_ALIGN, "device pointers must be 16-byte aligned");
  Q4_REQUIRE(dev_bytes >= q8_device_bytes(n, k), Q4_ERR_WORKSPACE, "dev_out holds %zu bytes, need %zu", dev_bytes,
             q8_device_bytes(n, k));
  return check_hip(launch_repack8(q, scales, n, k, flags == Q4_REPACK_GATE_UP, dev_out, stream), "repack8 launch");
}

int quantize_int2_g128(const void* w, int w_dtype, int64_t n, int64_t k, uint8_t* packed, uint16_t* scales,
                       int32_t* flags_dev, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(w_dtype == Q4_F32 || w_dtype == Q4_F16 || w_dtype == Q4_BF16, Q4_ERR_DTYPE, "w_dtype %d", w_dtype);
  Q4_REQUIRE(n >= 1 && k >= 128 && k % 128 == 0, Q4_ERR_SHAPE, "need n >= 1 and k a positive multiple of 128");
  Q4_REQUIRE(n * (k / 128) < (int64_t(1) << 31), Q4_ERR_SHAPE, "matrix too large");
  Q4_REQUIRE(w && packed && scales, Q4_ERR_NULL, "w, packed and scales are required");
  Q4_REQUIRE(!misaligned(w) && !misaligned(packed) && !misaligned(scales), Q4_ERR_ALIGN,
             "device pointers must be 16-byte aligned");
  return check_hip(launch_quantize2(w, w_dtype, n, k, packed, scales, flags_dev, stream), "quantize2 launch");
}

size_t q2_device_bytes(int64_t n, int64_t k) {
  if (n < 16 || n % 16 || k < 128 || k % 128) return 0;
  return size_t(a256(n * k / 4) + a256(2 * n * (k / 128)));
}

int q2_repack_device(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int flags, void* dev_out,
                     size_t dev_bytes, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(flags == Q4_REPACK_PLAIN || flags == Q4_REPACK_GATE_UP, Q4_ERR_DTYPE, "flags %d", flags);
  Q4_REQUIRE(k >= 128 && k % 128 == 0 && n >= 16 && n % (flags == Q4_REPACK_GATE_UP ? 32 : 16) == 0,
             Q4_ERR_SHAPE, "need k %% 128 == 0 and n %% %d == 0", flags == Q4_REPACK_GATE_UP ? 32 : 16);
  Q4_REQUIRE(packed && scales && dev_out, Q4_ERR_NULL, "packed, scales and dev_out are required");
  Q4_REQUIRE(!misaligned(packed) && !misaligned(dev_out), Q4_ERR_ALIGN, "device pointers must be 16-byte aligned");
  Q4_REQUIRE(dev_bytes >= q2_device_bytes(n, k), Q4_ERR_WORKSPACE, "dev_out holds %zu bytes, need %zu", dev_bytes,
             q2_device_bytes(n, k));
  return check_hip(launch_repack2(packed, scales, n, k, flags == Q4_REPACK_GATE_UP, dev_out, stream), "repack2 launch");
}

size_t moe_route_workspace_bytes(int64_t t, int64_t h, int32_t e) {
  if (t <= 0 || h <= 0 || e <= 0) return 0;
  return route_workspace_bytes(t, h, e);
}

int moe_route_topk(const uint16_t* x_bf16, const float* w_router, const float* bias, int64_t t, int64_t h, int32_t e,
                   int32_t k, float* logits_out, int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                   hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(t >= 0, Q4_ERR_SHAPE, "t < 0");
  Q4_REQUIRE(e >= 1 && e <= 1024 && k >= 1 && k <= e, Q4_ERR_SHAPE, "need 1 <= k <= e <= 1024 (k=%d, e=%d)", k, e);
  Q4_REQUIRE(h >= 16 && h % 16 == 0, Q4_ERR_SHAPE, "h must be a positive multiple of 16");
  if (t == 0) return ok();
  Q4_REQUIRE(x_bf16 && w_router && logits_out && topk_ids && topk_w, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(x_bf16) && !misaligned(w_router), Q4_ERR_ALIGN, "x and w_router must be 16-byte aligned");
  const size_t need = moe_route_workspace_bytes(t, h, e);
  Q4_REQUIRE(ws_bytes >= need && (need == 0 || workspace), Q4_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  Q4_REQUIRE(!misaligned(workspace), Q4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return check_hip(launch_route(x_bf16, w_router, bias, t, h, e, k, logits_out, topk_ids, topk_w,
                                static_cast<float*>(workspace), stream),
                   "route launch");
}

int moe_permute(const int32_t* ids, int64_t t, int32_t k, int32_t e, int32_t* counts, int32_t* offsets, int32_t* perm,
                int32_t* inv, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(t >= 0 && k >= 1 && k <= e && e <= 4096, Q4_ERR_SHAPE, "need 1 <= k <= e <= 4096, t >= 0");
  Q4_REQUIRE(t * k < (int64_t(1) << 31), Q4_ERR_SHAPE, "t * k too large");
  Q4_REQUIRE(counts && offsets, Q4_ERR_NULL, "counts and offsets are required");
  Q4_REQUIRE(t == 0 || (ids && perm && inv), Q4_ERR_NULL, "ids, perm and inv are required");
  return check_hip(launch_permute(ids, t, k, e, 0, counts, offsets, perm, inv, nullptr, nullptr, 16, stream),
                   "permute launch");
}

int act_quant_int8(const void* x, int x_dtype, int64_t rows, int64_t cols, int8_t* q, float* s, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(x_dtype == Q4_BF16 || x_dtype == Q4_F32, Q4_ERR_DTYPE, "x_dtype must be Q4_BF16 or Q4_F32");
  Q4_REQUIRE(rows >= 0 && cols >= 128 && cols % 128 == 0, Q4_ERR_SHAPE, "cols must be a positive multiple of 128");
  if (rows == 0) return ok();
  Q4_REQUIRE(x && q && s, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(x) && !misaligned(q), Q4_ERR_ALIGN, "x and q must be 16-byte aligned");
  return check_hip(launch_act_quant(x, x_dtype == Q4_F32, rows, cols, q, s, nullptr, stream), "act quant launch");
}

size_t moe_int4_ffn_workspace_bytes(const q4_moe_layer_t* layer, int64_t t, int mode) {
  if (!layer || t < 0 || validate_layer(layer) != Q4_OK) return 0;
  if (!mode_ok(layer, mode)) return 0;
  return size_t(carve(layer, t, mode, nullptr).bytes);
}

int moe_int4_ffn_plan(const q4_moe_layer_t* L, int64_t t, int mode, q4_ffn_plan_t* plan) {
  g_last_error.clear();
  Q4_REQUIRE(plan, Q4_ERR_NULL, "plan is NULL");
  *plan = q4_ffn_plan_t{};
  if (int rc = validate_layer(L)) return rc;
  Q4_REQUIRE(mode_ok(L, mode), Q4_ERR_DTYPE, "mode %d does not match the layer's weight format", mode);
  Q4_REQUIRE(t >= 0, Q4_ERR_SHAPE, "t < 0");
  const FwdWorkspace w = carve(L, t, mode, nullptr);
  plan->kernel = w.prefill ? Q4_PLAN_PREFILL : Q4_PLAN_DECODE;
  plan->tile_rows = w.tile_rows;
  plan->down_ksplit = w.ksplit;
  plan->prefill_addr_limited = (!w.prefill && wants_prefill(L, t, mode)) ? 1 : 0;
  plan->rows_in_token_order = one_expert_decode(L, w) ? 1 : 0;
  plan->combine_in_down = (plan->rows_in_token_order && w.ksplit == 1) ? 1 : 0;
  plan->slot_tiles = slot_tile_decode(L, t, w) ? 1 : 0;
  plan->workspace_bytes = w.bytes;
  return ok();
}

extern "C++" {  // internal helpers keep C++ linkage
namespace {

// Experts ordered by hit count, descending; equal counts keep the lower index first.
std::vector<int32_t> by_hotness(const int64_t* counts, int32_t e) {
  std::vector<int32_t> order(e);
  for (int32_t i = 0; i < e; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
  return order;
}

int check_counts(const int64_t* counts, int32_t e, const void* out) {
  Q4_REQUIRE(counts && out, Q4_ERR_NULL, "counts and the output array are required");
  Q4_REQUIRE(e >= 1 && e <= 4096, Q4_ERR_SHAPE, "e %d not in [1, 4096]", e);
  for (int32_t i = 0; i < e; ++i) Q4_REQUIRE(counts[i] >= 0, Q4_ERR_SHAPE, "counts[%d] < 0", i);
  return ok();
}

int64_t top_count(double frac, int32_t e) {
  return std::min<int64_t>(e, int64_t(std::ceil(frac * double(e) - 1e-9)));
}

}  // namespace
}  // extern "C++"

int moe_expert_bits_by_hotness(const int64_t* counts, int32_t e, double frac8, int shared, int32_t* bits_out) {
  g_last_error.clear();
  if (int rc = check_counts(counts, e, bits_out)) return rc;
  Q4_REQUIRE(frac8 >= 0.0 && frac8 <= 1.0, Q4_ERR_SHAPE, "frac8 must lie in [0, 1]");
  const std::vector<int32_t> order = by_hotness(counts, e);
  const int64_t n8 = top_count(frac8, e);
  for (int32_t i = 0; i < e; ++i) bits_out[i] = 4;
  for (int64_t i = 0; i < n8; ++i) bits_out[order[i]] = 8;
  if (shared) bits_out[e] = 8;   // the shared expert sees every token
  return ok();
}

int moe_expert_bits_apex(const int64_t* counts, int32_t e, double frac8, double cold_share, int shared,
                         int32_t* bits_out) {
  g_last_error.clear();
  if (int rc = check_counts(counts, e, bits_out)) return rc;
  Q4_REQUIRE(frac8 >= 0.0 && frac8 <= 1.0 && cold_share >= 0.0, Q4_ERR_SHAPE,
             "frac8 must lie in [0, 1] and cold_share be >= 0");
  int64_t total = 0;
  for (int32_t i = 0; i < e; ++i) total += counts[i];
  for (int32_t i = 0; i < e; ++i) bits_out[i] = double(counts[i] * e) < cold_share * double(total) ? 2 : 4;
  const std::vector<int32_t> order = by_hotness(counts, e);
  const int64_t n8 = top_count(frac8, e);
  for (int64_t i = 0; i < n8; ++i) bits_out[order[i]] = 8;
  if (shared) bits_out[e] = frac8 > 0.0 ? 8 : 4;
  return ok();
}

int moe_expert_groups_by_hotness(const int64_t* counts, int32_t e, double hot_frac, double cold_share, int shared,
                                 int32_t* groups_out) {
  g_last_error.clear();
  if (int rc = check_counts(counts, e, groups_out)) return rc;
  Q4_REQUIRE(hot_frac >= 0.0 && hot_frac <= 1.0 && cold_share >= 0.0, Q4_ERR_SHAPE,
             "hot_frac must lie in [0, 1] and cold_share be >= 0");
  int64_t total = 0;
  for (int32_t i = 0; i < e; ++i) total += counts[i];
  for (int32_t i = 0; i < e; ++i) groups_out[i] = double(counts[i] * e) < cold_share * double(total) ? 256 : 64;
  const std::vector<int32_t> order = by_hotness(counts, e);
  const int64_t nh = top_count(hot_frac, e);
  for (int64_t i = 0; i < nh; ++i) groups_out[order[i]] = 32;
  if (shared) groups_out[e] = 32;
  return ok();
}

extern "C++" {  // internal helpers keep C++ linkage
namespace {

int ffn_forward(const q4_moe_layer_t* L, const uint16_t* x_bf16, int64_t t, const int32_t* topk_ids,
                const float* topk_w, int mode, uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                hipStream_t stream, q4_ffn_views_t* views) {
  g_last_error.clear();
  if (views) *views = q4_ffn_views_t{};
  if (int rc = validate_layer(L)) return rc;
  Q4_REQUIRE(mode_ok(L, mode), Q4_ERR_DTYPE, "mode %d does not match the layer's weight format", mode);
  Q4_REQUIRE(t >= 0, Q4_ERR_SHAPE, "t < 0");
  if (t == 0) return ok();
  const int shared = L->shared_inter > 0 ? 1 : 0;
  const int64_t S = L->top_k + shared;
  Q4_REQUIRE(t * S * std::max(L->hidden, L->inter) < (int64_t(1) << 40) && t * S < (int64_t(1) << 31), Q4_ERR_SHAPE,
             "t too large");
  Q4_REQUIRE(x_bf16 && topk_ids && topk_w && out_bf16 && workspace, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(x_bf16) && !misaligned(out_bf16) && !misaligned(workspace), Q4_ERR_ALIGN,
             "x, out and workspace must be 16-byte aligned");
  FwdWorkspace w = carve(L, t, mode, workspace);
  Q4_REQUIRE(ws_bytes >= size_t(w.bytes), Q4_ERR_WORKSPACE, "workspace %zu < %lld", ws_bytes, (long long)w.bytes);
  if (views) {
    views->counts = w.counts;
    views->offsets = w.offsets;
    views->perm = w.perm;
    views->inv = w.inv;
    views->h = w.h;
    views->h_is_f32 = int8_acts(mode) ? 1 : 0;
    views->slots_per_token = int32_t(S);
    views->positions = t * S;
    views->y = w.y;
    views->y_slices = w.ksplit;
    views->y_slice_groups = int32_t((L->inter / 128 + w.ksplit - 1) / w.ksplit);
    views->y_slice_stride = t * S * L->hidden;
    views->q_x = w.qx;
    views->s_x = w.sx;
    views->q_h = w.qh;
    views->s_h = w.sh;
  }
  const int64_t H = L->hidden, I = L->inter;
  const int rb = w.tile_rows / 16;
  // A one-expert, one-choice layer without a shared expert (a dense SwiGLU FFN) at decode
  // sizes: the permutation is the identity, so the GEMMs read and write rows in token
  // order; without K slices the down projection also applies the weight and rounds to
  // bf16 in its epilogue (the combine's own arithmetic), so only the two GEMMs run.  The
  // debug call still runs the permutation and the separate combine, for its views.
  const bool dense = one_expert_decode(L, w);
  const bool fused_combine = dense && w.ksplit == 1 && !views;
  // A single token on a layer with one weight format: slot i of the token is its own
  // one-row tile (its experts are distinct, so the permutation would give the same
  // tiles), rows stay in slot order and the combine reads them there; no permutation
  // launch.  Each output row depends only on its own row and expert, so the results
  // equal the permuted path's bit for bit (the debug call takes that path, for its views).
  const bool slots = slot_tile_decode(L, t, w) && !views;
  int rc;
  stage_begin(Q4_STAGE_PERMUTE, stream);
  if ((!dense && !slots) || views) {
    if ((rc = check_hip(launch_permute(topk_ids, t, L->top_k, L->num_experts, shared, w.counts, w.offsets, w.perm,
                                       w.inv, w.tiles, w.num_tiles, w.tile_rows, stream, L->expert_bits,
                                       L->expert_groups, w.fmt_tiles, w.perm_scratch, w.perm_scratch_ints),
                        "permute")))
      return rc;
  }
  stage_end(Q4_STAGE_PERMUTE, stream);
  GemmArgs gu{};
  gu.perm = w.perm;
  gu.slots_per_token = int32_t(S);
  gu.w = static_cast<const uint8_t*>(L->gate_up);
  gu.w_stride = mat_bytes(L, 2 * I, H);
  gu.wbits = wbits_of(L);
  gu.sg = 1;
  gu.ebits = L->expert_bits;
  gu.egroups = L->expert_groups;
  gu.woffs = L->gate_up_offsets;
  gu.w_shared = static_cast<const uint8_t*>(L->shared_gate_up);
  gu.num_experts = L->num_experts;
  gu.asym = L->asymmetric;
  gu.N = 2 * I;
  gu.K = H;
  gu.tiles = dense ? nullptr : w.tiles;
  gu.num_tiles = w.num_tiles;
  gu.max_tiles = w.max_tiles;
  gu.dense_rows = t;
  gu.out = w.h;
  gu.a_rows = t;
  if (dense) gu.perm = nullptr;
  GemmArgs dn = gu;
  dn.a_rows = t * S;
  dn.perm = nullptr;
  dn.w = static_cast<const uint8_t*>(L->down);
  dn.w_stride = mat_bytes(L, H, I);
  dn.woffs = L->down_offsets;
  dn.w_shared = static_cast<const uint8_t*>(L->shared_down);
  dn.N = H;
  dn.K = I;
  dn.out = w.y;
  dn.ksplit = w.ksplit;
  dn.out_slice = t * S * H;
  dn.dense_rows = t * S;
  if (fused_combine) {
    dn.combine_w = topk_w;
    dn.out_bf16 = out_bf16;
  }
  if (slots) {
    gu.tiles = dn.tiles = nullptr;
    gu.slot_ids = dn.slot_ids = topk_ids;
    gu.slot_k = dn.slot_k = L->top_k;
    gu.perm = nullptr;
    gu.src_div = int32_t(S);   // x row = token = slot / S
    gu.dense_rows = dn.dense_rows = t * S;
  }
  auto gemm1 = [&](const GemmArgs& g, int act, int kind) {
    return w.prefill ? launch_gemm_prefill(g, act, kind, stream) : launch_gemm(g, act, kind, rb, stream);
  };
  // Layers whose experts differ in width or group size: the permutation orders the row
  // tiles by weight format (0: 4-bit, one scale entry per tile; 1: two; 2: four; 3: 8-bit;
  // 4: 2-bit) and one launch per format walks that format's tile range.  The 2-bit
  // experts (rarely routed ones) always run on the streaming kernel; in a prefill-sized
  // launch it walks the 128-row tiles in 64-row sub-tiles.  The bf16 prefill kernel
  // reads activation sums per scale group; they are recomputed at each launch's
  // granularity (rs_a: the activations, rs_rows their rows) before it.
  // The decode GEMM takes all 4-bit formats in one launch (each item picks its expert's
  // scale entries per tile).
  auto gemm = [&](const GemmArgs& g, int act, int kind, const void* rs_a = nullptr, int64_t rs_rows = 0) {
    if (!g.ebits && !g.egroups) return gemm1(g, act, kind);
    for (int f = 0; f < kNumFormats; ++f) {
      {
        if (f >= 3 && !g.ebits) continue;
        if ((f == 1 || f == 2) && !g.egroups) continue;
        const bool merged = !w.prefill && g.egroups && f < 3;   // formats 0..2 in one decode launch
        if (merged && f > 0) continue;
        const int sg = merged ? -1 : f == 2 ? 4 : f == 1 ? 2 : 1;
        GemmArgs a = g;
        a.wbits = f == 3 ? 8 : f == 4 ? 2 : 4;
        a.sg = sg;
        a.fmt_tiles = w.fmt_tiles;
        a.fmt = f;
        a.fmt_end = merged ? 3 : f + 1;
        if (f == 4) {
          if (w.prefill) a.built_rows = w.tile_rows;
          const hipError_t e = launch_gemm(a, act, kind, w.prefill ? 4 : rb, stream);
          if (e != hipSuccess) return e;
          continue;
        }
        if (rs_a && a.a_gsum) {
          const hipError_t e = launch_rowsum(rs_a, 0, rs_rows, a.K, const_cast<float*>(a.a_gsum), stream, sg);
          if (e != hipSuccess) return e;
        }
        const hipError_t e = gemm1(a, act, kind);
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  };
  if (mode == Q4_W4A16) {
    gu.a = x_bf16;
    dn.a = w.h;
    if (w.prefill) {
      stage_begin(Q4_STAGE_X_QUANT, stream);
      if ((rc = check_hip(launch_rowsum(x_bf16, 0, t, H, w.rs_x, stream), "x row sums"))) return rc;
      stage_end(Q4_STAGE_X_QUANT, stream);
      gu.a_gsum = static_cast<const float*>(w.rs_x);
      dn.a_gsum = static_cast<const float*>(w.rs_h);
    }
    stage_begin(Q4_STAGE_GATE_UP, stream);
    if ((rc = check_hip(gemm(gu, 0, GEMM_GATE_UP, x_bf16, t), "gate/up gemm"))) return rc;
    stage_end(Q4_STAGE_GATE_UP, stream);
    if (w.prefill) {
      stage_begin(Q4_STAGE_H_QUANT, stream);
      if ((rc = check_hip(launch_rowsum(w.h, 0, t * S, I, w.rs_h, stream), "h row sums"))) return rc;
      stage_end(Q4_STAGE_H_QUANT, stream);
    }
    stage_begin(Q4_STAGE_DOWN, stream);
    if ((rc = check_hip(gemm(dn, 0, GEMM_PLAIN, w.h, t * S), "down gemm"))) return rc;
    stage_end(Q4_STAGE_DOWN, stream);
  } else {
    stage_begin(Q4_STAGE_X_QUANT, stream);
    if ((rc = check_hip(launch_act_quant(x_bf16, 0, t, H, w.qx, w.sx, nullptr, stream), "x quant"))) return rc;
    if (w.prefill && L->asymmetric &&
        (rc = check_hip(launch_rowsum(w.qx, 1, t, H, w.rs_x, stream), "x code sums")))
      return rc;
    stage_end(Q4_STAGE_X_QUANT, stream);
    gu.a = w.qx;
    gu.a_scale = w.sx;
    gu.a_qsum = static_cast<const int32_t*>(w.rs_x);
    stage_begin(Q4_STAGE_GATE_UP, stream);
    if ((rc = check_hip(gemm(gu, 2, GEMM_GATE_UP), "gate/up gemm"))) return rc;
    stage_end(Q4_STAGE_GATE_UP, stream);
    stage_begin(Q4_STAGE_H_QUANT, stream);
    if ((rc = check_hip(launch_act_quant(w.h, 1, t * S, I, w.qh, w.sh, nullptr, stream), "h quant"))) return rc;
    if (w.prefill && L->asymmetric &&
        (rc = check_hip(launch_rowsum(w.qh, 1, t * S, I, w.rs_h, stream), "h code sums")))
      return rc;
    stage_end(Q4_STAGE_H_QUANT, stream);
    dn.a = w.qh;
    dn.a_scale = w.sh;
    dn.a_qsum = static_cast<const int32_t*>(w.rs_h);
    stage_begin(Q4_STAGE_DOWN, stream);
    if ((rc = check_hip(gemm(dn, 2, GEMM_PLAIN), "down gemm"))) return rc;
    stage_end(Q4_STAGE_DOWN, stream);
  }
  stage_begin(Q4_STAGE_COMBINE, stream);
  rc = fused_combine ? Q4_OK
                     : check_hip(launch_combine(w.y, (dense || slots) ? nullptr : w.inv, topk_w, t, L->top_k, shared,
                                                H, out_bf16, stream, dn.ksplit, dn.out_slice),
                                 "combine");
  stage_end(Q4_STAGE_COMBINE, stream);
  return rc;
}

}  // namespace
}  // extern "C++"

int moe_int4_ffn_forward(const q4_moe_layer_t* L, const uint16_t* x_bf16, int64_t t, const int32_t* topk_ids,
                         const float* topk_w, int mode, uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  return ffn_forward(L, x_bf16, t, topk_ids, topk_w, mode, out_bf16, workspace, ws_bytes, stream, nullptr);
}

int moe_int4_ffn_debug(const q4_moe_layer_t* L, const uint16_t* x_bf16, int64_t t, const int32_t* topk_ids,
                       const float* topk_w, int mode, uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                       q4_ffn_views_t* views, hipStream_t stream) {
  if (!views) {
    g_last_error = "views is NULL";
    return Q4_ERR_NULL;
  }
  return ffn_forward(L, x_bf16, t, topk_ids, topk_w, mode, out_bf16, workspace, ws_bytes, stream, views);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free forward
// The forward's workspace in a file-scope device array, one copy per GPU, for callers
// that cannot allocate.  Host code never passes `scratch` itself (on the host it only
// names the symbol): its device address is looked up once per device with
// hipGetSymbolAddress and that address is what the kernels get.  Nothing in the
// forward's workspace needs to start at zero (every buffer is written before it is
// read), so the last call's contents do no harm; overlapping calls on one GPU race.
static __device__ __align__(256) uint8_t scratch[Q4_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[Q4_MAX_DEVICES] = {};

// Device address of this device's scratch array (looked up on the first call with the
// device current), or NULL with the error text set.
void* scratch_for_current_device(int* rc) {
  int dev = -1;
  if ((*rc = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return nullptr;
  if (dev < 0 || dev >= Q4_MAX_DEVICES) {
    *rc = fail(Q4_ERR_UNSUPPORTED, "device %d beyond the %d this build tracks", dev, Q4_MAX_DEVICES);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((*rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_int4_ffn_forward_noalloc(const q4_moe_layer_t* L, const uint16_t* x_bf16, int64_t t, const int32_t* topk_ids,
                                 const float* topk_w, int mode, uint16_t* out_bf16, hipStream_t stream) {
  g_last_error.clear();
  if (int rc = validate_layer(L)) return rc;
  Q4_REQUIRE(mode_ok(L, mode), Q4_ERR_DTYPE, "mode %d does not match the layer's weight format", mode);
  Q4_REQUIRE(t >= 0, Q4_ERR_SHAPE, "t < 0");
  if (t == 0) return ok();
  Q4_REQUIRE(t * (L->top_k + (L->shared_inter > 0 ? 1 : 0)) < (int64_t(1) << 31), Q4_ERR_SHAPE, "t too large");
  const int64_t need = carve(L, t, mode, nullptr).bytes;
  Q4_REQUIRE(need <= int64_t(Q4_NOALLOC_SCRATCH_BYTES), Q4_ERR_WORKSPACE,
             "t = %lld needs %lld workspace bytes; the allocation-free forward holds %lld", (long long)t,
             (long long)need, (long long)Q4_NOALLOC_SCRATCH_BYTES);
  int rc = Q4_OK;
  void* ws = scratch_for_current_device(&rc);
  if (!ws) return rc;
  return ffn_forward(L, x_bf16, t, topk_ids, topk_w, mode, out_bf16, ws, size_t(Q4_NOALLOC_SCRATCH_BYTES), stream,
                     nullptr);
}

// ------------------------------------------------------------------ LoRA-mode experts
extern "C++" {  // internal helpers keep C++ linkage
namespace {

struct LoraWorkspace {
  float* base_gu = nullptr;   // [t][2I]
  float* a = nullptr;         // [t k][K chunks][2r] partial input projections
  float* d = nullptr;         // [t k][column blocks][r] partial down-adapter projections
  uint16_t* hw = nullptr;     // [t][I] bf16
  float* y = nullptr;         // [t][H]
  TileDesc* tiles = nullptr;  // dense row tiles (prefill GEMM)
  int32_t* num_tiles = nullptr;
  float* rs_x = nullptr;      // [t][H/128]
  float* rs_h = nullptr;      // [t][I/128]
  bool prefill = false;
  // grouped by expert (large batches): the permutation of the slots, its 64-slot tiles,
  // h per slot [t k][I] fp32
  bool grouped = false;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* perm = nullptr;
  int32_t* inv = nullptr;
  TileDesc* gtiles = nullptr;
  int32_t* gnum_tiles = nullptr;
  int32_t gmax_tiles = 0;
  float* h_slot = nullptr;
  int ncb = 0;                // column blocks of d (the kernel's own block width)
  int64_t bytes = 0;
};

constexpr int64_t kLoraPrefillRows = 256;
// From this many tokens (ranks 16 and 32) the adapter work runs grouped by expert, each
// expert's adapter rows loaded once per tile of slots instead of once per slot (T = 2048:
// the token-major kernel re-read 768 KB of adapter rows per slot).
constexpr int64_t kLoraGroupedRows = 256;

LoraWorkspace carve_lora(const q4_lora_layer_t* L, int64_t t, void* base) {
  LoraWorkspace w;
  const int64_t H = L->hidden, I = L->inter, r = L->rank, P = t * L->top_k;
  // the 128-row prefill tiles need a few hundred rows to give the dense GEMMs enough
  // work items (at 64-128 rows the down GEMM, N = hidden, had 16-32 of them; 32-row
  // decode tiles measured 35 % faster there, the prefill kernel faster from 256 rows)
  w.prefill = t >= kLoraPrefillRows && prefill_fits(t, H, 0, int64_t(q4_device_bytes(2 * I, H, L->asymmetric))) &&
              prefill_fits(t, I, 0, int64_t(q4_device_bytes(H, I, L->asymmetric)));
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off += a256(bytes);
    return base ? static_cast<uint8_t*>(base) + at : nullptr;
  };
  w.grouped = t >= kLoraGroupedRows && lora_grouped_rank(int(r));
  w.ncb = w.grouped ? lora_grp_col_blocks(I) : lora_col_blocks(I);
  w.base_gu = reinterpret_cast<float*>(take(t * 2 * I * 4));
  w.a = reinterpret_cast<float*>(take(P * lora_kchunks(H) * 2 * r * 4));
  w.d = reinterpret_cast<float*>(take(P * w.ncb * r * 4));
  if (w.grouped) {
    const int64_t E = L->num_experts;
    w.counts = reinterpret_cast<int32_t*>(take((E + 1) * 4));
    w.offsets = reinterpret_cast<int32_t*>(take((E + 2) * 4));
    w.perm = reinterpret_cast<int32_t*>(take(P * 4));
    w.inv = reinterpret_cast<int32_t*>(take(P * 4));
    w.gmax_tiles = int32_t(P / 64 + std::min<int64_t>(E, P) + 1);
    w.gtiles = reinterpret_cast<TileDesc*>(take(int64_t(w.gmax_tiles) * int64_t(sizeof(TileDesc))));
    w.gnum_tiles = reinterpret_cast<int32_t*>(take(4));
    w.h_slot = reinterpret_cast<float*>(take(P * I * 4));
  }
  w.hw = reinterpret_cast<uint16_t*>(take(t * I * 2));
  w.y = reinterpret_cast<float*>(take(t * H * 4));
  if (w.prefill) {
    w.tiles = reinterpret_cast<TileDesc*>(take((t / 128 + 1) * int64_t(sizeof(TileDesc))));
    w.num_tiles = reinterpret_cast<int32_t*>(take(4));
    w.rs_x = reinterpret_cast<float*>(take(t * (H / 128) * 4));
    w.rs_h = reinterpret_cast<float*>(take(t * (I / 128) * 4));
  }
  w.bytes = off;
  return w;
}

int validate_lora(const q4_lora_layer_t* L) {
  Q4_REQUIRE(L, Q4_ERR_NULL, "layer descriptor is NULL");
  Q4_REQUIRE(L->num_experts >= 1 && L->num_experts <= 4096, Q4_ERR_SHAPE, "num_experts %d not in [1, 4096]",
             L->num_experts);
  Q4_REQUIRE(L->top_k >= 1 && L->top_k <= L->num_experts, Q4_ERR_SHAPE, "top_k %d not in [1, num_experts]", L->top_k);
  Q4_REQUIRE(L->hidden > 0 && L->hidden % 128 == 0, Q4_ERR_SHAPE, "hidden %d must be a positive multiple of 128",
             L->hidden);
  Q4_REQUIRE(L->inter > 0 && L->inter % 128 == 0, Q4_ERR_SHAPE, "inter %d must be a positive multiple of 128",
             L->inter);
  Q4_REQUIRE(L->rank >= 8 && L->rank <= 64 && L->rank % 8 == 0, Q4_ERR_SHAPE, "rank %d not in {8, 16, ..., 64}",
             L->rank);
  Q4_REQUIRE(L->asymmetric == 0 || L->asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  Q4_REQUIRE(L->base_gate_up && L->base_down && L->a_gate_up && L->b_gate && L->b_up && L->a_down && L->b_down,
             Q4_ERR_NULL, "missing layer pointer");
  Q4_REQUIRE(!misaligned(L->base_gate_up) && !misaligned(L->base_down) && !misaligned(L->a_gate_up) &&
                 !misaligned(L->b_gate) && !misaligned(L->b_up) && !misaligned(L->a_down) && !misaligned(L->b_down),
             Q4_ERR_ALIGN, "layer pointers must be 16-byte aligned");
  return Q4_OK;
}

// y[rows][n] = a[rows][k] W^T for a PLAIN device-layout INT4 matrix (bf16 activations):
// the decode kernel for few rows, the prefill kernel (dense row tiles) for many.
// (prefill: tiles_ready, the row tiles of the rows are already built; rs_ready, rs
// already holds the row sums of a per group of 128.)
int dense_gemm(const uint16_t* a, int64_t rows, int64_t k, const void* w_dev, int64_t n, int asym, float* y,
               bool prefill, TileDesc* tiles, int32_t* num_tiles, float* rs, hipStream_t stream,
               bool tiles_ready = false, bool rs_ready = false) {
  GemmArgs g{};
  g.a = a;
  g.a_rows = rows;
  g.w = static_cast<const uint8_t*>(w_dev);
  g.w_stride = int64_t(q4_device_bytes(n, k, asym));
  g.num_experts = 1;
  g.asym = asym;
  g.N = n;
  g.K = k;
  g.out = y;
  if (prefill) {
    int rc;
    if (!tiles_ready && (rc = check_hip(launch_dense_tiles(rows, 128, tiles, num_tiles, stream), "dense tiles")))
      return rc;
    if (!rs_ready && (rc = check_hip(launch_rowsum(a, 0, rows, k, rs, stream), "row sums"))) return rc;
    g.tiles = tiles;
    g.num_tiles = num_tiles;
    g.max_tiles = int32_t(rows / 128 + 1);
    g.a_gsum = rs;
    return check_hip(launch_gemm_prefill(g, 0, GEMM_PLAIN, stream), "prefill gemm");
  }
  g.dense_rows = rows;
  // 16- or 32-row tiles: more work items than 64-row ones for the few-hundred-row range
  // below the prefill kernel's
  const int rb = rows <= 16 ? 1 : 2;
  return check_hip(launch_gemm(g, 0, GEMM_PLAIN, rb, stream), "gemm");
}

}  // namespace
}  // extern "C++"

size_t moe_lora_ffn_workspace_bytes(const q4_lora_layer_t* layer, int64_t t) {
  if (!layer || t < 0 || validate_lora(layer) != Q4_OK) return 0;
  return size_t(carve_lora(layer, t, nullptr).bytes);
}

int moe_lora_ffn_forward(const q4_lora_layer_t* L, const uint16_t* x_bf16, int64_t t, const int32_t* topk_ids,
                         const float* topk_w, uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  g_last_error.clear();
  if (int rc = validate_lora(L)) return rc;
  Q4_REQUIRE(t >= 0, Q4_ERR_SHAPE, "t < 0");
  if (t == 0) return ok();
  Q4_REQUIRE(t * L->top_k < (int64_t(1) << 31) && t * 2 * L->inter < (int64_t(1) << 40), Q4_ERR_SHAPE, "t too large");
  Q4_REQUIRE(x_bf16 && topk_ids && topk_w && out_bf16 && workspace, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(x_bf16) && !misaligned(out_bf16) && !misaligned(workspace), Q4_ERR_ALIGN,
             "x, out and workspace must be 16-byte aligned");
  LoraWorkspace w = carve_lora(L, t, workspace);
  Q4_REQUIRE(ws_bytes >= size_t(w.bytes), Q4_ERR_WORKSPACE, "workspace %zu < %lld", ws_bytes, (long long)w.bytes);
  const int64_t H = L->hidden, I = L->inter;
  const int r = L->rank, kk = L->top_k, E = L->num_experts;
  int rc;
  if ((rc = dense_gemm(x_bf16, t, H, L->base_gate_up, 2 * I, L->asymmetric, w.base_gu, w.prefill, w.tiles,
                       w.num_tiles, w.rs_x, stream)))
    return rc;
  if ((rc = check_hip(launch_lora_in(x_bf16, t, H, topk_ids, kk, E, L->a_gate_up, r, w.a, stream), "lora in")))
    return rc;
  if (w.grouped) {
    if ((rc = check_hip(launch_permute(topk_ids, t, kk, E, 0, w.counts, w.offsets, w.perm, w.inv, w.gtiles,
                                       w.gnum_tiles, 64, stream),
                        "lora permute")))
      return rc;
    if ((rc = check_hip(launch_lora_mid_grp(w.base_gu, I, w.perm, w.gtiles, w.gnum_tiles, w.gmax_tiles, kk, H, r,
                                            w.a, L->b_gate, L->b_up, L->a_down, w.d, w.h_slot, stream),
                        "lora mid (grouped)")))
      return rc;
    if ((rc = check_hip(launch_lora_hsum(w.h_slot, topk_w, t, kk, I, w.hw, w.prefill ? w.rs_h : nullptr, stream),
                        "lora hw")))
      return rc;
  } else if ((rc = check_hip(launch_lora_mid(w.base_gu, t, H, I, topk_ids, topk_w, kk, E, r, w.a, L->b_gate, L->b_up,
                                             L->a_down, w.d, w.hw, stream),
                             "lora mid")))
    return rc;
  // the row tiles of the t rows are the gate/up GEMM's; grouped, k_lora_hsum also formed
  // the row sums of hw
  if ((rc = dense_gemm(w.hw, t, I, L->base_down, H, L->asymmetric, w.y, w.prefill, w.tiles, w.num_tiles, w.rs_h,
                       stream, true, w.grouped)))
    return rc;
  return check_hip(launch_lora_out(w.y, t, H, I, topk_ids, topk_w, kk, E, r, w.d, L->b_down, out_bf16, stream, w.ncb),
                   "lora out");
}

int int4_linear_forward(const void* x, int x_dtype, int64_t t, int64_t k, const void* w_dev, int64_t n, int asymmetric,
                        float* y, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(x_dtype == Q4_F16 || x_dtype == Q4_BF16, Q4_ERR_DTYPE, "x_dtype must be Q4_F16 or Q4_BF16");
  Q4_REQUIRE(t >= 0 && k >= 128 && k % 128 == 0 && n >= 64 && n % 64 == 0, Q4_ERR_SHAPE,
             "need k %% 128 == 0 and n %% 64 == 0");
  Q4_REQUIRE(asymmetric == 0 || asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  if (t == 0) return ok();
  Q4_REQUIRE(x && w_dev && y, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(x) && !misaligned(w_dev) && !misaligned(y), Q4_ERR_ALIGN, "pointers must be 16-byte aligned");
  GemmArgs g{};
  g.a = x;
  g.w = static_cast<const uint8_t*>(w_dev);
  g.num_experts = 1;
  g.asym = asymmetric;
  g.N = n;
  g.K = k;
  g.dense_rows = t;
  g.a_rows = t;
  g.out = y;
  const int rb = t <= 16 ? 1 : (t <= 32 ? 2 : 4);
  return check_hip(launch_gemm(g, x_dtype == Q4_F16 ? 1 : 0, GEMM_PLAIN, rb, stream), "linear gemm");
}

int int8_w8a8_group_acc(const int8_t* q, int64_t rows, int64_t k, const void* w_dev, int64_t n, int32_t* acc,
                        hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(rows >= 0 && k >= 128 && k % 128 == 0 && n >= 64 && n % 64 == 0, Q4_ERR_SHAPE,
             "need k %% 128 == 0 and n %% 64 == 0");
  if (rows == 0) return ok();
  Q4_REQUIRE(q && w_dev && acc, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(q) && !misaligned(w_dev), Q4_ERR_ALIGN, "pointers must be 16-byte aligned");
  GemmArgs g{};
  g.a = q;
  g.w = static_cast<const uint8_t*>(w_dev);
  g.num_experts = 1;
  g.wbits = 8;
  g.N = n;
  g.K = k;
  g.dense_rows = rows;
  g.a_rows = rows;
  g.acc_out = acc;
  return check_hip(launch_gemm(g, 2, GEMM_GROUP_ACC, 1, stream), "group acc gemm");
}

int int2_w2a8_group_acc(const int8_t* q, int64_t rows, int64_t k, const void* w_dev, int64_t n, int32_t* acc,
                        hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(rows >= 0 && k >= 128 && k % 128 == 0 && n >= 64 && n % 64 == 0, Q4_ERR_SHAPE,
             "need k %% 128 == 0 and n %% 64 == 0");
  if (rows == 0) return ok();
  Q4_REQUIRE(q && w_dev && acc, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(q) && !misaligned(w_dev), Q4_ERR_ALIGN, "pointers must be 16-byte aligned");
  GemmArgs g{};
  g.a = q;
  g.w = static_cast<const uint8_t*>(w_dev);
  g.num_experts = 1;
  g.wbits = 2;
  g.N = n;
  g.K = k;
  g.dense_rows = rows;
  g.a_rows = rows;
  g.acc_out = acc;
  return check_hip(launch_gemm(g, 2, GEMM_GROUP_ACC, 1, stream), "group acc gemm");
}

int int4_w4a8_group_acc(const int8_t* q, int64_t rows, int64_t k, const void* w_dev, int64_t n, int asymmetric,
                        int32_t* acc, hipStream_t stream) {
  g_last_error.clear();
  Q4_REQUIRE(rows >= 0 && k >= 128 && k % 128 == 0 && n >= 64 && n % 64 == 0, Q4_ERR_SHAPE,
             "need k %% 128 == 0 and n %% 64 == 0");
  Q4_REQUIRE(asymmetric == 0 || asymmetric == 1, Q4_ERR_SHAPE, "asymmetric must be 0 or 1");
  if (rows == 0) return ok();
  Q4_REQUIRE(q && w_dev && acc, Q4_ERR_NULL, "missing pointer");
  Q4_REQUIRE(!misaligned(q) && !misaligned(w_dev), Q4_ERR_ALIGN, "pointers must be 16-byte aligned");
  GemmArgs g{};
  g.a = q;
  g.w = static_cast<const uint8_t*>(w_dev);
  g.num_experts = 1;
  g.asym = asymmetric;
  g.N = n;
  g.K = k;
  g.dense_rows = rows;
  g.a_rows = rows;
  g.acc_out = acc;
  return check_hip(launch_gemm(g, 2, GEMM_GROUP_ACC, 1, stream), "group acc gemm");
}

}  // extern "C"
