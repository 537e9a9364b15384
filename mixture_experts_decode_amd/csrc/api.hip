// C ABI layer: argument validation (host only, before any launch), workspace
// sizing, regime choice, and dispatch to the kernel translation units.

#include <stdint.h>

#include "internal.h"
#include <atomic>
#include <cmath>
#include <algorithm>

#include "moe_mi355x.h"
#include "moe_mi355x_util.h"

namespace {

using moe::kDecodeMaxEntries;
using moe::kMaxExpertsTotal;

constexpr int32_t kAbiVersion = 3;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the measurement kernels give each 16-byte element its own thread, in at
// most 2^31-1 workgroups of 256
constexpr size_t kUtilMaxElems = size_t(0x7fffffff) * 256;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

moe_status from_hip(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return MOE_ERR_HIP;
}

bool dtype_ok(int32_t d) { return d == MOE_DT_F32 || d == MOE_DT_BF16; }

moe_status check_weights(const moe_weights* W) {
  if (!W) return MOE_ERR_INVALID_ARG;
  if (W->hidden <= 0 || W->inter <= 0 || W->num_experts <= 0) return MOE_ERR_INVALID_ARG;
  if (W->num_shared != 0 && W->num_shared != 1) return MOE_ERR_INVALID_ARG;
  if (W->num_experts + W->num_shared > kMaxExpertsTotal) return MOE_ERR_UNSUPPORTED;
  if (!W->w13 || !W->w2 || !aligned16(W->w13) || !aligned16(W->w2)) return MOE_ERR_INVALID_ARG;
  switch (W->format) {
    case MOE_W_F32:
      if (W->hidden % 4 || W->inter % 4) return MOE_ERR_UNSUPPORTED;
      break;
    case MOE_W_MXFP8:
    case MOE_W_MXFP4:
      if (!W->w13_scale || !W->w2_scale) return MOE_ERR_INVALID_ARG;
      if (W->hidden % 32 || W->inter % 32) return MOE_ERR_UNSUPPORTED;
      break;
    case MOE_W_FP8_BLK128:
      if (!W->w13_scale || !W->w2_scale) return MOE_ERR_INVALID_ARG;
      if (W->hidden % 128 || W->inter % 128) return MOE_ERR_UNSUPPORTED;
      break;
    default:
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status check_routing(const moe_weights* W, int32_t T, int32_t k) {
  if (T < 0 || k < 0) return MOE_ERR_INVALID_ARG;
  if (k + W->num_shared < 1) return MOE_ERR_INVALID_ARG;
  if (k > W->num_experts) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * (k + W->num_shared) > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool grouped_supported(const moe_weights* W) {
  return W->format == MOE_W_MXFP8 || W->format == MOE_W_MXFP4 ||
         W->format == MOE_W_FP8_BLK128;
}

bool block_ok(int32_t bs) { return bs == 32 || bs == 64 || bs == 128; }

// Grouped M block for block_size == 0: by the expected (token, slot) entries
// per expert under uniform routing.  32-row blocks were fastest measured at
// decode-like loads (about 9-16 entries per expert), 128 at the 16384-token
// prefill (about 512).
int32_t auto_block(const moe_weights* W, int32_t T, int32_t k) {
  const double per = (double)T * (k + W->num_shared) / (W->num_experts + W->num_shared);
  return per <= 48.0 ? 32 : per <= 160.0 ? 64 : 128;
}

// Stored bytes of one expert (weights and scales of gate, up and down).
double expert_bytes(const moe_weights* W) {
  const double hi = (double)W->hidden * W->inter;
  switch (W->format) {
    case MOE_W_F32: return 3.0 * hi * 4.0;
    case MOE_W_MXFP8: return 3.0 * hi * (1.0 + 1.0 / 32);
    case MOE_W_MXFP4: return 3.0 * hi * (0.5 + 1.0 / 32);
    default: return 3.0 * hi * (1.0 + 4.0 / (128.0 * 128.0));
  }
}

// Regime choice: output-centric decode for small batches, expert-centric
// packing beyond (the warp-decode post's section on Composer).  Both costs
// are modelled in microseconds with constants fitted to MI355X sweeps of both
// paths (steps replayed from a HIP graph, 32-row blocks for the grouped
// path) over the Qwen3 (MXFP8), DeepSeek-V3 (FP8 128x128) and MXFP4 layers:
//  decode : the touched experts' bytes at 5.9 TB/s and VALU work of
//           1.45e-7 us per (token, slot) entry per H*I overlap, with half of
//           the smaller of the two showing through, plus 4 us;
//           For E2M1 weights both decode kernels run on the matrix cores
//           and stream an expert's rows once per pass of up to 2, 8 or 12
//           entries: the touched experts' bytes at 4.86 TB/s, the bytes of
//           the further passes at 5.99 TB/s, 0.081 us per entry and 12.1 us;
//  grouped: the same bytes at 5.2 TB/s with the matrix work hidden, plus
//           25 us for sort, quantisation, combine and launches; for E2M1
//           weights 5.11 TB/s, 0.0057 us per entry and 42.8 us.
// (The E2M1 constants are a least-squares fit to both paths measured at
// B = 1, 2, 8, 24, 32, 40, 48, 56, 64, 96, 128, 256; the fit switches at
// 33 tokens, the measurements between 40 and 48 under uniform routing and
// below 24 under Zipf routing.)
// The touched experts are their expectation under uniform routing; skewed
// routing touches fewer, which favours the grouped path a little earlier
// than this predicts.
int32_t model_path(const moe_weights* W, int32_t T, int32_t k) {
  const double n = W->num_experts;
  const double p = std::min(1.0, (double)k / n);
  const double u = n * (1.0 - std::pow(1.0 - p, (double)T)) + W->num_shared;
  const double bytes = u * expert_bytes(W);
  const double entries = (double)T * (k + W->num_shared);
  double t_dec;
  if (moe::decode_on_matrix_cores(*W)) {
    const double extra = std::max(0.0, moe::decode_matrix_core_passes(*W, T, k) - u);
    t_dec = bytes / 4.86e6 + extra * expert_bytes(W) / 5.99e6 + 0.081 * entries + 12.1;
  } else {
    const double valu = entries * W->hidden * W->inter * 1.45e-7;
    const double mem_d = bytes / 5.9e6;
    t_dec = std::max(mem_d, valu) + 0.5 * std::min(mem_d, valu) + 4.0;
  }
  const double t_grp = W->format == MOE_W_MXFP4 ? bytes / 5.11e6 + 0.0057 * entries + 42.8
                                                 : bytes / 5.2e6 + 25.0;
  return t_grp < t_dec ? MOE_PATH_GROUPED : MOE_PATH_DECODE;
}

struct GroupedLayout {
  size_t sorted, expert_ids, offsets, npp, as_ws, xq, xs, hq, hs, slot_out, total;
  int32_t cap;
};

GroupedLayout grouped_layout(const moe_weights* W, int32_t T, int32_t k, int32_t bs) {
  GroupedLayout L{};
  const int32_t slots = k + W->num_shared;
  const int32_t n = T * slots;
  const int32_t n_exp = W->num_experts + W->num_shared;
  L.cap = n + n_exp * (bs - 1);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  L.sorted = take((size_t)L.cap * 4);
  L.expert_ids = take((size_t)(L.cap / bs + 1) * 4);
  L.offsets = take((size_t)(n_exp + 1) * 4);
  L.npp = take(4);
  L.as_ws = take(moe::align_sort_workspace_bytes(n, n_exp));
  L.xq = take((size_t)T * W->hidden);                // each token quantised once
  L.xs = take((size_t)T * (W->hidden / 32));
  L.hq = take((size_t)2 * L.cap * W->inter);          // hi and lo terms
  L.hs = take((size_t)2 * L.cap * (W->inter / 32));
  L.slot_out = take((size_t)n * W->hidden * 2);      // BF16 slot outputs
  L.total = off;
  return L;
}

// The decode path keeps h in BF16 (FP32 with FP32 weights), the precision of
// the warp-decode post's activations (accuracy section).
int32_t decode_h_dtype(const moe_weights* W) {
  return W->format == MOE_W_F32 ? MOE_DT_F32 : MOE_DT_BF16;
}

size_t decode_h_bytes(const moe_weights* W, int32_t T, int32_t k) {
  const size_t el = decode_h_dtype(W) == MOE_DT_BF16 ? 2 : 4;
  return align_up((size_t)T * (k + W->num_shared) * W->inter * el);
}

// The decode path's workspace: h, then (when AUTO runs the down product
// expert-major) the FP32 slot outputs.
size_t decode_slot_bytes(const moe_weights* W, int32_t T, int32_t k) {
  if (moe::down_auto_variant(*W, T, k) != MOE_DOWN_EXPERT_MAJOR) return 0;
  return align_up((size_t)T * (k + W->num_shared) * W->hidden * 4);
}

size_t decode_workspace(const moe_weights* W, int32_t T, int32_t k) {
  return decode_h_bytes(W, T, k) + decode_slot_bytes(W, T, k);
}

// ---- workspace held by the library, for callers that cannot allocate -----

constexpr size_t kScratchBytes = size_t(32) << 20;   // per device
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];

}  // namespace

// The workspace of moe_layer_noalloc: one copy per device, alive until the
// process ends.  Host code never passes the symbol itself to a kernel (on the
// host it only names the variable); it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of the current device's copy of `scratch`, looked up on
// that device's first call and kept.  Concurrent first calls look it up twice
// and store the same address.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int32_t moe_abi_version(void) { return kAbiVersion; }

int32_t moe_decode_max_entries(void) { return kDecodeMaxEntries; }

moe_status moe_gate_up(const moe_weights* W, const void* x, int32_t x_dtype,
                       const int32_t* topk_ids, int32_t T, int32_t k, void* h, int32_t h_dtype,
                       void* stream) {
  moe_status st = check_weights(W);
  if (st != MOE_OK) return st;
  if ((st = check_routing(W, T, k)) != MOE_OK) return st;
  if (!dtype_ok(x_dtype) || !dtype_ok(h_dtype)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !h || (k > 0 && !topk_ids) || !aligned16(x)) return MOE_ERR_INVALID_ARG;
  if (x_dtype == MOE_DT_F32 && W->format != MOE_W_F32) return MOE_ERR_UNSUPPORTED;
  // FP32 weights pair with an FP32 h: moe_down takes no BF16 h for them
  if (h_dtype == MOE_DT_BF16 && W->format == MOE_W_F32) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * (k + W->num_shared) > kDecodeMaxEntries) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_gate_up_decode(*W, x, x_dtype, topk_ids, T, k, h, h_dtype,
                                             as_stream(stream)));
}

size_t moe_down_workspace_bytes(const moe_weights* W, int32_t T, int32_t k) {
  if (check_weights(W) != MOE_OK || T < 0 || k < 0) return 0;
  return (size_t)T * (k + W->num_shared) * W->hidden * sizeof(float);
}

moe_status moe_down(const moe_weights* W, const void* h, int32_t h_dtype,
                    const int32_t* topk_ids, const float* topk_weights, int32_t T, int32_t k,
                    void* y, int32_t y_dtype, int32_t variant, void* workspace,
                    size_t workspace_bytes, void* stream) {
  moe_status st = check_weights(W);
  if (st != MOE_OK) return st;
  if ((st = check_routing(W, T, k)) != MOE_OK) return st;
  if (!dtype_ok(h_dtype) || !dtype_ok(y_dtype)) return MOE_ERR_INVALID_ARG;
  if (variant < MOE_DOWN_AUTO || variant > MOE_DOWN_EXPERT_MAJOR) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!h || !y || (k > 0 && (!topk_ids || !topk_weights)) || !aligned16(h))
    return MOE_ERR_INVALID_ARG;
  if (h_dtype == MOE_DT_BF16 && W->format == MOE_W_F32) return MOE_ERR_UNSUPPORTED;
  if (k + W->num_shared > 64) return MOE_ERR_UNSUPPORTED;   // one slot per lane
  if (moe::down_lanes_per_row(W->format, W->inter, h_dtype) == 0) return MOE_ERR_UNSUPPORTED;
  if (variant == MOE_DOWN_AUTO) variant = moe::down_auto_variant(*W, T, k);
  if (variant == MOE_DOWN_EXPERT_MAJOR) {
    if (!workspace) return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < moe_down_workspace_bytes(W, T, k)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  }
  return from_hip(moe::launch_down_decode(*W, h, h_dtype, topk_ids, topk_weights, T, k, y,
                                          y_dtype, variant, reinterpret_cast<float*>(workspace),
                                          as_stream(stream)));
}

size_t moe_align_sort_capacity(int32_t T, int32_t k, int32_t num_experts, int32_t num_shared,
                               int32_t block_size) {
  if (T < 0 || k < 0 || num_experts < 1 || num_shared < 0 || block_size < 1) return 0;
  return (size_t)T * (k + num_shared) + (size_t)(num_experts + num_shared) * (block_size - 1);
}

size_t moe_align_sort_workspace_bytes(int32_t T, int32_t k, int32_t num_experts,
                                      int32_t num_shared, int32_t block_size) {
  (void)block_size;
  if (T < 0 || k < 0 || num_experts < 1 || num_shared < 0) return 0;
  return moe::align_sort_workspace_bytes(T * (k + num_shared), num_experts + num_shared);
}

moe_status moe_align_sort(const int32_t* topk_ids, int32_t T, int32_t k, int32_t num_experts,
                          int32_t num_shared, int32_t block_size, int32_t* sorted_token_ids,
                          int32_t* expert_ids, int32_t* expert_offsets,
                          int32_t* num_tokens_post_padded, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (T < 0 || k < 0 || num_experts < 1 || (num_shared != 0 && num_shared != 1))
    return MOE_ERR_INVALID_ARG;
  if (k + num_shared < 1 || k > num_experts) return MOE_ERR_INVALID_ARG;
  if (num_experts + num_shared > kMaxExpertsTotal) return MOE_ERR_UNSUPPORTED;
  if (block_size < 1 || block_size > 1024) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * (k + num_shared) + (int64_t)(num_experts + num_shared) * block_size >
      INT32_MAX / 2)
    return MOE_ERR_UNSUPPORTED;
  if ((k > 0 && T > 0 && !topk_ids) || !sorted_token_ids || !expert_ids || !expert_offsets ||
      !num_tokens_post_padded || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes <
      moe_align_sort_workspace_bytes(T, k, num_experts, num_shared, block_size))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(moe::launch_align_sort(topk_ids, T, k, num_experts, num_shared, block_size,
                                         sorted_token_ids, expert_ids, expert_offsets,
                                         num_tokens_post_padded, workspace,
                                         as_stream(stream)));
}

moe_status moe_quant_rows(const void* x, int32_t x_dtype, int32_t T, int32_t H, uint8_t* xq,
                          uint8_t* xs, void* stream) {
  if (!dtype_ok(x_dtype) || T < 0 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !xq || !xs) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * H > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_quant_rows(x, x_dtype, T, H, xq, xs, as_stream(stream)));
}

moe_status moe_grouped_gate_up(const moe_weights* W, const uint8_t* xq, const uint8_t* xs,
                               int32_t T, int32_t k, const int32_t* sorted_token_ids,
                               const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                               int32_t capacity, int32_t block_size, uint8_t* hq, uint8_t* hs,
                               void* stream) {
  moe_status st = check_weights(W);
  if (st != MOE_OK) return st;
  if ((st = check_routing(W, T, k)) != MOE_OK) return st;
  if (!grouped_supported(W) || !block_ok(block_size)) return MOE_ERR_UNSUPPORTED;
  if (W->hidden % 128 || W->inter % 128) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * W->hidden > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  if (capacity == 0 || T == 0) return MOE_OK;
  if (!xq || !xs || !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !hq || !hs)
    return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_grouped_gate_up(*W, xq, xs, T, k + W->num_shared, sorted_token_ids,
                                              expert_ids, num_tokens_post_padded, capacity,
                                              block_size, hq, hs, as_stream(stream)));
}

moe_status moe_grouped_down(const moe_weights* W, const uint8_t* hq, const uint8_t* hs,
                            const int32_t* sorted_token_ids, const int32_t* expert_ids,
                            const int32_t* num_tokens_post_padded, int32_t capacity,
                            int32_t block_size, const float* topk_weights, int32_t T, int32_t k,
                            uint16_t* slot_out, void* stream) {
  moe_status st = check_weights(W);
  if (st != MOE_OK) return st;
  if ((st = check_routing(W, T, k)) != MOE_OK) return st;
  if (!grouped_supported(W) || !block_ok(block_size)) return MOE_ERR_UNSUPPORTED;
  if (W->hidden % 128 || W->inter % 128) return MOE_ERR_UNSUPPORTED;
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  if (capacity == 0 || T == 0) return MOE_OK;
  if (!hq || !hs || !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !slot_out ||
      (k > 0 && !topk_weights))
    return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_grouped_down(*W, hq, hs, sorted_token_ids, expert_ids,
                                           num_tokens_post_padded, capacity, block_size,
                                           topk_weights, T, k, slot_out, as_stream(stream)));
}

moe_status moe_combine(const uint16_t* slot_out, int32_t T, int32_t slots, int32_t H, void* y,
                       int32_t y_dtype, void* stream) {
  if (T < 0 || slots < 1 || H <= 0 || !dtype_ok(y_dtype)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!slot_out || !y) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_combine(slot_out, MOE_DT_BF16, T, slots, H, y, y_dtype,
                                      as_stream(stream)));
}

moe_status moe_topk_route(const float* scores, const float* bias, int32_t T, int32_t E, int32_t k,
                          int32_t* topk_ids, float* topk_weights, void* stream) {
  if (T < 0 || E < 1 || E > kMaxExpertsTotal || k < 1 || k > E || k > 64)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!scores || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * E > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_topk_route(scores, bias, T, E, k, topk_ids, topk_weights,
                                         as_stream(stream)));
}

moe_status moe_check_routing(const int32_t* topk_ids, int32_t T, int32_t k, int32_t num_experts,
                             int32_t* result, void* stream) {
  if (T < 0 || k < 1 || num_experts < 1) return MOE_ERR_INVALID_ARG;
  if (!result || (T > 0 && !topk_ids)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_check_routing(topk_ids, T * k, num_experts, result,
                                            as_stream(stream)));
}

int32_t moe_choose_path(const moe_weights* W, int32_t T, int32_t k) {
  if (check_weights(W) != MOE_OK || check_routing(W, T, k) != MOE_OK) return MOE_PATH_DECODE;
  if (!grouped_supported(W) || W->hidden % 128 || W->inter % 128) return MOE_PATH_DECODE;
  // a path the decode kernels refuse (too many entries to stage on chip, more
  // than 64 slots, a row length with no compiled shape) is never picked
  if (moe::decode_supported(*W, T, k, decode_h_dtype(W)) != hipSuccess)
    return MOE_PATH_GROUPED;
  return model_path(W, T, k);
}

size_t moe_layer_workspace_bytes(const moe_weights* W, int32_t T, int32_t k, int32_t path,
                                 int32_t block_size) {
  if (check_weights(W) != MOE_OK || T < 0 || k < 0) return 0;
  if (path == MOE_PATH_AUTO) path = moe_choose_path(W, T, k);
  if (path == MOE_PATH_DECODE) return decode_workspace(W, T, k);
  if (block_size == 0) block_size = auto_block(W, T, k);
  if (path == MOE_PATH_GROUPED && block_ok(block_size))
    return grouped_layout(W, T, k, block_size).total;
  return 0;
}

moe_status moe_layer(const moe_weights* W, const void* x, int32_t x_dtype,
                     const int32_t* topk_ids, const float* topk_weights, int32_t T, int32_t k,
                     void* y, int32_t y_dtype, int32_t path, int32_t block_size, void* workspace,
                     size_t workspace_bytes, int32_t* chosen, void* stream) {
  moe_status st = check_weights(W);
  if (st != MOE_OK) return st;
  if ((st = check_routing(W, T, k)) != MOE_OK) return st;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return MOE_ERR_INVALID_ARG;
  if (path != MOE_PATH_AUTO && path != MOE_PATH_DECODE && path != MOE_PATH_GROUPED)
    return MOE_ERR_INVALID_ARG;
  if (path == MOE_PATH_AUTO) path = moe_choose_path(W, T, k);
  if (chosen) *chosen = path;
  if (T == 0) return MOE_OK;
  if (!x || !y || (k > 0 && (!topk_ids || !topk_weights)) || !workspace)
    return MOE_ERR_INVALID_ARG;
  // FP32 activations go with FP32 weights only, on either path
  if (x_dtype == MOE_DT_F32 && W->format != MOE_W_F32) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const int32_t slots = k + W->num_shared;
  if (path == MOE_PATH_DECODE) {
    if (workspace_bytes < decode_workspace(W, T, k)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace) || !aligned16(x)) return MOE_ERR_INVALID_ARG;
    const int32_t hdt = decode_h_dtype(W);
    // every shape limit of both kernels is checked before the first launch
    if (moe::decode_supported(*W, T, k, hdt) != hipSuccess) return MOE_ERR_UNSUPPORTED;
    st = moe_gate_up(W, x, x_dtype, topk_ids, T, k, workspace, hdt, stream);
    if (st != MOE_OK) return st;
    const size_t hb = decode_h_bytes(W, T, k);
    const size_t sb = decode_slot_bytes(W, T, k);
    return moe_down(W, workspace, hdt, topk_ids, topk_weights, T, k, y, y_dtype, MOE_DOWN_AUTO,
                    sb ? reinterpret_cast<char*>(workspace) + hb : nullptr, sb, stream);
  }
  // grouped
  if (block_size == 0) block_size = auto_block(W, T, k);
  if (!grouped_supported(W) || !block_ok(block_size)) return MOE_ERR_UNSUPPORTED;
  if (W->hidden % 128 || W->inter % 128) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * W->hidden > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x)) return MOE_ERR_INVALID_ARG;
  const GroupedLayout L = grouped_layout(W, T, k, block_size);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_ERR_INVALID_ARG;
  char* ws = reinterpret_cast<char*>(workspace);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(ws + L.expert_ids);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* npp = reinterpret_cast<int32_t*>(ws + L.npp);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + L.xs);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + L.hs);
  uint16_t* so = reinterpret_cast<uint16_t*>(ws + L.slot_out);
  hipError_t e = moe::launch_front_end(topk_ids, T, k, W->num_experts, W->num_shared, block_size,
                                       sorted, eids, offs, npp, ws + L.as_ws, x, x_dtype, W->hidden,
                                       xq, xs, s);
  if (e != hipSuccess) return from_hip(e);
  e = moe::launch_grouped_gate_up(*W, xq, xs, T, slots, sorted, eids, npp, L.cap, block_size, hq,
                                  hs, s);
  if (e != hipSuccess) return from_hip(e);
  e = moe::launch_grouped_down(*W, hq, hs, sorted, eids, npp, L.cap, block_size, topk_weights, T,
                               k, so, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(moe::launch_combine(so, MOE_DT_BF16, T, slots, W->hidden, y, y_dtype, s));
}

size_t moe_layer_noalloc_max_bytes(void) { return kScratchBytes; }

moe_status moe_layer_noalloc(const moe_weights* W, const void* x, int32_t x_dtype,
                             const int32_t* topk_ids, const float* topk_weights, int32_t T,
                             int32_t k, void* y, int32_t y_dtype, int32_t path,
                             int32_t block_size, int32_t* chosen, void* stream) {
  moe_status st = check_weights(W);
  if (st != MOE_OK) return st;
  if ((st = check_routing(W, T, k)) != MOE_OK) return st;
  if (path != MOE_PATH_AUTO && path != MOE_PATH_DECODE && path != MOE_PATH_GROUPED)
    return MOE_ERR_INVALID_ARG;
  if (T == 0)
    return moe_layer(W, x, x_dtype, topk_ids, topk_weights, T, k, y, y_dtype, path, block_size,
                     nullptr, 0, chosen, stream);
  // the whole workspace of this call must fit the library's array
  if (moe_layer_workspace_bytes(W, T, k, path, block_size) > kScratchBytes)
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return from_hip(e);
  return moe_layer(W, x, x_dtype, topk_ids, topk_weights, T, k, y, y_dtype, path, block_size, ws,
                   kScratchBytes, chosen, stream);
}

// ---- measurement helpers -----------------------------------------------

moe_status moe_util_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  if (bytes / 16 > kUtilMaxElems) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_copy(src, dst, bytes, as_stream(stream)));
}

moe_status moe_util_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes % 16 || !aligned16(src)) return MOE_ERR_INVALID_ARG;
  if (bytes / 16 > kUtilMaxElems) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_read(src, bytes, sink, as_stream(stream)));
}

int32_t moe_util_read_sink_len(void) { return moe::kReadSinkLen; }

moe_status moe_util_fill(void* dst, size_t bytes, uint32_t value, void* stream) {
  if (!dst || bytes % 16 || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  if (bytes / 16 > kUtilMaxElems) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_fill(dst, bytes, value, as_stream(stream)));
}

int32_t moe_util_num_cus(void) { return moe::device_num_cus(); }

}  // extern "C"
