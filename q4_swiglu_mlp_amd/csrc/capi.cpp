// C ABI of the library (include/zinc_mlp.h): host-side argument checks, then
// the launchers.  Every check runs before the first HIP call, so a rejected
// call enqueues nothing and needs no GPU.
#include "../../include/zinc_mlp.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include <cmath>

#include "launch.hpp"
#include "util_kernels.hpp"

namespace {

constexpr int kMaxHidden = 16384;
constexpr int kMaxInter = 65536;
constexpr int kMaxShift = 30;
constexpr int kMaxDecodeM = 8;
constexpr int kMaxExperts = 1024;
constexpr long long kMaxPrefillM = 1 << 20;
constexpr long long kMaxMoeSlots = 1 << 24;
constexpr int kMaxRouterTopK = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dim_ok(int32_t v, int32_t max) { return v > 0 && v % 256 == 0 && v <= max; }

// The fused 64-token unit addresses its staged activation, (M + 1) tokens x
// (hidden / 256) columns x 544 bytes, with 32-bit byte offsets.
bool staged_ok(long long M, int32_t hidden) { return (M + 1) * (hidden / 256) * 544LL <= 0xFFFFFFFFLL; }

// The MoE partial rows of one intermediate chunk, (M*top_k + 1) x hidden fp16,
// are addressed with 32-bit byte offsets: they must stay below 2 GiB.
bool moe_rows_ok(int32_t M, int32_t top_k, int32_t hidden) {
  return ((long long)M * top_k + 1) * hidden * 2 <= 0x7FFFFFFFLL;
}

thread_local const char* t_last_hip_error = "no HIP error";

int from_hip(hipError_t e) { return zinc::status_from_hip(e); }

// Checks shared by the dense entry points.
int check_dense(const void* wg, const void* wu, const void* wd, int32_t hidden, int32_t inter, const void* x,
                const void* y, int32_t M, int32_t inter_shift, int32_t out_shift, long long max_m) {
  if (!wg || !wu || !wd || !x || !y) return ZINC_ERR_NULL;
  if (!dim_ok(hidden, kMaxHidden) || !dim_ok(inter, kMaxInter)) return ZINC_ERR_SHAPE;
  if (!aligned16(wg) || !aligned16(wu) || !aligned16(wd) || !aligned16(x) || !aligned16(y)) return ZINC_ERR_ALIGN;
  if (M < 0 || M > max_m || !staged_ok(M, hidden)) return ZINC_ERR_ARG;
  if (inter_shift < 0 || inter_shift > kMaxShift || out_shift < 0 || out_shift > kMaxShift) return ZINC_ERR_ARG;
  return ZINC_OK;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The block entry points: the normalised activation sits after the wrapped
// call's own workspace.
size_t xn_bytes(int32_t M, int32_t hidden) { return align256((size_t)(M > 0 ? M : 1) * hidden * 2); }

int check_block(const void* norm_weight, float eps, float mlp_scale) {
  if (!norm_weight) return ZINC_ERR_NULL;
  if (!aligned16(norm_weight)) return ZINC_ERR_ALIGN;
  if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(mlp_scale)) return ZINC_ERR_ARG;
  return ZINC_OK;
}

}  // namespace

namespace zinc {

int status_from_hip(hipError_t e) {
  if (e == hipSuccess) return ZINC_OK;
  t_last_hip_error = hipGetErrorString(e);
  return ZINC_ERR_HIP;
}

}  // namespace zinc

extern "C" {

const char* zinc_strerror(int status) {
  switch (status) {
    case ZINC_OK: return "ok";
    case ZINC_ERR_NULL: return "a required pointer is NULL";
    case ZINC_ERR_SHAPE: return "hidden/inter/cols must be positive multiples of 256 within the supported range";
    case ZINC_ERR_ALIGN: return "a pointer is not aligned as required (16 bytes; 4 for ids/weights/error flag)";
    case ZINC_ERR_WORKSPACE: return "workspace smaller than the matching *_workspace_size()";
    case ZINC_ERR_ARG: return "argument out of range (M, shift or top_k)";
    case ZINC_ERR_HIP: return "a HIP launch or runtime call failed";
    case ZINC_ERR_UNSUPPORTED: return "size not supported by the library";
    default: return "unknown zinc status";
  }
}

const char* zinc_hip_error_string(void) { return t_last_hip_error; }

int zinc_q4k_dequant_f32(const void* blocks, int32_t rows, int32_t cols, float* out, void* stream) {
  if (!blocks || !out) return ZINC_ERR_NULL;
  if (cols <= 0 || cols % 256 != 0) return ZINC_ERR_SHAPE;
  if (rows < 0) return ZINC_ERR_ARG;
  if ((long long)rows * cols > INT32_MAX) return ZINC_ERR_SHAPE;
  if (!aligned16(blocks) || !aligned16(out)) return ZINC_ERR_ALIGN;
  if (rows == 0) return ZINC_OK;
  (void)hipGetLastError();
  return from_hip(zinc::launch_q4k_dequant_f32(blocks, rows, cols, out, static_cast<hipStream_t>(stream)));
}

static int q5_dequant(int fmt, const void* blocks, int32_t rows, int32_t cols, float* out, void* stream) {
  if (!blocks || !out) return ZINC_ERR_NULL;
  if (cols <= 0 || cols % (fmt == 1 ? 256 : 32) != 0) return ZINC_ERR_SHAPE;
  if (rows < 0) return ZINC_ERR_ARG;
  if ((long long)rows * cols > INT32_MAX) return ZINC_ERR_SHAPE;
  if (!aligned16(blocks) || !aligned16(out)) return ZINC_ERR_ALIGN;
  if (rows == 0) return ZINC_OK;
  (void)hipGetLastError();
  return from_hip(zinc::launch_q5_dequant_f32(fmt, blocks, rows, cols, out, static_cast<hipStream_t>(stream)));
}

int zinc_q5k_dequant_f32(const void* blocks, int32_t rows, int32_t cols, float* out, void* stream) {
  return q5_dequant(1, blocks, rows, cols, out, stream);
}

int zinc_q5_1_dequant_f32(const void* blocks, int32_t rows, int32_t cols, float* out, void* stream) {
  return q5_dequant(2, blocks, rows, cols, out, stream);
}

size_t zinc_mlp_q4k_prefill_workspace_size(int32_t M, int32_t hidden, int32_t inter) {
  if (M < 0 || M > kMaxPrefillM || !dim_ok(hidden, kMaxHidden) || !dim_ok(inter, kMaxInter)) return 0;
  if (!staged_ok(M, hidden)) return 0;
  return zinc::prefill_workspace_bytes(M, hidden, inter);
}

int zinc_mlp_q4k_prefill(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden, int32_t inter,
                         const void* x_f16, void* y_f16, int32_t M, int32_t inter_shift, int32_t out_shift,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift, kMaxPrefillM);
  if (st != ZINC_OK) return st;
  if (M == 0) return ZINC_OK;
  if (!workspace) return ZINC_ERR_NULL;
  if (!aligned16(workspace)) return ZINC_ERR_ALIGN;
  if (workspace_bytes < zinc::prefill_workspace_bytes(M, hidden, inter)) return ZINC_ERR_WORKSPACE;
  (void)hipGetLastError();
  return from_hip(zinc::launch_prefill(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift,
                                       workspace, static_cast<hipStream_t>(stream)));
}

size_t zinc_mlp_q4k_prefill_block_workspace_size(int32_t M, int32_t hidden, int32_t inter) {
  const size_t base = zinc_mlp_q4k_prefill_workspace_size(M, hidden, inter);
  return base ? align256(base) + xn_bytes(M, hidden) : 0;
}

int zinc_mlp_q4k_prefill_block(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden,
                               int32_t inter, const void* x_f16, const void* norm_weight_f16, float norm_eps,
                               float mlp_scale, void* y_f16, int32_t M, int32_t inter_shift, int32_t out_shift,
                               void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift, kMaxPrefillM);
  if (st != ZINC_OK) return st;
  st = check_block(norm_weight_f16, norm_eps, mlp_scale);
  if (st != ZINC_OK) return st;
  if (M == 0) return ZINC_OK;
  if (!workspace) return ZINC_ERR_NULL;
  if (!aligned16(workspace)) return ZINC_ERR_ALIGN;
  const size_t base = align256(zinc::prefill_workspace_bytes(M, hidden, inter));
  if (workspace_bytes < base + xn_bytes(M, hidden)) return ZINC_ERR_WORKSPACE;
  _Float16* xn = reinterpret_cast<_Float16*>(static_cast<uint8_t*>(workspace) + base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  zinc::launch_rms_norm(static_cast<const _Float16*>(x_f16), static_cast<const _Float16*>(norm_weight_f16), norm_eps,
                        hidden, M, xn, s);
  return from_hip(zinc::launch_prefill(w_gate, w_up, w_down, hidden, inter, xn, y_f16, M, inter_shift, out_shift,
                                       workspace, s, mlp_scale, x_f16));
}

size_t zinc_mlp_q4k_prefill_staged_workspace_size(int32_t M, int32_t hidden, int32_t inter) {
  if (M < 0 || M > kMaxPrefillM || !dim_ok(hidden, kMaxHidden) || !dim_ok(inter, kMaxInter) || !staged_ok(M, hidden))
    return 0;
  return zinc::prefill_staged_workspace_bytes(M, hidden, inter);
}

int zinc_mlp_q4k_prefill_staged(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden,
                                int32_t inter, const void* x_f16, void* y_f16, int32_t M, int32_t inter_shift,
                                int32_t out_shift, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift, kMaxPrefillM);
  if (st != ZINC_OK) return st;
  if (M == 0) return ZINC_OK;
  if (!workspace) return ZINC_ERR_NULL;
  if (!aligned16(workspace)) return ZINC_ERR_ALIGN;
  if (workspace_bytes < zinc::prefill_staged_workspace_bytes(M, hidden, inter)) return ZINC_ERR_WORKSPACE;
  (void)hipGetLastError();
  return from_hip(zinc::launch_prefill_staged(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift,
                                              out_shift, workspace, static_cast<hipStream_t>(stream)));
}

size_t zinc_mlp_q4k_decode_workspace_size(int32_t M, int32_t hidden, int32_t inter) {
  if (M < 0 || M > kMaxDecodeM || !dim_ok(hidden, kMaxHidden) || !dim_ok(inter, kMaxInter)) return 0;
  return zinc::decode_workspace_bytes(M, hidden, inter);
}

int zinc_mlp_q4k_decode(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden, int32_t inter,
                        const void* x_f16, void* y_f16, int32_t M, int32_t inter_shift, int32_t out_shift,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift, kMaxDecodeM);
  if (st != ZINC_OK) return st;
  if (M == 0) return ZINC_OK;
  if (!workspace) return ZINC_ERR_NULL;
  if (!aligned16(workspace)) return ZINC_ERR_ALIGN;
  if (workspace_bytes < zinc::decode_workspace_bytes(M, hidden, inter)) return ZINC_ERR_WORKSPACE;
  (void)hipGetLastError();
  return from_hip(zinc::launch_decode(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift,
                                      workspace, static_cast<hipStream_t>(stream)));
}

size_t zinc_moe_q4k_experts_workspace_size(int32_t M, int32_t top_k, int32_t n_experts, int32_t hidden,
                                           int32_t inter) {
  if (M < 0 || n_experts < 1 || n_experts > kMaxExperts || top_k < 1 || top_k > n_experts) return 0;
  if ((long long)M * top_k > kMaxMoeSlots) return 0;
  if (!dim_ok(hidden, kMaxHidden) || !dim_ok(inter, kMaxInter)) return 0;
  if (!moe_rows_ok(M, top_k, hidden) || !staged_ok(M, hidden)) return 0;
  return zinc::moe_workspace_bytes(M, top_k, n_experts, hidden, inter);
}

int zinc_moe_q4k_experts(const void* w_gate, const void* w_up, const void* w_down, int32_t n_experts, int32_t hidden,
                         int32_t inter, const void* x_f16, int32_t M, const int32_t* expert_ids,
                         const float* expert_weights, int32_t top_k, void* y_f16, int32_t inter_shift,
                         int32_t out_shift, void* workspace, size_t workspace_bytes, int32_t* dev_error,
                         void* stream) {
  return zinc_moe_experts_fmt(w_gate, w_up, w_down, ZINC_DOWN_Q4_K, n_experts, hidden, inter, x_f16, M, expert_ids,
                              expert_weights, top_k, y_f16, inter_shift, out_shift, workspace, workspace_bytes,
                              dev_error, stream);
}

int zinc_moe_experts_fmt(const void* w_gate, const void* w_up, const void* w_down, int32_t down_format,
                         int32_t n_experts, int32_t hidden, int32_t inter, const void* x_f16, int32_t M,
                         const int32_t* expert_ids, const float* expert_weights, int32_t top_k, void* y_f16,
                         int32_t inter_shift, int32_t out_shift, void* workspace, size_t workspace_bytes,
                         int32_t* dev_error, void* stream) {
  if (!w_gate || !w_up || !w_down || !x_f16 || !y_f16 || !expert_ids || !expert_weights) return ZINC_ERR_NULL;
  if (!dim_ok(hidden, kMaxHidden) || !dim_ok(inter, kMaxInter)) return ZINC_ERR_SHAPE;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(x_f16) || !aligned16(y_f16) ||
      !aligned4(expert_ids) || !aligned4(expert_weights) || (dev_error && !aligned4(dev_error)))
    return ZINC_ERR_ALIGN;
  if (n_experts < 1 || n_experts > kMaxExperts || top_k < 1 || top_k > n_experts) return ZINC_ERR_ARG;
  if (M < 0 || (long long)M * top_k > kMaxMoeSlots) return ZINC_ERR_ARG;
  if (!moe_rows_ok(M, top_k, hidden) || !staged_ok(M, hidden)) return ZINC_ERR_ARG;
  if (inter_shift < 0 || inter_shift > kMaxShift || out_shift < 0 || out_shift > kMaxShift) return ZINC_ERR_ARG;
  if (down_format != ZINC_DOWN_Q4_K && down_format != ZINC_DOWN_Q5_K && down_format != ZINC_DOWN_Q5_1)
    return ZINC_ERR_ARG;
  if (M == 0) return ZINC_OK;
  if (!workspace) return ZINC_ERR_NULL;
  if (!aligned16(workspace)) return ZINC_ERR_ALIGN;
  if (workspace_bytes < zinc::moe_workspace_bytes(M, top_k, n_experts, hidden, inter)) return ZINC_ERR_WORKSPACE;
  (void)hipGetLastError();
  return from_hip(zinc::launch_moe(w_gate, w_up, w_down, n_experts, hidden, inter, x_f16, M, expert_ids,
                                   expert_weights, top_k, y_f16, inter_shift, out_shift, workspace, dev_error,
                                   static_cast<hipStream_t>(stream), down_format));
}

int zinc_moe_route_topk(const float* logits, int32_t M, int32_t n_experts, int32_t top_k, int32_t* expert_ids,
                        float* expert_weights, void* stream) {
  if (n_experts < 1 || n_experts > kMaxExperts || top_k < 1 || top_k > n_experts || top_k > kMaxRouterTopK)
    return ZINC_ERR_ARG;
  if (M < 0 || (long long)M * top_k > kMaxMoeSlots) return ZINC_ERR_ARG;
  if (M == 0) return ZINC_OK;   // nothing is read or written (empty buffers may be NULL)
  if (!logits || !expert_ids || !expert_weights) return ZINC_ERR_NULL;
  if (!aligned4(logits) || !aligned4(expert_ids) || !aligned4(expert_weights)) return ZINC_ERR_ALIGN;
  (void)hipGetLastError();
  return from_hip(zinc::launch_route_topk(logits, M, n_experts, top_k, expert_ids, expert_weights,
                                          static_cast<hipStream_t>(stream)));
}

size_t zinc_mlp_q4k_decode_block_workspace_size(int32_t M, int32_t hidden, int32_t inter) {
  const size_t base = zinc_mlp_q4k_decode_workspace_size(M, hidden, inter);
  return base ? align256(base) + xn_bytes(M, hidden) : 0;
}

int zinc_mlp_q4k_decode_block(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden,
                              int32_t inter, const void* x_f16, const void* norm_weight_f16, float norm_eps,
                              float mlp_scale, void* y_f16, int32_t M, int32_t inter_shift, int32_t out_shift,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift, kMaxDecodeM);
  if (st != ZINC_OK) return st;
  st = check_block(norm_weight_f16, norm_eps, mlp_scale);
  if (st != ZINC_OK) return st;
  if (M == 0) return ZINC_OK;
  if (!workspace) return ZINC_ERR_NULL;
  if (!aligned16(workspace)) return ZINC_ERR_ALIGN;
  const size_t base = align256(zinc::decode_workspace_bytes(M, hidden, inter));
  if (workspace_bytes < base + xn_bytes(M, hidden)) return ZINC_ERR_WORKSPACE;
  void* xn = static_cast<uint8_t*>(workspace) + base;
  (void)hipGetLastError();
  return from_hip(zinc::launch_decode(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift,
                                      workspace, static_cast<hipStream_t>(stream), mlp_scale, x_f16,
                                      norm_weight_f16, norm_eps, xn));
}

}  // extern "C"
