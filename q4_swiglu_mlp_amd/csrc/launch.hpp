// Host-side launchers of the library's kernels.  Every launcher assumes its
// arguments were validated by the C ABI layer (capi.cpp): shapes are
// multiples of 256, pointers are 16-byte aligned, sizes fit the workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zinc {

// ZINC_OK for hipSuccess; otherwise ZINC_ERR_HIP, and `e` becomes the text
// that zinc_hip_error_string() returns on this thread (capi.cpp).
int status_from_hip(hipError_t e);

// Kernel timing hook (timing.cpp): no-ops unless zinc_timing_enable() was called.
void timing_begin(hipStream_t stream);
void timing_end(hipStream_t stream);

hipError_t launch_q4k_dequant_f32(const void* blocks, int rows, int cols, float* out, hipStream_t stream);
// fmt 1: Q5_K (cols % 256 == 0), 2: Q5_1 (cols % 32 == 0).
hipError_t launch_q5_dequant_f32(int fmt, const void* blocks, int rows, int cols, float* out, hipStream_t stream);

// Fused prefill.
size_t prefill_workspace_bytes(int M, int hidden, int inter);
// mlp_scale multiplies the MLP output; res (nullable, [M x hidden] fp16, may be
// y) is added at the output scale: y = fp16((res + mlp_scale * MLP(x)) * 2^-out_shift).
hipError_t launch_prefill(const void* wg, const void* wu, const void* wd, int hidden, int inter,
                          const void* x, void* y, int M, int inter_shift, int out_shift, void* ws,
                          hipStream_t stream, float mlp_scale = 1.0f, const void* res = nullptr);

// The staged comparison baseline of the prefill: the same units with the
// gate/up outputs and the intermediate in device memory (four main launches).
size_t prefill_staged_workspace_bytes(int M, int hidden, int inter);
hipError_t launch_prefill_staged(const void* wg, const void* wu, const void* wd, int hidden, int inter,
                                 const void* x, void* y, int M, int inter_shift, int out_shift, void* ws,
                                 hipStream_t stream);

// Decode, 1 <= M <= 8: row-streaming dot products for M = 1 (k_decode.hip),
// 16x16x32 MFMA tiles for M >= 2 (k_decode_mfma.hip); both write the fp16
// intermediate [M x inter] into the workspace between their two kernels.
size_t decode_workspace_bytes(int M, int hidden, int inter);
// gamma (nullable): the pre-MLP RMS norm of x with weight gamma and eps is the
// MLP's input; xn ([M x hidden] fp16 scratch) receives it where a kernel of its
// own computes it.
hipError_t launch_decode(const void* wg, const void* wu, const void* wd, int hidden, int inter,
                         const void* x, void* y, int M, int inter_shift, int out_shift, void* ws,
                         hipStream_t stream, float mlp_scale = 1.0f, const void* res = nullptr,
                         const void* gamma = nullptr, float eps = 0.0f, void* xn = nullptr);
hipError_t launch_decode_mfma(const void* wg, const void* wu, const void* wd, int hidden, int inter,
                              const void* x, void* y, int M, int inter_shift, int out_shift, void* ws,
                              hipStream_t stream, float mlp_scale = 1.0f, const void* res = nullptr);

// Batched-expert MoE.
size_t moe_workspace_bytes(int M, int top_k, int n_experts, int hidden, int inter);
// down_fmt: 0 Q4_K, 1 Q5_K, 2 Q5_1 (W_down's block format; gate and up are Q4_K).
hipError_t launch_moe(const void* wg, const void* wu, const void* wd, int n_experts, int hidden, int inter,
                      const void* x, int M, const int32_t* ids, const float* p, int top_k, void* y,
                      int inter_shift, int out_shift, void* ws, int32_t* dev_error, hipStream_t stream,
                      int down_fmt = 0);

// MoE router: per token the top_k largest logits' experts and their softmax
// weights (k_router.hip).  1 <= top_k <= min(64, n_experts), n_experts <= 1024.
hipError_t launch_route_topk(const float* logits, int M, int n_experts, int top_k, int32_t* ids, float* p,
                             hipStream_t stream);

}  // namespace zinc
