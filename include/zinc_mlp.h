/*
 * zinc_mlp.h -- C ABI of the MI355X (gfx950) Q4_K SwiGLU MLP library.
 *
 * The operation is the SwiGLU feed-forward block described on the page
 * "Fused SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth" (section "The MLP is
 * two trips up to a wider width"): the hidden state is projected up twice, by
 * a gate weight and an up weight, combined by SwiGLU, and projected back down:
 *
 *     y = W_down . ( silu(W_gate . x)  (*)  (W_up . x) ),   silu(z) = z / (1 + e^-z)
 *
 * with every weight matrix stored as Q4_K super-blocks and unpacked in
 * registers on the way into the multiply (same page, opening Q&A; "VGPR
 * pressure caps the fused RDNA4 prefill GEMM at nine waves", section "What the
 * fused GEMM actually spends registers on").
 *
 * Q4_K (the GGUF block; the pages name it but print no layout): 144 bytes hold
 * 256 consecutive weights of one row along the contraction dimension --
 * bytes 0-1 fp16 d, bytes 2-3 fp16 dmin, bytes 4-15 eight 6-bit scales sc_j
 * and eight 6-bit mins m_j packed as
 *     j < 4 : sc_j = S[j] & 63,  m_j = S[j+4] & 63
 *     j >= 4: sc_j = (S[j+4] & 15) | (S[j-4] >> 6) << 4,  m_j = (S[j+4] >> 4) | (S[j] >> 6) << 4
 * and bytes 16-143 the 4-bit quants: weight i sits in byte 16 + 32*(i/64) + i%32,
 * low nibble if i%64 < 32, else high nibble.  Weight i = d*sc_{i/32}*q_i - dmin*m_{i/32}.
 * A matrix [rows x cols] (cols % 256 == 0) is rows x (cols/256) blocks, row-major,
 * blocks running along cols.  W_gate and W_up are [inter x hidden]; W_down is
 * [hidden x inter].
 *
 * Activations: x and y are fp16, row-major [M x hidden].  Accumulation is fp32.
 *
 * fp16 range: the intermediate is stored in fp16 on chip and y in fp16 in
 * memory.  Both are divided by an exact power of two first:
 *     intermediate held as fp16(h * 2^-inter_shift),  y written as fp16(y * 2^-out_shift).
 * With real-model weights both shifts are 0; synthetic weights with a large
 * non-zero mean need positive shifts to stay below 65504.  Shifts are in [0, 30].
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers owned by the caller, 16-byte aligned.
 *     Nothing is allocated or freed inside; the workspace is caller-provided.
 *   - Every argument check runs on the host before any HIP call; a failed check
 *     returns a negative zinc_status and enqueues nothing.
 *   - On success the call only enqueues work on `stream` (a hipStream_t; NULL
 *     means the null stream) and returns ZINC_OK without synchronising the
 *     host.  Buffers must stay valid until the stream has passed the call.
 *   - A failed kernel launch returns ZINC_ERR_HIP.
 *   - M == 0 is a no-op returning ZINC_OK.
 *   - Calls hold no state between them (the optional timing hook at the end of
 *     this header is the one process-wide recorder, off by default and outside
 *     this statement); concurrent calls need distinct workspaces and outputs.
 *   - y must not alias x, the weights or the workspace.
 */
#ifndef ZINC_MLP_H
#define ZINC_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZINC_OK = 0,
  ZINC_ERR_NULL = -1,        /* a required pointer is NULL */
  ZINC_ERR_SHAPE = -2,       /* hidden or inter not a positive multiple of 256, or too large */
  ZINC_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  ZINC_ERR_WORKSPACE = -4,   /* workspace smaller than the matching *_workspace_size() */
  ZINC_ERR_ARG = -5,         /* M < 0, M above the entry point's limit, shift or top_k out of range */
  ZINC_ERR_HIP = -6,         /* a HIP launch or runtime call failed */
  ZINC_ERR_UNSUPPORTED = -7  /* a size the library does not handle */
} zinc_status;

/* Text of a status code (static storage; never NULL). */
const char* zinc_strerror(int status);

/* HIP's description of the error behind the most recent ZINC_ERR_HIP returned
 * on the calling thread, or "no HIP error" (static storage; never NULL). */
const char* zinc_hip_error_string(void);

/*
 * Q4_K block decoder: out[r*cols + c] = the fp32 weight (row r, column c) of the
 * Q4_K matrix `blocks` [rows x cols], cols % 256 == 0.  Every weight is the exact
 * value d*sc*q - dmin*m rounded once to nearest-even fp32 (all the products are
 * exact in fp32), so the result is bit-for-bit unique.
 * Definition: the Q4_K block named on "Fused SwiGLU MLP: ZINC RDNA4 Down-Projection
 * Bandwidth" (opening Q&A), layout above.
 * rows >= 0; rows * cols must fit in int32.
 */
int zinc_q4k_dequant_f32(const void* blocks, int32_t rows, int32_t cols, float* out, void* stream);

/*
 * The decoders of the two other block formats the experts' down projections
 * use ("Four bottlenecks, one CUDA backend", "Bottleneck 2": Q5_K for one MoE
 * family, Q5_1 for the other; layouts are the public GGUF blocks):
 *   Q5_K: 176-byte super-blocks of 256 weights: bytes 0-15 as Q4_K (d, dmin,
 *         6-bit scales and mins), bytes 16-47 the fifth bits (bit 2c+u of byte
 *         l for weight 64c + 32u + l), bytes 48-175 the low nibbles as Q4_K;
 *         w = d*sc*q - dmin*m with q in 0..31.  cols % 256 == 0.
 *   Q5_1: 24-byte blocks of 32 weights: fp16 d, fp16 m, a 32-bit word of fifth
 *         bits (bit i for weight i), 16 quant bytes (weight i < 16 the low
 *         nibble of byte i, weight 16 + i the high nibble); w = d*q + m.
 *         cols % 32 == 0.
 * Each weight is the exact value rounded once to fp32 (unique); out is
 * [rows x cols] fp32, 16-byte aligned, as blocks.  Errors as the Q4_K decoder.
 */
int zinc_q5k_dequant_f32(const void* blocks, int32_t rows, int32_t cols, float* out, void* stream);
int zinc_q5_1_dequant_f32(const void* blocks, int32_t rows, int32_t cols, float* out, void* stream);

/*
 * Batched prefill: y[M x hidden] = MLP(x[M x hidden]) for any M >= 0.
 * One fused kernel decodes the gate/up Q4_K blocks in registers into fp16 MFMA
 * operands (fp32 accumulation), applies SwiGLU in registers, stages the
 * tokens x intermediate strip in LDS and runs the down projection on it, so
 * the intermediate never reaches device memory ("Fused SwiGLU MLP: ZINC RDNA4
 * Down-Projection Bandwidth", sections "Why this fusion is harder than the
 * last one" and "What it is worth").  `workspace` holds the activation
 * rearranged into the MFMA operand order (written first, by a small kernel)
 * and the down-projection partial sums of the intermediate chunks, stored as
 * fp16 at the output scale and summed in fp32 by a reduce kernel.  The
 * workspace size is non-decreasing in M (here and for the _staged and _block
 * variants): a workspace sized for M serves every call with fewer tokens.
 * The kernel plan (unit shape and chunk count) is a function of (M, hidden,
 * inter) only.
 * Limits: hidden, inter multiples of 256, hidden <= 16384, inter <= 65536,
 * M <= 2^20 and (M + 1) * (hidden / 256) * 544 < 2^32 (else ZINC_ERR_ARG, and
 * the workspace size query returns 0).
 */
size_t zinc_mlp_q4k_prefill_workspace_size(int32_t M, int32_t hidden, int32_t inter);
int zinc_mlp_q4k_prefill(const void* w_gate, const void* w_up, const void* w_down,
                         int32_t hidden, int32_t inter,
                         const void* x_f16, void* y_f16, int32_t M,
                         int32_t inter_shift, int32_t out_shift,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The MLP block with its neighbours folded in: the pre-MLP RMS norm and the
 * post-MLP residual ("Four bottlenecks, one CUDA backend", "Bottleneck 3":
 * norm and residual steps fused into fewer launches, with the per-layer output
 * scale folded into the norm + residual step):
 *   r_t     = 1 / sqrt(mean_k x[t][k]^2 + norm_eps)           (fp32)
 *   xn[t]   = fp16(x[t] * r_t * norm_weight)                   (the MLP's input)
 *   y[t]    = fp16((x[t] + mlp_scale * MLP(xn[t])) * 2^-out_shift)
 * with MLP and the shifts as in zinc_mlp_q4k_prefill / _decode (inter_shift
 * scales the intermediate).  x is the residual stream; y may be x itself (an
 * in-place residual update).  norm_weight_f16: fp16 [hidden], 16-byte aligned.
 * norm_eps >= 0 and mlp_scale finite, else ZINC_ERR_ARG (with norm_eps == 0 an
 * all-zero row gives NaN).  The norm runs as one small kernel writing xn to the
 * workspace; the residual and the scale are applied where y is written (the
 * reduce kernel, or the decode down-projection kernel), so neither costs a
 * launch of its own.  Other arguments, limits and errors as the plain entry
 * points (_decode_block: 1 <= M <= 8), with their own workspace sizes.
 */
size_t zinc_mlp_q4k_prefill_block_workspace_size(int32_t M, int32_t hidden, int32_t inter);
int zinc_mlp_q4k_prefill_block(const void* w_gate, const void* w_up, const void* w_down,
                               int32_t hidden, int32_t inter,
                               const void* x_f16, const void* norm_weight_f16, float norm_eps,
                               float mlp_scale, void* y_f16, int32_t M,
                               int32_t inter_shift, int32_t out_shift,
                               void* workspace, size_t workspace_bytes, void* stream);
size_t zinc_mlp_q4k_decode_block_workspace_size(int32_t M, int32_t hidden, int32_t inter);
int zinc_mlp_q4k_decode_block(const void* w_gate, const void* w_up, const void* w_down,
                              int32_t hidden, int32_t inter,
                              const void* x_f16, const void* norm_weight_f16, float norm_eps,
                              float mlp_scale, void* y_f16, int32_t M,
                              int32_t inter_shift, int32_t out_shift,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The staged comparison baseline of the prefill -- measurement only, not a
 * product path.  The same y as zinc_mlp_q4k_prefill, computed with the
 * intermediate in device memory, as the unfused dataflow the fusion replaces
 * ("Fused SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth", "The MLP is two
 * trips up to a wider width" and "Counting the bytes"): the gate/up pass stores
 * fp16 G and U [M x inter], a SwiGLU kernel reads them and stores the fp16
 * intermediate, and the down pass reads it back -- six crossings of
 * M x inter x 2 bytes that the fused call keeps on chip.  The units, their
 * decode and the split-K reduction are the fused call's, so the difference
 * between the two calls is what the fusion saves.  G and U are rounded to fp16
 * unscaled (they must stay below 65504 in magnitude); the shifts apply as in
 * the fused call.  Arguments, limits and errors as zinc_mlp_q4k_prefill, with
 * its own workspace size.
 */
size_t zinc_mlp_q4k_prefill_staged_workspace_size(int32_t M, int32_t hidden, int32_t inter);
int zinc_mlp_q4k_prefill_staged(const void* w_gate, const void* w_up, const void* w_down,
                                int32_t hidden, int32_t inter,
                                const void* x_f16, void* y_f16, int32_t M,
                                int32_t inter_shift, int32_t out_shift,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode, 1 <= M <= 8 tokens: the same block as a pair of HBM-bound matvecs.
 * The first streams W_gate and W_up once, computing both projections from one
 * read of x and applying SwiGLU (the same-input gate/up pair fusion of "Four
 * bottlenecks, one CUDA backend", "Bottleneck 3"); the second streams W_down.
 * The per-token intermediate, fp16(h * 2^-inter_shift) [M x inter], lives in
 * `workspace` between the two kernels -- for decode it is small and consumed at
 * once ("Fused SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth", opening Q&A
 * "Does this affect decode?").  Both shifts apply as above.  M > 8 returns
 * ZINC_ERR_ARG.
 */
size_t zinc_mlp_q4k_decode_workspace_size(int32_t M, int32_t hidden, int32_t inter);
int zinc_mlp_q4k_decode(const void* w_gate, const void* w_up, const void* w_down,
                        int32_t hidden, int32_t inter,
                        const void* x_f16, void* y_f16, int32_t M,
                        int32_t inter_shift, int32_t out_shift,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The same call and result as
 * zinc_mlp_q4k_decode (the same kernels), with the intermediate held in a
 * device array the library owns instead of a caller workspace: one array per
 * GPU, zinc_mlp_q4k_decode_noalloc_max_bytes() bytes (512 KiB), kept until the
 * process ends.  Its address on each device is looked up on the first call
 * made with that device current.  M * inter * 2 bytes (rounded up to 256)
 * must fit it, else ZINC_ERR_WORKSPACE before any HIP call (e.g. M = 8 allows
 * inter <= 32768).  `stream` must belong to the current device, else
 * ZINC_ERR_ARG.  Every call on a GPU uses that GPU's one array: calls that
 * overlap in time on one GPU (different streams, or threads) race on it and
 * must be serialised by the caller.  Other arguments and errors as
 * zinc_mlp_q4k_decode; no hipMalloc, hipFree or other allocating call is made.
 */
size_t zinc_mlp_q4k_decode_noalloc_max_bytes(void);
int zinc_mlp_q4k_decode_noalloc(const void* w_gate, const void* w_up, const void* w_down,
                                int32_t hidden, int32_t inter,
                                const void* x_f16, void* y_f16, int32_t M,
                                int32_t inter_shift, int32_t out_shift, void* stream);

/*
 * Batched-expert MoE MLP: y[t] = sum_{s < top_k} p[t,s] * MLP_{ids[t,s]}(x[t]).
 * Expert ids (int32 [M x top_k]) and mixing weights (fp32 [M x top_k]) are read
 * on the GPU; the host never reads them back and launches a fixed number of
 * kernels whatever the routing: the batched-expert form of "Four bottlenecks,
 * one CUDA backend", "Bottleneck 2", where the device code looks the routing
 * up and addresses each chosen expert's weights without a host round trip.  w_gate / w_up hold n_experts [inter x hidden] Q4_K
 * matrices back to back, w_down n_experts [hidden x inter] matrices.
 * A slot whose id is outside [0, n_experts) contributes nothing; the kernel
 * then ORs 1 into *dev_error (a device int32, may be NULL) -- the flag is
 * sticky and the caller clears it.  Duplicate ids within a token each count.
 * 1 <= top_k <= n_experts <= 1024; M * top_k <= 2^24, (M * top_k + 1) * hidden * 2 < 2^31
 * and (M + 1) * (hidden / 256) * 544 < 2^32 (else ZINC_ERR_ARG, and the
 * workspace size query returns 0).
 */
size_t zinc_moe_q4k_experts_workspace_size(int32_t M, int32_t top_k, int32_t n_experts,
                                           int32_t hidden, int32_t inter);
int zinc_moe_q4k_experts(const void* w_gate, const void* w_up, const void* w_down,
                         int32_t n_experts, int32_t hidden, int32_t inter,
                         const void* x_f16, int32_t M,
                         const int32_t* expert_ids, const float* expert_weights, int32_t top_k,
                         void* y_f16, int32_t inter_shift, int32_t out_shift,
                         void* workspace, size_t workspace_bytes, int32_t* dev_error,
                         void* stream);

/*
 * The batched-expert call with W_down in another block format ("Four
 * bottlenecks, one CUDA backend", "Bottleneck 2": one MoE family's experts
 * project down in Q5_K, another's in Q5_1; gate and up stay Q4_K).
 * down_format: ZINC_DOWN_Q4_K (the same as zinc_moe_q4k_experts), ZINC_DOWN_Q5_K
 * (w_down holds n_experts [hidden x inter] matrices of 176-byte blocks) or
 * ZINC_DOWN_Q5_1 (24-byte blocks of 32 weights); the layouts are those of the
 * decoders above.  The fifth bits are OR'ed into the same fp16 operand
 * patterns, so the unit and its arithmetic are the Q4_K call's; the Q5_1 min
 * term (+m per 32 weights) is contracted against the strip's 32-row means as
 * the Q4_K one is.  Any other down_format -> ZINC_ERR_ARG.  Everything else
 * (arguments, limits, errors, workspace size) as zinc_moe_q4k_experts.
 */
enum { ZINC_DOWN_Q4_K = 0, ZINC_DOWN_Q5_K = 1, ZINC_DOWN_Q5_1 = 2 };
int zinc_moe_experts_fmt(const void* w_gate, const void* w_up, const void* w_down, int32_t down_format,
                         int32_t n_experts, int32_t hidden, int32_t inter,
                         const void* x_f16, int32_t M,
                         const int32_t* expert_ids, const float* expert_weights, int32_t top_k,
                         void* y_f16, int32_t inter_shift, int32_t out_shift,
                         void* workspace, size_t workspace_bytes, int32_t* dev_error,
                         void* stream);

/*
 * MoE router: for every token t, the top_k experts with the largest router
 * logits and their mixing weights, written to the device buffers that
 * zinc_moe_q4k_experts reads, so no host read-back separates the router from
 * the experts ("Four bottlenecks, one CUDA backend", "Bottleneck 2": every MoE
 * layer computes router logits and picks the top-k experts; "What's next, and
 * what it's worth" names the router's host synchronisation as the step left).
 *   logits          fp32 [M x n_experts] row-major, device
 *   expert_ids      int32 [M x top_k], device, written: slot s holds the expert
 *                   of the s-th largest logit; equal logits go to the lower
 *                   expert index first; a NaN logit ranks below every number
 *   expert_weights  fp32 [M x top_k], device, written: the softmax of the chosen
 *                   logits, exp(l_s - l_0) / sum_j exp(l_j - l_0) (one NaN among
 *                   them makes the token's weights NaN)
 * This is the reading taken of the pages' "top-k experts" plus mixing weights:
 * the softmax is over the k chosen logits (the full softmax renormalised over
 * the chosen experts, which is the same value).
 * Limits: 1 <= top_k <= min(64, n_experts), n_experts <= 1024, M >= 0,
 * M * top_k <= 2^24 (else ZINC_ERR_ARG); M == 0 then returns ZINC_OK without
 * reading the pointers (an empty buffer may be NULL); otherwise pointers must
 * be non-NULL (ZINC_ERR_NULL) and 4-byte aligned (ZINC_ERR_ALIGN).
 * One kernel, enqueued on `stream`; no workspace.
 */
int zinc_moe_route_topk(const float* logits, int32_t M, int32_t n_experts, int32_t top_k,
                        int32_t* expert_ids, float* expert_weights, void* stream);

/*
 * Kernel timing for benchmarks and profiles (off by default; not needed for
 * correct use).  After zinc_timing_enable(capacity), every prefill, decode and
 * MoE call records a HIP event pair on its stream immediately around its main
 * kernel -- the fused unit kernel for prefill and MoE; for decode, one pair
 * around the gate/up matvec and one around the down matvec -- for up to
 * `capacity` pairs.  The events are recorded without a system-scope fence
 * (hipEventDisableSystemFence), so they add no cache write-back of their own
 * to the work they bracket.  zinc_timing_collect() waits for the recorded events,
 * writes each pair's elapsed milliseconds to ms[0..*n_out) in launch order and
 * restarts the recording; zinc_timing_disable() stops it and destroys the
 * events.  Not meant to be used while other threads call the library.
 * Errors: capacity outside [1, 2^20] -> ZINC_ERR_ARG; event failures -> ZINC_ERR_HIP.
 */
int zinc_timing_enable(int32_t capacity);
int zinc_timing_collect(float* ms, int32_t capacity, int32_t* n_out);
void zinc_timing_disable(void);

#ifdef __cplusplus
}
#endif

#endif /* ZINC_MLP_H */
