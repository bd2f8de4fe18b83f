// MoE router on the GPU: the top-k experts of each token and their mixing
// weights, from the router logits, written straight into the device buffers
// the batched-expert call reads.  Every MoE layer picks its experts from the
// router logits; choosing them on the GPU removes the last host read-back of a
// layer, which that page names as the remaining per-layer synchronisation
// ("Four bottlenecks, one CUDA backend", "Bottleneck 2" and "What's next, and
// what it's worth").
//
// Selection order: larger logit first; equal logits by lower expert index; a
// NaN logit ranks below every number (so it is chosen only when fewer than k
// logits are numbers).  Mixing weights: the softmax of the k chosen logits,
// exp(l_i - l_max) / sum_j exp(l_j - l_max) in fp32.
//
// One wave per token.  Lane l holds the logits l*PER .. l*PER + PER-1 as
// order-preserving 32-bit ranks, so a lower lane, and within a lane a lower
// slot, is a lower expert index.  A round takes each lane's best live rank
// (lowest slot among equals), the wave-wide maximum of those (DPP), and the
// lowest lane holding it (a ballot): that lane's best is the next expert, and
// the lane retires it.  Lane r keeps round r's pick, and the softmax runs
// across lanes 0..k-1.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace zinc {
namespace {

constexpr int kRouterTokensPerBlock = 4;   // one wave each

// Order-preserving image of a float in [2, 2^32): NaN -> 1, every number
// above it (-inf -> 0x007FFFFF); 0 marks a retired or absent entry.
__device__ __forceinline__ uint32_t rank_of(float v) {
  if (v != v) return 1u;
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float value_of(uint32_t r) {
  return __uint_as_float((r & 0x80000000u) ? (r & 0x7FFFFFFFu) : ~r);   // rank 1 -> a NaN pattern
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
  return o > v ? o : v;
}

// Maximum over the wave, valid in every lane: within quads, half-rows and rows
// of 16 lanes, then row 0's into row 1 and rows 0-1's into rows 2-3 (row
// broadcasts), which leaves the total in lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0xB1>(v);         // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E>(v);         // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141>(v);        // row_half_mirror
  v = dpp_max_step<0x140>(v);        // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15
  v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int PER>   // logits per lane: E <= 64 * PER
__global__ __launch_bounds__(64 * kRouterTokensPerBlock) void k_route_topk(const float* __restrict__ logits, int M,
                                                                             int E, int top_k,
                                                                             int32_t* __restrict__ ids,
                                                                             float* __restrict__ p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouterTokensPerBlock + (int)(threadIdx.x >> 6);
  if (t >= M) return;   // whole waves
  const float* row = logits + (size_t)t * E;
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane * PER + i;
    key[i] = (j < E) ? rank_of(row[j]) : 0u;
  }
  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < top_k; ++r) {
    uint32_t best = key[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < PER; ++i)
      if (key[i] > best) {
        best = key[i];
        bi = i;
      }
    const uint32_t top = wave_max_u32(best);   // a live key remains: top_k <= E
    const uint64_t holders = __ballot(best == top);
    const int wl = (int)__builtin_ctzll(holders);
    const int j = wl * PER + __builtin_amdgcn_readlane(bi, wl);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == bi) key[i] = 0u;
    }
    if (lane == r) {
      my_id = j;
      my_val = value_of(top);
    }
  }
  // softmax over the chosen logits; the first pick was the largest (or NaN, if
  // every logit is NaN, which makes every weight NaN as the definition does)
  const float lmax = __shfl(my_val, 0, 64);
  const float e = (lane < top_k) ? expf(my_val - lmax) : 0.0f;
  const float s = wave_sum(e);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    p[(size_t)t * top_k + lane] = e / s;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int M, int n_experts, int top_k, int32_t* ids, float* p,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((M + kRouterTokensPerBlock - 1) / kRouterTokensPerBlock));
  const dim3 block(64 * kRouterTokensPerBlock);
  const int per = (n_experts + 63) / 64;
  timing_begin(stream);
  if (per <= 1)
    hipLaunchKernelGGL(k_route_topk<1>, grid, block, 0, stream, logits, M, n_experts, top_k, ids, p);
  else if (per <= 2)
    hipLaunchKernelGGL(k_route_topk<2>, grid, block, 0, stream, logits, M, n_experts, top_k, ids, p);
  else if (per <= 4)
    hipLaunchKernelGGL(k_route_topk<4>, grid, block, 0, stream, logits, M, n_experts, top_k, ids, p);
  else if (per <= 8)
    hipLaunchKernelGGL(k_route_topk<8>, grid, block, 0, stream, logits, M, n_experts, top_k, ids, p);
  else
    hipLaunchKernelGGL(k_route_topk<16>, grid, block, 0, stream, logits, M, n_experts, top_k, ids, p);
  timing_end(stream);
  return hipGetLastError();
}

}  // namespace zinc
