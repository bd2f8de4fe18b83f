// Dense batched prefill: the fused Q4_K SwiGLU unit (fused_core.hpp) over
// (64-token tiles) x (128-row intermediate chunks), then a scaling epilogue.
#include "fused_core.hpp"
#include "launch.hpp"
#include "util_kernels.hpp"

namespace zinc {

namespace {

constexpr int TT_DENSE = 2;   // 64 tokens per unit
constexpr int RT_DENSE = 1;   // 128 intermediate rows per unit
using DenseCfg = FusedCfg<TT_DENSE, RT_DENSE>;

__global__ __launch_bounds__(FU_THREADS) void k_prefill_fused(const uint8_t* __restrict__ wg,
                                                              const uint8_t* __restrict__ wu,
                                                              const uint8_t* __restrict__ wd, int H, int I,
                                                              const _Float16* __restrict__ x, int M,
                                                              float* __restrict__ y32t, int Mpad, float inter_scale,
                                                              int n_tiles, int n_chunks) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[DenseCfg::MT * DenseCfg::XS];
  __shared__ __attribute__((aligned(16))) _Float16 hs[DenseCfg::MT * DenseCfg::HS];
  __shared__ int tok[DenseCfg::MT];
  __shared__ float wrow[DenseCfg::MT];

  // Units of the same intermediate chunk share block id mod 8, so they land on
  // the same XCD and its L2 serves that weight chunk to every token tile.
  const int bid = blockIdx.x;
  const int grp = bid / (8 * n_tiles), rem = bid % (8 * n_tiles);
  const int tile = rem >> 3;
  const int chunk = grp * 8 + (rem & 7);
  if (chunk >= n_chunks) return;

  if (threadIdx.x < DenseCfg::MT) {
    const int t = tile * DenseCfg::MT + threadIdx.x;
    tok[threadIdx.x] = (t < M) ? t : -1;
    wrow[threadIdx.x] = 1.0f;
  }
  __syncthreads();
  fused_unit<TT_DENSE, RT_DENSE>(wg, wu, wd, H, I, x, tok, wrow, chunk, y32t, Mpad, inter_scale, xs, hs);
}

int round_up(int a, int b) { return (a + b - 1) / b * b; }

}  // namespace

size_t prefill_workspace_bytes(int M, int hidden, int inter) {
  (void)inter;
  const int Mpad = round_up(M > 0 ? M : 1, 64);
  return (size_t)hidden * Mpad * sizeof(float);
}

hipError_t launch_prefill(const void* wg, const void* wu, const void* wd, int hidden, int inter, const void* x,
                          void* y, int M, int inter_shift, int out_shift, void* ws, hipStream_t stream) {
  const int Mpad = round_up(M, 64);
  float* y32t = static_cast<float*>(ws);
  launch_fill_zero(y32t, (size_t)hidden * Mpad, stream);
  const int n_tiles = (M + DenseCfg::MT - 1) / DenseCfg::MT;
  const int n_chunks = (inter + DenseCfg::IC - 1) / DenseCfg::IC;
  const int n_groups = (n_chunks + 7) / 8;
  const float inter_scale = ldexpf(1.0f, -inter_shift);
  hipLaunchKernelGGL(k_prefill_fused, dim3(n_groups * 8 * n_tiles), dim3(FU_THREADS), 0, stream,
                     static_cast<const uint8_t*>(wg), static_cast<const uint8_t*>(wu),
                     static_cast<const uint8_t*>(wd), hidden, inter, static_cast<const _Float16*>(x), M, y32t, Mpad,
                     inter_scale, n_tiles, n_chunks);
  launch_y32t_to_f16(y32t, Mpad, static_cast<_Float16*>(y), hidden, M, ldexpf(1.0f, inter_shift - out_shift), stream);
  return hipGetLastError();
}

}  // namespace zinc
