#include "util_kernels.hpp"

namespace zinc {

namespace {

__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, size_t n4) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t st = (size_t)gridDim.x * 256;
  for (; i < n4; i += st) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// 64x64 tile transpose through LDS: reads along t, writes along n.
__global__ __launch_bounds__(256) void k_y32t_to_f16(const float* __restrict__ y32t, int Mpad,
                                                    _Float16* __restrict__ y, int H, int M, float scale) {
  __shared__ float tile[64][65];
  const int n0 = blockIdx.x * 64, t0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) tile[ty + 4 * i][tx] = y32t[(size_t)(n0 + ty + 4 * i) * Mpad + t0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + ty + 4 * i;
    if (t < M) y[(size_t)t * H + n0 + tx] = (_Float16)(tile[tx][ty + 4 * i] * scale);
  }
}

}  // namespace

void launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  const size_t n4 = n / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<float4*>(p), n4);
}

void launch_y32t_to_f16(const float* y32t, int Mpad, _Float16* y, int H, int M, float scale, hipStream_t stream) {
  hipLaunchKernelGGL(k_y32t_to_f16, dim3(H / 64, Mpad / 64), dim3(256), 0, stream, y32t, Mpad, y, H, M, scale);
}

}  // namespace zinc
