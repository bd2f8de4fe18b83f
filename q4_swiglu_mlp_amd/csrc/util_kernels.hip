#include "util_kernels.hpp"

namespace zinc {

namespace {

__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, size_t n4) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t st = (size_t)gridDim.x * 256;
  for (; i < n4; i += st) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

void launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  const size_t n4 = n / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<float4*>(p), n4);
}

}  // namespace zinc
