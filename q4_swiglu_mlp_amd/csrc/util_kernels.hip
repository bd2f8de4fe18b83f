#include "util_kernels.hpp"

namespace zinc {

namespace {

__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, size_t n4) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t st = (size_t)gridDim.x * 256;
  for (; i < n4; i += st) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

typedef _Float16 half8_u __attribute__((ext_vector_type(8)));

// One workgroup of 256 threads per token: each thread loads its (at most
// eight) 16-byte pieces of the row once, the squares are summed over the
// workgroup, and the same registers are scaled and stored.  K <= 16384.
constexpr int kNormPieces = 8;

__global__ __launch_bounds__(256) void k_rms_norm(const _Float16* __restrict__ x, const _Float16* __restrict__ gamma,
                                                  float eps, int K, _Float16* __restrict__ xn) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int n8 = K / 8;
  const _Float16* row = x + (size_t)t * K;
  half8_u v[kNormPieces];
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < kNormPieces; ++u) {
    const int i = threadIdx.x + 256 * u;
    v[u] = (i < n8) ? *reinterpret_cast<const half8_u*>(row + 8 * i) : half8_u{};
  }
#pragma unroll
  for (int u = 0; u < kNormPieces; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (float)v[u][e] * (float)v[u][e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)K + eps);
  _Float16* out = xn + (size_t)t * K;
#pragma unroll
  for (int u = 0; u < kNormPieces; ++u) {
    const int i = threadIdx.x + 256 * u;
    if (i < n8) {
      const half8_u gm = *reinterpret_cast<const half8_u*>(gamma + 8 * i);
      half8_u o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (_Float16)((float)v[u][e] * r * (float)gm[e]);
      *reinterpret_cast<half8_u*>(out + 8 * i) = o;
    }
  }
}

}  // namespace

void launch_rms_norm(const _Float16* x, const _Float16* gamma, float eps, int K, int M, _Float16* xn,
                     hipStream_t stream) {
  hipLaunchKernelGGL(k_rms_norm, dim3((unsigned)M), dim3(256), 0, stream, x, gamma, eps, K, xn);
}

void launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  const size_t n4 = n / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<float4*>(p), n4);
}

}  // namespace zinc
