// Measured-peak microbenchmarks for the roofline denominators: what the chip
// delivers in practice for dense fp16 MFMA and for streaming HBM reads and
// copies.  Built as its own small library (libzinc_peaks.so), used only by the
// benchmark; not part of the MLP library.
//
//   zinc_peak_mfma_f16   every wave issues `iters` rounds of eight independent
//                        fp16 MFMAs (16x16x32 or 32x32x16) into accumulators it
//                        keeps in registers; nothing but the MFMAs is in the loop
//   zinc_peak_hbm_read   streams a buffer with 16-byte loads, four in flight per
//                        thread, grid-stride; one 4-byte result per thread
//   zinc_peak_hbm_copy   the same loads, each stored to a second buffer
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 768 threads (12 waves, three per SIMD): with a register budget of 168 the
// accumulators stay in plain VGPRs (a 256-thread bound lets the compiler move
// them through AGPRs inside the loop, which halves the rate)
template <int SHAPE>
__global__ __launch_bounds__(768) void k_mfma_peak(int iters, float* __restrict__ out) {
  const int tid = threadIdx.x;
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (float)((tid + e) & 7));
    b[e] = (_Float16)(0.002f * (float)((tid * 3 + e) & 7));
  }
  float s = 0.0f;
  if constexpr (SHAPE == 16) {
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][3];
  } else {
    f32x16 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[k][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) s += acc[k][0] + acc[k][15];
  }
  out[(size_t)blockIdx.x * blockDim.x + tid] = s;
}

__global__ __launch_bounds__(256) void k_hbm_read(const uint4* __restrict__ src, size_t n16, uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    acc ^= (v0.x ^ v0.y ^ v0.z ^ v0.w) + (v1.x ^ v1.y ^ v1.z ^ v1.w) + (v2.x ^ v2.y ^ v2.z ^ v2.w) +
           (v3.x ^ v3.y ^ v3.z ^ v3.w);
  }
  for (; i < n16; i += stride) acc ^= src[i].x ^ src[i].w;
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_hbm_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    dst[i] = v0;
    dst[i + stride] = v1;
    dst[i + 2 * stride] = v2;
    dst[i + 3 * stride] = v3;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// blocks x 768 threads; `out` holds blocks * 768 floats.  Returns the flops
// the launch performs (0 on a launch error or an unknown shape).
double zinc_peak_mfma_f16(int shape, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape == 16)
    hipLaunchKernelGGL(k_mfma_peak<16>, dim3(blocks), dim3(768), 0, s, iters, out);
  else if (shape == 32)
    hipLaunchKernelGGL(k_mfma_peak<32>, dim3(blocks), dim3(768), 0, s, iters, out);
  else
    return 0.0;
  if (hipGetLastError() != hipSuccess) return 0.0;
  // 16x16x32: 2*16*16*32 = 16384 flops per MFMA; 32x32x16: 2*32*32*16 = 32768
  const double per_mfma = (shape == 16) ? 16384.0 : 32768.0;
  return (double)blocks * 12 * (double)iters * 8 * per_mfma;
}

// Reads `bytes` (a multiple of 16) from src; `out` holds blocks * 256 uint32.
int zinc_peak_hbm_read(const void* src, size_t bytes, int blocks, uint32_t* out, void* stream) {
  if (!src || !out || bytes % 16 || blocks < 1) return -1;
  hipLaunchKernelGGL(k_hbm_read, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Copies `bytes` (a multiple of 16) from src to dst.
int zinc_peak_hbm_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks < 1) return -1;
  hipLaunchKernelGGL(k_hbm_copy, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
