// Standalone Q4_K -> fp32 decoder (bit-exact; see q4k_weight_f32).
#include "q4k_device.hpp"
#include "launch.hpp"

namespace zinc {

// One thread per (super-block, group of 8 consecutive weights).  Group g of a
// block holds weights 8g..8g+7: sub-block g/4, quant bytes 32*(g/8) + 8*(g%4)
// .. +7, low nibbles when (g/4) is even, high nibbles otherwise.
__global__ __launch_bounds__(256) void k_q4k_dequant_f32(const uint8_t* __restrict__ blocks, int64_t nblocks,
                                                         int nb_per_row, int cols, float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nblocks * 32) return;
  const int64_t blk = gid >> 5;
  const int g = (int)(gid & 31);
  const uint8_t* bp = blocks + blk * BLOCK_BYTES;
  const uint4 hdr = *reinterpret_cast<const uint4*>(bp);
  const float d = half_bits_to_float(hdr.x & 0xFFFFu);
  const float dmin = half_bits_to_float(hdr.x >> 16);
  const SixBit sb = unpack_sixbit(hdr.y, hdr.z, hdr.w);
  const int j = g >> 2;                         // sub-block
  const uint32_t sc = sixbit_sc(sb, j), m = sixbit_m(sb, j);
  const int byte0 = 32 * (g >> 3) + 8 * (g & 3);
  const uint2 qq = *reinterpret_cast<const uint2*>(bp + 16 + byte0);
  const int shift = (j & 1) ? 4 : 0;
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t word = (e < 4) ? qq.x : qq.y;
    const uint32_t q = (word >> (8 * (e & 3) + shift)) & 0xFu;
    w[e] = q4k_weight_f32(d, dmin, sc, m, q);
  }
  const int64_t row = blk / nb_per_row;
  const int64_t col = (blk % nb_per_row) * QK + 8 * g;
  float4* o = reinterpret_cast<float4*>(out + row * cols + col);
  o[0] = make_float4(w[0], w[1], w[2], w[3]);
  o[1] = make_float4(w[4], w[5], w[6], w[7]);
}

hipError_t launch_q4k_dequant_f32(const void* blocks, int rows, int cols, float* out, hipStream_t stream) {
  const int nb = cols / QK;
  const int64_t nblocks = (int64_t)rows * nb;
  const int64_t threads = nblocks * 32;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(k_q4k_dequant_f32, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(blocks), nblocks, nb, cols, out);
  return hipGetLastError();
}

// Q5_K -> fp32, the same thread layout over 176-byte blocks: group g holds
// weights 64c + 32u + l0 + e (c = g/8, u = (g/4)%2, l0 = 8(g%4), e < 8), low
// four bits from quant byte 48 + 32c + l0 + e (nibble u), the fifth bit from
// bit 2c + u of byte 16 + l0 + e.  d*sc*q is exact in fp32 (22 bits), so the
// fused multiply-add rounds once: the unique fp32 weight.
__global__ __launch_bounds__(256) void k_q5k_dequant_f32(const uint8_t* __restrict__ blocks, int64_t nblocks,
                                                         int nb_per_row, int cols, float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nblocks * 32) return;
  const int64_t blk = gid >> 5;
  const int g = (int)(gid & 31);
  const uint8_t* bp = blocks + blk * Q5K_BLOCK_BYTES;
  const uint4 hdr = *reinterpret_cast<const uint4*>(bp);
  const float d = half_bits_to_float(hdr.x & 0xFFFFu);
  const float dmin = half_bits_to_float(hdr.x >> 16);
  const SixBit sb = unpack_sixbit(hdr.y, hdr.z, hdr.w);
  const int c = g >> 3, u = (g >> 2) & 1, l0 = 8 * (g & 3);
  const int j = 2 * c + u;                      // sub-block
  const uint32_t sc = sixbit_sc(sb, j), m = sixbit_m(sb, j);
  const uint2 qq = *reinterpret_cast<const uint2*>(bp + 48 + 32 * c + l0);
  const uint2 hh = *reinterpret_cast<const uint2*>(bp + 16 + l0);
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t qw = (e < 4) ? qq.x : qq.y, hw = (e < 4) ? hh.x : hh.y;
    const uint32_t q = ((qw >> (8 * (e & 3) + 4 * u)) & 0xFu) | (((hw >> (8 * (e & 3) + j)) & 1u) << 4);
    w[e] = q4k_weight_f32(d, dmin, sc, m, q);
  }
  const int64_t row = blk / nb_per_row;
  const int64_t col = (blk % nb_per_row) * QK + 64 * c + 32 * u + l0;
  float4* o = reinterpret_cast<float4*>(out + row * cols + col);
  o[0] = make_float4(w[0], w[1], w[2], w[3]);
  o[1] = make_float4(w[4], w[5], w[6], w[7]);
}

// Q5_1 -> fp32: 24-byte blocks of 32 weights, one thread per group of eight:
// group g holds weights 8g + e, low nibbles of quant bytes 8 + 8g + e for
// g < 2, high nibbles of bytes 8 + 8(g-2) + e after; the fifth bit of weight i
// is bit i of the 32-bit word at byte 4.  d*q is exact, so fma(d, q, m) rounds
// once.
__global__ __launch_bounds__(256) void k_q5_1_dequant_f32(const uint8_t* __restrict__ blocks, int64_t nblocks,
                                                          int nb_per_row, int cols, float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nblocks * 4) return;
  const int64_t blk = gid >> 2;
  const int g = (int)(gid & 3);
  const uint8_t* bp = blocks + blk * Q5_1_BLOCK_BYTES;
  const uint2 hd = *reinterpret_cast<const uint2*>(bp);   // d, m | fifth bits
  const float d = half_bits_to_float(hd.x & 0xFFFFu);
  const float mm = half_bits_to_float(hd.x >> 16);
  const uint2 qq = *reinterpret_cast<const uint2*>(bp + 8 + 8 * (g & 1));
  const int shift = (g >= 2) ? 4 : 0;
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t qw = (e < 4) ? qq.x : qq.y;
    const uint32_t q = ((qw >> (8 * (e & 3) + shift)) & 0xFu) | (((hd.y >> (8 * g + e)) & 1u) << 4);
    w[e] = __builtin_fmaf(d, (float)q, mm);
  }
  const int64_t row = blk / nb_per_row;
  const int64_t col = (blk % nb_per_row) * 32 + 8 * g;
  float4* o = reinterpret_cast<float4*>(out + row * cols + col);
  o[0] = make_float4(w[0], w[1], w[2], w[3]);
  o[1] = make_float4(w[4], w[5], w[6], w[7]);
}

hipError_t launch_q5_dequant_f32(int fmt, const void* blocks, int rows, int cols, float* out, hipStream_t stream) {
  const int per = (fmt == 1) ? QK : 32;
  const int nb = cols / per;
  const int64_t nblocks = (int64_t)rows * nb;
  const int64_t threads = nblocks * ((fmt == 1) ? 32 : 4);
  const int64_t grid = (threads + 255) / 256;
  if (fmt == 1)
    hipLaunchKernelGGL(k_q5k_dequant_f32, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(blocks), nblocks, nb, cols, out);
  else
    hipLaunchKernelGGL(k_q5_1_dequant_f32, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(blocks), nblocks, nb, cols, out);
  return hipGetLastError();
}

}  // namespace zinc
