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

}  // namespace zinc
