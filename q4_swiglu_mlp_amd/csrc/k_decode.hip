// Decode (1 <= M <= 8 tokens): the SwiGLU block as two HBM-bound Q4_K matvecs.
//
//   k_decode_mv<GATEUP=true>  streams W_gate and W_up once: both projections
//     share one read of x (the same-input gate/up pair fusion of "Four
//     bottlenecks, one CUDA backend", "Bottleneck 3"), SwiGLU is applied and the
//     per-token intermediate is written as fp16(h * 2^-inter_shift) to the
//     workspace (M x inter; small and consumed at once, as the decode Q&A of
//     "Fused SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth" says).
//   k_decode_mv<GATEUP=false> streams W_down against that intermediate and
//     writes y = fp16(acc * 2^(inter_shift - out_shift)).
//
// Work split: a 256-thread block owns NR = 8 rows; 32 threads per row.  Within
// a row, thread q handles part p = q % 8 of each block (16 quant bytes = 16 low
// + 16 high nibbles, i.e. half of sub-blocks 2c and 2c+1, c = p/2) for blocks
// b = q/8, q/8 + 4, ...; the 32 partial sums are reduced with cross-lane
// shuffles.  The activation is staged in LDS, K-chunk by K-chunk, as fp16 with
// the middle two elements of every group of four swapped, which matches the
// pair order the nibble unpack produces, plus per-16 sums used to remove the
// exact fp16 nibble offsets (1024 or 64) and the mins in fp32:
//   sum_k w_k x_k = s*(A - off*X16) - dm*X16  with A = sum (off + q_k) x_k.
#include "q4k_device.hpp"
#include "launch.hpp"

namespace zinc {

namespace {

constexpr int DTHREADS = 256;
constexpr int NR = 8;                    // rows per block
constexpr int TPR = DTHREADS / NR;       // threads per row (32)
constexpr int BPH = TPR / 8;             // block phases per row (4)
constexpr int KC = 2048;                 // K elements staged per chunk

__device__ __forceinline__ int swap_mid4(int k) {
  const int e = k & 3;
  return (k & ~3) | ((e == 1) ? 2 : (e == 2) ? 1 : e);
}

template <int MM, bool GATEUP>
__global__ __launch_bounds__(DTHREADS) void k_decode_mv(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                                                        int K, int N, const _Float16* __restrict__ xin, int M,
                                                        _Float16* __restrict__ out, float scale) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[MM * KC];
  __shared__ float x16[MM * (KC / 16)];

  const int tid = threadIdx.x;
  const int rloc = tid / TPR, q = tid % TPR;
  const int p = q & 7, bph = q >> 3;
  const int c = p >> 1;                      // 64-weight chunk of the block
  const int lhalf = (p & 1) * 16;            // first position within the chunk's 32
  const int row = blockIdx.x * NR + rloc;    // N % NR == 0 (N is a multiple of 256)
  const int nb = K / QK;

  float acc0[MM], acc1[MM];
#pragma unroll
  for (int t = 0; t < MM; ++t) acc0[t] = acc1[t] = 0.0f;

  const uint8_t* r0 = W0 + (size_t)row * nb * BLOCK_BYTES;
  const uint8_t* r1 = GATEUP ? W1 + (size_t)row * nb * BLOCK_BYTES : nullptr;

  for (int k0 = 0; k0 < K; k0 += KC) {
    const int kc = min(KC, K - k0);          // multiple of 256
    __syncthreads();
    // stage: MM x kc fp16, 8 per piece, plus sums of 16
    const int pieces = MM * (kc / 8);
    for (int ci = tid; ci < pieces; ci += DTHREADS) {
      const int t = ci / (kc / 8), a = ci % (kc / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < M) v = *reinterpret_cast<const uint4*>(xin + (size_t)t * K + k0 + 8 * a);
      const uint32_t lo0 = (v.x & 0xFFFFu) | (v.y << 16);
      const uint32_t lo1 = (v.x >> 16) | (v.y & 0xFFFF0000u);
      const uint32_t hi0 = (v.z & 0xFFFFu) | (v.w << 16);
      const uint32_t hi1 = (v.z >> 16) | (v.w & 0xFFFF0000u);
      *reinterpret_cast<uint4*>(xs + t * KC + 8 * a) = make_uint4(lo0, lo1, hi0, hi1);
      const half8 hv = __builtin_bit_cast(half8, v);
      float s8 = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s8 += (float)hv[e];
      // pieces 2i and 2i+1 of a row form one group of 16 (kc/8 is even)
      const float other = __shfl_xor(s8, 1, 64);
      if ((a & 1) == 0) x16[t * (KC / 16) + (a >> 1)] = s8 + other;
    }
    __syncthreads();

    for (int bl = bph; bl < kc / QK; bl += BPH) {
      const int b = k0 / QK + bl;
      const uint8_t* bp0 = r0 + (size_t)b * BLOCK_BYTES;
      const uint4 h0 = *reinterpret_cast<const uint4*>(bp0);
      const uint4 q0 = *reinterpret_cast<const uint4*>(bp0 + 16 + 32 * c + lhalf);
      uint4 h1 = make_uint4(0, 0, 0, 0), q1 = make_uint4(0, 0, 0, 0);
      if (GATEUP) {
        const uint8_t* bp1 = r1 + (size_t)b * BLOCK_BYTES;
        h1 = *reinterpret_cast<const uint4*>(bp1);
        q1 = *reinterpret_cast<const uint4*>(bp1 + 16 + 32 * c + lhalf);
      }
      const int kl = bl * QK + 64 * c + lhalf;      // local index of the low-nibble run
      float A0lo[MM], A0hi[MM], A1lo[MM], A1hi[MM];
#pragma unroll
      for (int t = 0; t < MM; ++t) A0lo[t] = A0hi[t] = A1lo[t] = A1hi[t] = 0.0f;
#pragma unroll
      for (int dwi = 0; dwi < 4; ++dwi) {
        const uint32_t Q0 = (dwi == 0) ? q0.x : (dwi == 1) ? q0.y : (dwi == 2) ? q0.z : q0.w;
        const uint32_t Q1 = (dwi == 0) ? q1.x : (dwi == 1) ? q1.y : (dwi == 2) ? q1.z : q1.w;
        const half2v a0 = bits_h2((Q0 & 0x000F000Fu) | 0x64006400u);
        const half2v a1 = bits_h2(((Q0 >> 8) & 0x000F000Fu) | 0x64006400u);
        const half2v a2 = bits_h2((Q0 & 0x00F000F0u) | 0x54005400u);
        const half2v a3 = bits_h2(((Q0 >> 8) & 0x00F000F0u) | 0x54005400u);
        half2v b0, b1, b2, b3;
        if (GATEUP) {
          b0 = bits_h2((Q1 & 0x000F000Fu) | 0x64006400u);
          b1 = bits_h2(((Q1 >> 8) & 0x000F000Fu) | 0x64006400u);
          b2 = bits_h2((Q1 & 0x00F000F0u) | 0x54005400u);
          b3 = bits_h2(((Q1 >> 8) & 0x00F000F0u) | 0x54005400u);
        }
#pragma unroll
        for (int t = 0; t < MM; ++t) {
          const uint2 xl = *reinterpret_cast<const uint2*>(xs + t * KC + kl + 4 * dwi);
          const uint2 xh = *reinterpret_cast<const uint2*>(xs + t * KC + kl + 32 + 4 * dwi);
          A0lo[t] = __builtin_amdgcn_fdot2(a0, bits_h2(xl.x), A0lo[t], false);
          A0lo[t] = __builtin_amdgcn_fdot2(a1, bits_h2(xl.y), A0lo[t], false);
          A0hi[t] = __builtin_amdgcn_fdot2(a2, bits_h2(xh.x), A0hi[t], false);
          A0hi[t] = __builtin_amdgcn_fdot2(a3, bits_h2(xh.y), A0hi[t], false);
          if (GATEUP) {
            A1lo[t] = __builtin_amdgcn_fdot2(b0, bits_h2(xl.x), A1lo[t], false);
            A1lo[t] = __builtin_amdgcn_fdot2(b1, bits_h2(xl.y), A1lo[t], false);
            A1hi[t] = __builtin_amdgcn_fdot2(b2, bits_h2(xh.x), A1hi[t], false);
            A1hi[t] = __builtin_amdgcn_fdot2(b3, bits_h2(xh.y), A1hi[t], false);
          }
        }
      }
      // fold: s*(A - off*X) - dm*X = s*A - (off*s + dm)*X, per sub-block
      {
        const float d = half_bits_to_float(h0.x & 0xFFFFu), dmin = half_bits_to_float(h0.x >> 16);
        const SixBit sb = unpack_sixbit(h0.y, h0.z, h0.w);
        const float slo = d * (float)sixbit_sc(sb, 2 * c), shi = d * (float)sixbit_sc(sb, 2 * c + 1);
        const float clo = 1024.0f * slo + dmin * (float)sixbit_m(sb, 2 * c);
        const float chi = 64.0f * shi + dmin * (float)sixbit_m(sb, 2 * c + 1);
        const int xi = (kl >> 4);
#pragma unroll
        for (int t = 0; t < MM; ++t) {
          const float Xlo = x16[t * (KC / 16) + xi], Xhi = x16[t * (KC / 16) + xi + 2];
          acc0[t] += slo * A0lo[t] - clo * Xlo + shi * A0hi[t] - chi * Xhi;
        }
      }
      if (GATEUP) {
        const float d = half_bits_to_float(h1.x & 0xFFFFu), dmin = half_bits_to_float(h1.x >> 16);
        const SixBit sb = unpack_sixbit(h1.y, h1.z, h1.w);
        const float slo = d * (float)sixbit_sc(sb, 2 * c), shi = d * (float)sixbit_sc(sb, 2 * c + 1);
        const float clo = 1024.0f * slo + dmin * (float)sixbit_m(sb, 2 * c);
        const float chi = 64.0f * shi + dmin * (float)sixbit_m(sb, 2 * c + 1);
        const int xi = (kl >> 4);
#pragma unroll
        for (int t = 0; t < MM; ++t) {
          const float Xlo = x16[t * (KC / 16) + xi], Xhi = x16[t * (KC / 16) + xi + 2];
          acc1[t] += slo * A1lo[t] - clo * Xlo + shi * A1hi[t] - chi * Xhi;
        }
      }
    }
  }

  // reduce over the 32 threads of the row (one half of the wave)
#pragma unroll
  for (int t = 0; t < MM; ++t) {
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) {
      acc0[t] += __shfl_xor(acc0[t], m, 64);
      if (GATEUP) acc1[t] += __shfl_xor(acc1[t], m, 64);
    }
  }
  if (q == 0) {
#pragma unroll
    for (int t = 0; t < MM; ++t) {
      if (t < M) {
        float v;
        if (GATEUP) v = silu_f32(acc0[t]) * acc1[t] * scale;
        else v = acc0[t] * scale;
        out[(size_t)t * N + row] = (_Float16)v;
      }
    }
  }
}

template <int MM>
hipError_t launch_decode_mm(const void* wg, const void* wu, const void* wd, int hidden, int inter, const void* x,
                            void* y, int M, int inter_shift, int out_shift, void* ws, hipStream_t stream) {
  _Float16* hbuf = static_cast<_Float16*>(ws);
  hipLaunchKernelGGL((k_decode_mv<MM, true>), dim3(inter / NR), dim3(DTHREADS), 0, stream,
                     static_cast<const uint8_t*>(wg), static_cast<const uint8_t*>(wu), hidden, inter,
                     static_cast<const _Float16*>(x), M, hbuf, ldexpf(1.0f, -inter_shift));
  hipLaunchKernelGGL((k_decode_mv<MM, false>), dim3(hidden / NR), dim3(DTHREADS), 0, stream,
                     static_cast<const uint8_t*>(wd), static_cast<const uint8_t*>(nullptr), inter, hidden, hbuf, M,
                     static_cast<_Float16*>(y), ldexpf(1.0f, inter_shift - out_shift));
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int M, int hidden, int inter) {
  (void)hidden;
  return ((size_t)(M > 0 ? M : 1) * inter * sizeof(_Float16) + 255) / 256 * 256;
}

hipError_t launch_decode(const void* wg, const void* wu, const void* wd, int hidden, int inter, const void* x, void* y,
                         int M, int inter_shift, int out_shift, void* ws, hipStream_t stream) {
  if (M <= 1) return launch_decode_mm<1>(wg, wu, wd, hidden, inter, x, y, M, inter_shift, out_shift, ws, stream);
  if (M <= 2) return launch_decode_mm<2>(wg, wu, wd, hidden, inter, x, y, M, inter_shift, out_shift, ws, stream);
  if (M <= 4) return launch_decode_mm<4>(wg, wu, wd, hidden, inter, x, y, M, inter_shift, out_shift, ws, stream);
  return launch_decode_mm<8>(wg, wu, wd, hidden, inter, x, y, M, inter_shift, out_shift, ws, stream);
}

}  // namespace zinc
