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
// Work split.  A wave owns 16 rows; lane l works on row l/4 and 64-weight
// chunk c = l%4 of every block it visits (32 quant bytes: sub-blocks 2c in the
// low nibbles, 2c+1 in the high ones), so the four lanes of a row read the
// block's 128 quant bytes contiguously.  KSPLIT waves of a block share the same
// 16 rows and take every KSPLIT-th block (cross-wave sums through LDS), which
// gives the short-row down projection enough waves to keep HBM busy.  Blocks
// are fetched UNROLL at a time so several loads per lane are in flight.
// The activation is staged once per block of threads in LDS as fp16 with the
// middle two elements of every group of four swapped -- the pair order the
// nibble unpack produces -- plus fp32 sums of every 32-element sub-block, which
// remove the exact fp16 nibble offsets (1024, 64) and the mins:
//   sum_k w_k x_k = s*A - (off*s + dmin*m)*X32,  A = sum_k (off + q_k) x_k.
#include "q4k_device.hpp"
#include "launch.hpp"

namespace zinc {

namespace {

constexpr int DTHREADS = 256;
constexpr int UNROLL = 4;

// K elements staged per pass: the gate/up matvec stages 4096 (one pass at
// hidden 4096); the down matvec stages as much of the intermediate as about
// 88 KB of LDS holds.
constexpr int KC_GATEUP = 4096;
template <int MM>
struct DownKC {
  static constexpr int value = (MM <= 2) ? 16384 : (MM <= 4) ? 11264 : 5632;
};

struct BlockData {
  uint4 hdr, q0, q1;
};

__device__ __forceinline__ BlockData load_block(const uint8_t* bp, int c) {
  BlockData d;
  d.hdr = *reinterpret_cast<const uint4*>(bp);
  d.q0 = *reinterpret_cast<const uint4*>(bp + 16 + 32 * c);
  d.q1 = *reinterpret_cast<const uint4*>(bp + 32 + 32 * c);
  return d;
}

// Accumulate one block's contribution (this lane's chunk c) into acc[t].
template <int MM>
__device__ __forceinline__ void block_dot(const BlockData& bd, int c, const _Float16* __restrict__ xs,
                                          const float* __restrict__ x32, int KC, int kl, float* acc) {
  float Alo[MM], Ahi[MM];
#pragma unroll
  for (int t = 0; t < MM; ++t) Alo[t] = Ahi[t] = 0.0f;
#pragma unroll
  for (int dwi = 0; dwi < 8; ++dwi) {
    const uint4& qq = (dwi < 4) ? bd.q0 : bd.q1;
    const int k4 = dwi & 3;
    const uint32_t Q = (k4 == 0) ? qq.x : (k4 == 1) ? qq.y : (k4 == 2) ? qq.z : qq.w;
    const half2v a0 = bits_h2((Q & 0x000F000Fu) | 0x64006400u);
    const half2v a1 = bits_h2(((Q >> 8) & 0x000F000Fu) | 0x64006400u);
    const half2v a2 = bits_h2((Q & 0x00F000F0u) | 0x54005400u);
    const half2v a3 = bits_h2(((Q >> 8) & 0x00F000F0u) | 0x54005400u);
#pragma unroll
    for (int t = 0; t < MM; ++t) {
      const uint2 xl = *reinterpret_cast<const uint2*>(xs + t * KC + kl + 4 * dwi);
      const uint2 xh = *reinterpret_cast<const uint2*>(xs + t * KC + kl + 32 + 4 * dwi);
      Alo[t] = __builtin_amdgcn_fdot2(a0, bits_h2(xl.x), Alo[t], false);
      Alo[t] = __builtin_amdgcn_fdot2(a1, bits_h2(xl.y), Alo[t], false);
      Ahi[t] = __builtin_amdgcn_fdot2(a2, bits_h2(xh.x), Ahi[t], false);
      Ahi[t] = __builtin_amdgcn_fdot2(a3, bits_h2(xh.y), Ahi[t], false);
    }
  }
  const float d = half_bits_to_float(bd.hdr.x & 0xFFFFu), dmin = half_bits_to_float(bd.hdr.x >> 16);
  const SixBit sb = unpack_sixbit(bd.hdr.y, bd.hdr.z, bd.hdr.w);
  const float slo = d * (float)sixbit_sc(sb, 2 * c), shi = d * (float)sixbit_sc(sb, 2 * c + 1);
  const float clo = 1024.0f * slo + dmin * (float)sixbit_m(sb, 2 * c);
  const float chi = 64.0f * shi + dmin * (float)sixbit_m(sb, 2 * c + 1);
  const int xi = kl >> 5;
#pragma unroll
  for (int t = 0; t < MM; ++t)
    acc[t] += slo * Alo[t] - clo * x32[t * (KC / 32) + xi] + shi * Ahi[t] - chi * x32[t * (KC / 32) + xi + 1];
}

template <int MM, bool GATEUP, int KSPLIT, int KCMAX>
__global__ __launch_bounds__(DTHREADS) void k_decode_mv(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                                                        int K, int N, const _Float16* __restrict__ xin, int M,
                                                        _Float16* __restrict__ out, float scale) {
  constexpr int RG = 4 / KSPLIT;                 // 16-row groups per block of threads
  __shared__ __attribute__((aligned(16))) _Float16 xs[MM * KCMAX];
  __shared__ float x32[MM * (KCMAX / 32)];
  __shared__ float red[(KSPLIT > 1) ? (4 * 64 * MM * (GATEUP ? 2 : 1)) : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int rg = wave / KSPLIT, kph = wave % KSPLIT;
  const int r = lane >> 2, c = lane & 3;
  const int row = (blockIdx.x * RG + rg) * 16 + r;   // N % 256 == 0
  const int nb = K / QK;
  const int KC = min(K, KCMAX);

  float acc0[MM], acc1[MM];
#pragma unroll
  for (int t = 0; t < MM; ++t) acc0[t] = acc1[t] = 0.0f;
  const uint8_t* r0 = W0 + (size_t)row * nb * BLOCK_BYTES;
  const uint8_t* r1 = GATEUP ? W1 + (size_t)row * nb * BLOCK_BYTES : nullptr;

  for (int k0 = 0; k0 < K; k0 += KC) {
    const int kc = min(KC, K - k0);              // multiple of 256
    if (k0 > 0) __syncthreads();
    // stage x[0..M) x [k0, k0+kc): 8 elements per piece; 4 pieces form a 32-sum
    const int per_row = kc / 8;
    for (int ci = tid; ci < MM * per_row; ci += DTHREADS) {
      const int t = ci / per_row, a = ci % per_row;
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
      // per_row is a multiple of 32, so a group of 4 pieces never straddles
      // rows or the active-lane boundary of the last iteration
      s8 += __shfl_xor(s8, 1, 64);
      s8 += __shfl_xor(s8, 2, 64);
      if ((a & 3) == 0) x32[t * (KC / 32) + (a >> 2)] = s8;
    }
    __syncthreads();

    const int b_begin = k0 / QK, b_end = (k0 + kc) / QK;
    for (int b = b_begin + kph; b < b_end; b += UNROLL * KSPLIT) {
      BlockData d0[UNROLL], d1[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int bb = b + u * KSPLIT;
        if (bb < b_end) {
          d0[u] = load_block(r0 + (size_t)bb * BLOCK_BYTES, c);
          if (GATEUP) d1[u] = load_block(r1 + (size_t)bb * BLOCK_BYTES, c);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int bb = b + u * KSPLIT;
        if (bb < b_end) {
          const int kl = (bb - b_begin) * QK + 64 * c;
          block_dot<MM>(d0[u], c, xs, x32, KC, kl, acc0);
          if (GATEUP) block_dot<MM>(d1[u], c, xs, x32, KC, kl, acc1);
        }
      }
    }
  }

  // reduce over the 4 lanes of a row, then over the KSPLIT waves
#pragma unroll
  for (int t = 0; t < MM; ++t) {
    acc0[t] += __shfl_xor(acc0[t], 1, 64);
    acc0[t] += __shfl_xor(acc0[t], 2, 64);
    if (GATEUP) {
      acc1[t] += __shfl_xor(acc1[t], 1, 64);
      acc1[t] += __shfl_xor(acc1[t], 2, 64);
    }
  }
  if (KSPLIT > 1) {
    if (c == 0) {
#pragma unroll
      for (int t = 0; t < MM; ++t) {
        red[((wave * 16 + r) * MM + t) * (GATEUP ? 2 : 1)] = acc0[t];
        if (GATEUP) red[((wave * 16 + r) * MM + t) * 2 + 1] = acc1[t];
      }
    }
    __syncthreads();
    if (kph != 0) return;
    if (c == 0) {
#pragma unroll
      for (int t = 0; t < MM; ++t) {
        float s0 = 0.0f, s1 = 0.0f;
        for (int w = 0; w < KSPLIT; ++w) {
          s0 += red[(((rg * KSPLIT + w) * 16 + r) * MM + t) * (GATEUP ? 2 : 1)];
          if (GATEUP) s1 += red[(((rg * KSPLIT + w) * 16 + r) * MM + t) * 2 + 1];
        }
        acc0[t] = s0;
        acc1[t] = s1;
      }
    }
  }
  if (c == 0) {
#pragma unroll
    for (int t = 0; t < MM; ++t) {
      if (t < M) {
        const float v = GATEUP ? silu_f32(acc0[t]) * acc1[t] * scale : acc0[t] * scale;
        out[(size_t)t * N + row] = (_Float16)v;
      }
    }
  }
}

template <int MM>
hipError_t launch_decode_mm(const void* wg, const void* wu, const void* wd, int hidden, int inter, const void* x,
                            void* y, int M, int inter_shift, int out_shift, void* ws, hipStream_t stream) {
  _Float16* hbuf = static_cast<_Float16*>(ws);
  // gate/up: pairs of waves share 16 rows (32 rows per block of threads)
  timing_begin(stream);
  hipLaunchKernelGGL((k_decode_mv<MM, true, 2, KC_GATEUP>), dim3(inter / 32), dim3(DTHREADS), 0, stream,
                     static_cast<const uint8_t*>(wg), static_cast<const uint8_t*>(wu), hidden, inter,
                     static_cast<const _Float16*>(x), M, hbuf, ldexpf(1.0f, -inter_shift));
  timing_end(stream);
  // down: 4 waves share 16 rows, each taking every 4th block
  timing_begin(stream);
  hipLaunchKernelGGL((k_decode_mv<MM, false, 4, DownKC<MM>::value>), dim3(hidden / 16), dim3(DTHREADS), 0, stream,
                     static_cast<const uint8_t*>(wd), static_cast<const uint8_t*>(nullptr), inter, hidden, hbuf, M,
                     static_cast<_Float16*>(y), ldexpf(1.0f, inter_shift - out_shift));
  timing_end(stream);
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
