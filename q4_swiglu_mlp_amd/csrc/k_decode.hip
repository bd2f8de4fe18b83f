// Decode of one token (M = 1 and inter <= 16384; larger M or a longer
// down-projection contraction use the MFMA kernels of k_decode_mfma.hip): the
// SwiGLU block as two HBM-bound Q4_K passes.
//
//   k_decode_rows<GATEUP=true>  streams W_gate and W_up once: both projections
//     share one staging of x (the same-input gate/up pair fusion of "Four
//     bottlenecks, one CUDA backend", "Bottleneck 3"), SwiGLU is applied and the
//     per-token intermediate is written as fp16(h * 2^-inter_shift), row-major
//     [M x inter], to the workspace (small and consumed at once, as the decode
//     Q&A of "Fused SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth" says).
//   k_decode_rows<GATEUP=false> streams W_down against that intermediate and
//     writes y = fp16(acc * 2^(inter_shift - out_shift)).
//
// Shape.  Weight rows are independent dot products, so each wave owns whole
// rows and walks them grid-stride (at any moment the grid reads one contiguous
// window of the matrix): no tiles, no barriers inside the loop, no cross-wave
// sums.  The workgroups are persistent (a fixed number per CU, see DrCfg) and
// stage the contraction vector once in LDS, under the latency of their first
// rows' loads; each wave keeps one or more rows in flight (a template depth),
// computing one while the next one's loads are outstanding.  A lane takes the
// same chunks of every row, so for one token and up to three chunks per lane
// it copies its activation slices from LDS into registers once, and the loop
// reads only weights from memory.
//
// Lanes.  A row's super-blocks split into 64-weight chunks; lane l takes chunks
// q = l, l+64, ... of the row, i.e. the block's 16-byte header and its 32 quant
// bytes (sub-block 2c in the low nibbles, 2c+1 in the high ones, c = q%4), so
// four consecutive lanes read a block's 128 quant bytes contiguously.
//
// Arithmetic per chunk and token: A = sum (1024+q) x over the low nibbles and
// sum (64+q) x over the high ones, both exact fp16 operands (the nibble OR'ed
// into an fp16 exponent pattern) fed to v_dot2_f32_f16 with fp32 accumulation;
// then  w.x = s*A - (off*s + dmin*m) * X  per sub-block, with X the staged
// fp32 sub-block sum of the activation.  The activation sits in LDS with the
// middle two elements of every group of four swapped -- the pair order the
// nibble unpack produces.
#include "fused_core.hpp"
#include "launch.hpp"
#include "util_kernels.hpp"

#include <algorithm>
#include <atomic>

namespace zinc {

namespace {

// waves per workgroup
template <int W>
struct DrShape {
  static constexpr int WAVES = W;
  static constexpr int THREADS = 64 * WAVES;
};
constexpr int DR_KMAX = 16384;               // longest contraction (the library's hidden limit)
constexpr int DR_KQ_MAX = DR_KMAX / 64 / 64; // chunk slots per lane (4)

// Cross-lane sums on the VALU (DPP).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}

// Sum over the 64 lanes; the total lands in lane 63.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f<0xB1>(v);          // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);          // quad_perm [2,3,0,1]
  v += dpp_f<0x114>(v);         // row_shr:4
  v += dpp_f<0x118>(v);         // row_shr:8
  v += dpp_f<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
  return v;
}

struct Chunk {
  uint4 hdr, q0, q1;   // block header; quant bytes [32c, 32c+16) and [32c+16, 32c+32)
};

// One chunk's contribution for MM tokens.  xs: staged activation (pair order)
// of token 0 at this chunk's 64 weights, token stride TS halves; X: the fp32
// sums of sub-blocks 2c and 2c+1 per token.
template <int MM>
__device__ __forceinline__ void chunk_dot(const Chunk& ch, int c, const _Float16* xs, int TS, const float* X2,
                                          int X2S, const NibbleK& nk, float* acc) {
  float alo[MM], ahi[MM];
#pragma unroll
  for (int t = 0; t < MM; ++t) alo[t] = ahi[t] = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 qq = h ? ch.q1 : ch.q0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t Q = (k == 0) ? qq.x : (k == 1) ? qq.y : (k == 2) ? qq.z : qq.w;
      const uint32_t Q8 = Q >> 8;
      const half2v a0 = bits_h2((Q & nk.lo_mask) | nk.lo_magic);    // 1024 + q, bytes 0, 2 (low nibbles)
      const half2v a1 = bits_h2((Q8 & nk.lo_mask) | nk.lo_magic);   // bytes 1, 3
      const half2v a2 = bits_h2((Q & nk.hi_mask) | nk.hi_magic);    // 64 + q (high nibbles)
      const half2v a3 = bits_h2((Q8 & nk.hi_mask) | nk.hi_magic);
      const int e = 16 * h + 4 * k;   // first weight of this dword within the chunk's low half
#pragma unroll
      for (int t = 0; t < MM; ++t) {
        const uint2 xl = *reinterpret_cast<const uint2*>(xs + t * TS + e);        // x[e], x[e+2], x[e+1], x[e+3]
        const uint2 xh = *reinterpret_cast<const uint2*>(xs + t * TS + 32 + e);
        alo[t] = __builtin_amdgcn_fdot2(a0, bits_h2(xl.x), alo[t], false);
        alo[t] = __builtin_amdgcn_fdot2(a1, bits_h2(xl.y), alo[t], false);
        ahi[t] = __builtin_amdgcn_fdot2(a2, bits_h2(xh.x), ahi[t], false);
        ahi[t] = __builtin_amdgcn_fdot2(a3, bits_h2(xh.y), ahi[t], false);
      }
    }
  }
  const float d = half_bits_to_float(ch.hdr.x & 0xFFFFu), dmin = half_bits_to_float(ch.hdr.x >> 16);
  const SixBit sb = unpack_sixbit(ch.hdr.y, ch.hdr.z, ch.hdr.w);
  const float slo = d * (float)sixbit_sc(sb, 2 * c), shi = d * (float)sixbit_sc(sb, 2 * c + 1);
  const float clo = 1024.0f * slo + dmin * (float)sixbit_m(sb, 2 * c);
  const float chi = 64.0f * shi + dmin * (float)sixbit_m(sb, 2 * c + 1);
#pragma unroll
  for (int t = 0; t < MM; ++t)
    acc[t] += slo * alo[t] - clo * X2[t * X2S] + shi * ahi[t] - chi * X2[t * X2S + 1];
}

// One token's chunk contribution as chunk_dot<1>, with the chunk's 64
// activations in registers (pair order, eight halves per uint4) and the fp32
// sums of its two sub-blocks.
__device__ __forceinline__ float chunk_dot_reg(const Chunk& ch, int c, const uint4 (&xr)[8], float xlo, float xhi,
                                               const NibbleK& nk) {
  float alo = 0.0f, ahi = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 qq = h ? ch.q1 : ch.q0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t Q = (k == 0) ? qq.x : (k == 1) ? qq.y : (k == 2) ? qq.z : qq.w;
      const uint32_t Q8 = Q >> 8;
      const int e = 16 * h + 4 * k;
      const uint4 vl = xr[e >> 3], vh = xr[(32 + e) >> 3];
      const uint32_t l0 = (e & 4) ? vl.z : vl.x, l1 = (e & 4) ? vl.w : vl.y;
      const uint32_t h0 = (e & 4) ? vh.z : vh.x, h1 = (e & 4) ? vh.w : vh.y;
      alo = __builtin_amdgcn_fdot2(bits_h2((Q & nk.lo_mask) | nk.lo_magic), bits_h2(l0), alo, false);
      alo = __builtin_amdgcn_fdot2(bits_h2((Q8 & nk.lo_mask) | nk.lo_magic), bits_h2(l1), alo, false);
      ahi = __builtin_amdgcn_fdot2(bits_h2((Q & nk.hi_mask) | nk.hi_magic), bits_h2(h0), ahi, false);
      ahi = __builtin_amdgcn_fdot2(bits_h2((Q8 & nk.hi_mask) | nk.hi_magic), bits_h2(h1), ahi, false);
    }
  }
  const float d = half_bits_to_float(ch.hdr.x & 0xFFFFu), dmin = half_bits_to_float(ch.hdr.x >> 16);
  const SixBit sb = unpack_sixbit(ch.hdr.y, ch.hdr.z, ch.hdr.w);
  const float slo = d * (float)sixbit_sc(sb, 2 * c), shi = d * (float)sixbit_sc(sb, 2 * c + 1);
  const float clo = 1024.0f * slo + dmin * (float)sixbit_m(sb, 2 * c);
  const float chi = 64.0f * shi + dmin * (float)sixbit_m(sb, 2 * c + 1);
  return slo * alo - clo * xlo + shi * ahi - chi * xhi;
}

template <int MM, bool GATEUP, int KQ, int DEPTH, int NW>
__global__ __launch_bounds__(DrShape<NW>::THREADS) void k_decode_rows(const uint8_t* __restrict__ W0,
                                                            const uint8_t* __restrict__ W1, int K, int N,
                                                            const _Float16* __restrict__ xin, int M,
                                                            _Float16* out, float scale, const _Float16* res,
                                                            float res_scale, const _Float16* gamma, float eps) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int DR_WAVES = DrShape<NW>::WAVES, DR_THREADS = DrShape<NW>::THREADS;
  extern __shared__ __attribute__((aligned(16))) unsigned char dr_smem[];
  const int nb = K / QK;
  const int Q = 4 * nb;                   // chunks per row
  const int TS = K + 8;                   // staged token stride (halves)
  _Float16* xs = reinterpret_cast<_Float16*>(dr_smem);
  float* X2 = reinterpret_cast<float*>(dr_smem + (size_t)MM * TS * 2);   // [MM][2*Q] sub-block sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const NibbleK nk = nibble_consts();

  const size_t row_bytes = (size_t)nb * BLOCK_BYTES;
  const int nwaves = gridDim.x * DR_WAVES;
  const int w0 = blockIdx.x * DR_WAVES + wave;
  // this lane's chunks: q = lane + 64k; byte offsets within a row
  int cq[KQ];
  size_t boff[KQ], qoff[KQ];
  bool has[KQ];
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const int q = lane + 64 * k;
    has[k] = q < Q;
    const int qc = has[k] ? q : 0;
    cq[k] = qc & 3;
    boff[k] = (size_t)(qc >> 2) * BLOCK_BYTES;
    qoff[k] = boff[k] + 16 + 32 * (qc & 3);
  }
  // one token and at most three chunks per lane: the lane's activation
  // slices (the same for every row it takes) are read from LDS into registers
  // once, after staging
  constexpr bool XREG = (MM == 1 && KQ <= 3);
  uint4 xr[KQ][8];
  float xr2[KQ][2];
  using Buf = Chunk[NMAT][KQ];
  // past the last row: re-read row fb (the wave's current row, cache-hot), or
  // row 0 if that is past the end too (never used either way)
  auto load_row = [&](int j, Buf& buf, int fb = 0) __attribute__((always_inline)) {
    const int jj = j < N ? j : (fb < N ? fb : 0);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const uint8_t* row = (m ? W1 : W0) + (size_t)jj * row_bytes;
#pragma unroll
      for (int k = 0; k < KQ; ++k) {
        buf[m][k].hdr = *reinterpret_cast<const uint4*>(row + boff[k]);
        buf[m][k].q0 = *reinterpret_cast<const uint4*>(row + qoff[k]);
        buf[m][k].q1 = *reinterpret_cast<const uint4*>(row + qoff[k] + 16);
      }
    }
  };
  auto compute_row = [&](int j, const Buf& buf) __attribute__((always_inline)) {
    float acc[NMAT][MM];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < MM; ++t) acc[m][t] = 0.0f;
#pragma unroll
    for (int k = 0; k < KQ; ++k) {
      if (!has[k]) continue;
      if constexpr (XREG) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m][0] += chunk_dot_reg(buf[m][k], cq[k], xr[k], xr2[k][0], xr2[k][1], nk);
      } else {
        const int q = lane + 64 * k;
        const _Float16* xq = xs + 64 * q;        // chunk q covers weights [64q, 64q+64)
        const float* xq2 = X2 + 2 * q;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) chunk_dot<MM>(buf[m][k], cq[k], xq, TS, xq2, 2 * Q, nk, acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < MM; ++t) acc[m][t] = wave_sum_to_lane63(acc[m][t]);
    if (lane == 63) {
#pragma unroll
      for (int t = 0; t < MM; ++t) {
        if (t < M) {
          float v = GATEUP ? silu_f32(acc[0][t]) * acc[NMAT - 1][t] * scale : acc[0][t] * scale;
          // the residual (down pass only; it may be out itself: read, then written, here)
          if (!GATEUP && res) v += (float)res[(size_t)t * N + j] * res_scale;
          out[(size_t)t * N + j] = (_Float16)v;
        }
      }
    }
  };

  // Order of the memory traffic (loads complete in issue order): the
  // activation pieces first, then the first two rows' weights, then the
  // staging arithmetic, which waits for the activation only.
  constexpr int NXG = (MM * (DR_KMAX / 8) + DR_THREADS - 1) / DR_THREADS;   // 16-byte groups per thread (bound)
  const int ngroups = MM * (K / 8);
  uint4 xv[NXG];
#pragma unroll
  for (int u = 0; u < NXG; ++u) {
    const int g = tid + u * DR_THREADS;
    const int t = g / (K / 8), a = g % (K / 8);
    xv[u] = make_uint4(0, 0, 0, 0);
    if (g < ngroups && t < M) xv[u] = *reinterpret_cast<const uint4*>(xin + (size_t)t * K + 8 * a);
  }
  Buf bufs[DEPTH];
  int j = w0;
  load_row(j, bufs[0]);
  // the pre-MLP RMS norm (gate/up pass of one token, gamma non-null): every
  // workgroup holds the whole activation, so it sums the squares itself and
  // scales its pieces before they are staged
  if (MM == 1 && gamma) {
    __shared__ float part[DR_WAVES];
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < NXG; ++u) {
      const half8 hv = __builtin_bit_cast(half8, xv[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (float)hv[e] * (float)hv[e];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if (lane == 0) part[wave] = ss;
    lds_barrier();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < DR_WAVES; ++w) tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)K + eps);
#pragma unroll
    for (int u = 0; u < NXG; ++u) {
      const int g = tid + u * DR_THREADS;
      if (g < ngroups) {
        const half8 hv = __builtin_bit_cast(half8, xv[u]);
        const half8 gm = *reinterpret_cast<const half8*>(gamma + 8 * g);
        half8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (_Float16)((float)hv[e] * r * (float)gm[e]);
        xv[u] = __builtin_bit_cast(uint4, o);
      }
    }
  }
  // stage x: groups of four with the middle two swapped; fp32 sums of every 32
  // elements (four consecutive groups = four consecutive lanes of a quad)
#pragma unroll
  for (int u = 0; u < NXG; ++u) {
    const int g = tid + u * DR_THREADS;
    const int t = g / (K / 8), a = g % (K / 8);
    const uint4 v = xv[u];
    if (g < ngroups)
      *reinterpret_cast<uint4*>(xs + t * TS + 8 * a) =
          make_uint4((v.x & 0xFFFFu) | (v.y << 16), (v.x >> 16) | (v.y & 0xFFFF0000u),
                     (v.z & 0xFFFFu) | (v.w << 16), (v.z >> 16) | (v.w & 0xFFFF0000u));
    const half8 hv = __builtin_bit_cast(half8, v);
    float s8 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s8 += (float)hv[e];
    s8 += dpp_f<0xB1>(s8);
    s8 += dpp_f<0x4E>(s8);
    if (g < ngroups && (a & 3) == 0) X2[t * 2 * Q + (a >> 2)] = s8;
  }
  lds_barrier();
  if constexpr (XREG) {
#pragma unroll
    for (int k = 0; k < KQ; ++k) {
      const int q = has[k] ? lane + 64 * k : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) xr[k][i] = *reinterpret_cast<const uint4*>(xs + 64 * q + 8 * i);
      xr2[k][0] = X2[2 * q];
      xr2[k][1] = X2[2 * q + 1];
    }
  }

  if constexpr (DEPTH > 1) {
    // DEPTH rows in flight per wave: a buffer is refilled with the row DEPTH
    // strides ahead as soon as it has been consumed, so the arithmetic of one
    // row runs under the loads of the next ones (the ring is unrolled, so
    // every buffer stays in registers)
#pragma unroll
    for (int d = 1; d < DEPTH; ++d) load_row(j + d * nwaves, bufs[d], j);
    for (; j < N; j += DEPTH * nwaves) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int jd = j + d * nwaves;
        if (jd >= N) break;
        compute_row(jd, bufs[d]);
        load_row(jd + DEPTH * nwaves, bufs[d], jd);
      }
    }
  } else {
    for (; j < N; j += nwaves) {
      if (j != w0) load_row(j, bufs[0]);
      compute_row(j, bufs[0]);
    }
  }
}

// Per-device CU count, looked up once per device (atomics: calls may come from
// several host threads).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::atomic<int>& c = cache[dev & 63];
  int n = c.load(std::memory_order_relaxed);
  if (n == 0) {
    n = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    c.store(n, std::memory_order_relaxed);
  }
  return n;
}

// Raises a kernel's dynamic-LDS limit to at least `smem` bytes; `set` holds the
// largest limit set so far for that kernel (shared by host threads).
hipError_t raise_lds_limit(const void* kernel, size_t smem, std::atomic<size_t>& set) {
  if (smem <= set.load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  size_t cur = set.load(std::memory_order_relaxed);
  while (cur < smem && !set.compare_exchange_weak(cur, smem, std::memory_order_relaxed)) {
  }
  return hipSuccess;
}

// Persistent grid: as many workgroups as are resident at once (occupancy of
// this instantiation at this LDS size), so no workgroup waits for another to end.
// Launch shape of the row kernels: rows in flight per wave, waves per
// workgroup, workgroups per CU.  Measured on the 4096/11008 layer sweep (graph
// replay) with the activation slices in registers: one row in flight on three
// four-wave workgroups per CU for the gate/up pass (about 7 rows per wave),
// two rows on one eight-wave workgroup per CU for the down pass (2 rows per
// wave): 20.8-20.9 us per layer against 22.1-22.3 for two rows on two
// four-wave workgroups (gate/up) and one (down); 3 or 4 rows in flight were
// slower for either pass.
template <int MM, bool GATEUP, int KQ, int DEPTH, int NW>
hipError_t launch_rows_cfg(const void* W0, const void* W1, int K, int N, const _Float16* x, int M, _Float16* out,
                           float scale, const _Float16* res, float res_scale, const _Float16* gamma, float eps,
                           int wg_per_cu, hipStream_t stream) {
  const size_t smem = (size_t)MM * (K + 8) * 2 + (size_t)MM * 2 * (4 * (K / QK)) * 4;
  static std::atomic<size_t> attr_set{0};   // largest dynamic LDS size allowed so far
  hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&k_decode_rows<MM, GATEUP, KQ, DEPTH, NW>), smem,
                                 attr_set);
  if (e != hipSuccess) return e;
  // occupancy at the last LDS size asked for, cached as (smem << 8) | occupancy
  static std::atomic<uint64_t> occ_key{0};
  uint64_t key = occ_key.load(std::memory_order_relaxed);
  int occ = (int)(key & 0xFFu);
  if (occ == 0 || (key >> 8) != (uint64_t)smem) {
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_rows<MM, GATEUP, KQ, DEPTH, NW>,
                                                     DrShape<NW>::THREADS, smem);
    if (e != hipSuccess) return e;
    occ = per_cu < 1 ? 1 : (per_cu > 255 ? 255 : per_cu);
    occ_key.store(((uint64_t)smem << 8) | (uint64_t)occ, std::memory_order_relaxed);
  }
  const int per_cu = (wg_per_cu > 0 && wg_per_cu < occ) ? wg_per_cu : occ;
  const int grid = std::max(1, std::min(cu_count() * per_cu, (N + NW - 1) / NW));
  hipLaunchKernelGGL((k_decode_rows<MM, GATEUP, KQ, DEPTH, NW>), dim3(grid), dim3(DrShape<NW>::THREADS), smem, stream,
                     static_cast<const uint8_t*>(W0), static_cast<const uint8_t*>(W1), K, N, x, M, out, scale, res,
                     res_scale, gamma, eps);
  return hipGetLastError();
}

template <int MM, bool GATEUP, int KQ>
hipError_t launch_rows(const void* W0, const void* W1, int K, int N, const _Float16* x, int M, _Float16* out,
                       float scale, const _Float16* res, float res_scale, const _Float16* gamma, float eps,
                       hipStream_t stream) {
  if constexpr (GATEUP)
    return launch_rows_cfg<MM, GATEUP, KQ, 1, 4>(W0, W1, K, N, x, M, out, scale, res, res_scale, gamma, eps, 3, stream);
  else
    return launch_rows_cfg<MM, GATEUP, KQ, 2, 8>(W0, W1, K, N, x, M, out, scale, res, res_scale, gamma, eps, 1, stream);
}

template <int MM, bool GATEUP>
hipError_t launch_rows_k(const void* W0, const void* W1, int K, int N, const _Float16* x, int M, _Float16* out,
                         float scale, const _Float16* res, float res_scale, const _Float16* gamma, float eps,
                         hipStream_t stream) {
  const int Q = 4 * (K / QK);
  if (Q <= 64) return launch_rows<MM, GATEUP, 1>(W0, W1, K, N, x, M, out, scale, res, res_scale, gamma, eps, stream);
  if (Q <= 128) return launch_rows<MM, GATEUP, 2>(W0, W1, K, N, x, M, out, scale, res, res_scale, gamma, eps, stream);
  if (Q <= 192) return launch_rows<MM, GATEUP, 3>(W0, W1, K, N, x, M, out, scale, res, res_scale, gamma, eps, stream);
  return launch_rows<MM, GATEUP, 4>(W0, W1, K, N, x, M, out, scale, res, res_scale, gamma, eps, stream);
}

// The down pass of one token with each row's contraction split over S waves
// (S = ceil(chunks / 64), chunks = inter / 64), so a lane holds the activation
// of one 64-weight chunk in registers and a wave's work per row is one chunk
// per lane.  Twelve waves per workgroup take R = 12 / S rows at a time (wave w:
// row slot w / S, segment w % S); the S partial sums of a row meet in LDS and
// are added in segment order, so the result does not depend on scheduling.
// Persistent workgroups walk the row groups grid-stride with the next group's
// chunk loaded while the current one is computed.  Against whole rows per wave
// (three chunks per lane at inter = 11008), a wave's latency chain per row is a
// third as long and the kernel needs a third of the registers.
template <int S>
struct SplitShape {
  static constexpr int R = 12 / S;                 // rows per group
  static constexpr int WAVES = R * S;
  static constexpr int THREADS = 64 * WAVES;
};

template <int S>
__global__ __launch_bounds__(SplitShape<S>::THREADS) void k_decode_down_split(const uint8_t* __restrict__ W, int K,
                                                                             int N, const _Float16* __restrict__ hin,
                                                                             _Float16* out, float scale,
                                                                             const _Float16* res, float res_scale) {
  using SH = SplitShape<S>;
  constexpr int R = SH::R, THREADS = SH::THREADS;
  extern __shared__ __attribute__((aligned(16))) unsigned char ds_smem[];
  const int nb = K / QK;
  const int Q = 4 * nb;                              // chunks per row
  _Float16* xs = reinterpret_cast<_Float16*>(ds_smem);
  float* X2 = reinterpret_cast<float*>(ds_smem + (size_t)K * 2);          // [2*Q] sub-block sums
  float* part = X2 + 2 * Q;                                                 // [2][R][S] partial sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rs = wave / S, seg = wave - rs * S;
  const NibbleK nk = nibble_consts();
  const size_t row_bytes = (size_t)nb * BLOCK_BYTES;
  const int q = 64 * seg + lane;                      // this lane's chunk
  const bool has = q < Q;
  const int qc = has ? q : 0;
  const int cq = qc & 3;
  const size_t boff = (size_t)(qc >> 2) * BLOCK_BYTES, qoff = boff + 16 + 32 * (qc & 3);
  const int ngroups = (N + R - 1) / R;

  auto load_row = [&](int g, Chunk& c) __attribute__((always_inline)) {
    int j = g * R + rs;
    j = j < N ? j : N - 1;                            // past the end: re-read the last row (never used)
    const uint8_t* row = W + (size_t)j * row_bytes;
    c.hdr = *reinterpret_cast<const uint4*>(row + boff);
    c.q0 = *reinterpret_cast<const uint4*>(row + qoff);
    c.q1 = *reinterpret_cast<const uint4*>(row + qoff + 16);
  };
  // the activation loads first, then the first group's weights
  constexpr int NXG = (DR_KMAX / 8 + THREADS - 1) / THREADS;
  const int nxg = K / 8;
  uint4 xv[NXG];
#pragma unroll
  for (int u = 0; u < NXG; ++u) {
    const int gi = tid + u * THREADS;
    xv[u] = (gi < nxg) ? *reinterpret_cast<const uint4*>(hin + 8 * gi) : make_uint4(0, 0, 0, 0);
  }
  int g = blockIdx.x;
  Chunk cur, nxt;
  load_row(g < ngroups ? g : 0, cur);
  // stage: groups of four with the middle two swapped; fp32 sums of every 32
#pragma unroll
  for (int u = 0; u < NXG; ++u) {
    const int gi = tid + u * THREADS;
    const uint4 v = xv[u];
    if (gi < nxg)
      *reinterpret_cast<uint4*>(xs + 8 * gi) =
          make_uint4((v.x & 0xFFFFu) | (v.y << 16), (v.x >> 16) | (v.y & 0xFFFF0000u),
                     (v.z & 0xFFFFu) | (v.w << 16), (v.z >> 16) | (v.w & 0xFFFF0000u));
    const half8 hv = __builtin_bit_cast(half8, v);
    float s8 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s8 += (float)hv[e];
    s8 += dpp_f<0xB1>(s8);
    s8 += dpp_f<0x4E>(s8);
    if (gi < nxg && (gi & 3) == 0) X2[gi >> 2] = s8;
  }
  lds_barrier();
  uint4 xr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xr[i] = *reinterpret_cast<const uint4*>(xs + 64 * qc + 8 * i);
  const float xlo = X2[2 * qc], xhi = X2[2 * qc + 1];

  for (int it = 0; g < ngroups; ++it, g += gridDim.x) {
    load_row(g + (int)gridDim.x < ngroups ? g + (int)gridDim.x : g, nxt);
    float acc = has ? chunk_dot_reg(cur, cq, xr, xlo, xhi, nk) : 0.0f;
    acc = wave_sum_to_lane63(acc);
    float* pb = part + (it & 1) * R * S;
    if (lane == 63) pb[rs * S + seg] = acc;
    lds_barrier();
    if (tid < R) {
      const int j = g * R + tid;
      if (j < N) {
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < S; ++k) v += pb[tid * S + k];
        v *= scale;
        if (res) v += (float)res[j] * res_scale;   // may be out itself: read, then written, here
        out[j] = (_Float16)v;
      }
    }
    cur = nxt;
  }
}

template <int S>
hipError_t launch_down_split(const void* W, int K, int N, const _Float16* h, _Float16* out, float scale,
                             const _Float16* res, float res_scale, hipStream_t stream) {
  using SH = SplitShape<S>;
  const size_t smem = (size_t)K * 2 + (size_t)2 * (4 * (K / QK)) * 4 + (size_t)2 * SH::R * S * 4;
  static std::atomic<size_t> attr_set{0};
  hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&k_decode_down_split<S>), smem, attr_set);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_down_split<S>, SH::THREADS, smem);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int ngroups = (N + SH::R - 1) / SH::R;
  const int grid = std::max(1, std::min(cu_count() * per_cu, ngroups));
  hipLaunchKernelGGL((k_decode_down_split<S>), dim3(grid), dim3(SH::THREADS), smem, stream,
                     static_cast<const uint8_t*>(W), K, N, h, out, scale, res, res_scale);
  return hipGetLastError();
}

hipError_t launch_down_split_k(const void* W, int K, int N, const _Float16* h, _Float16* out, float scale,
                               const _Float16* res, float res_scale, hipStream_t stream) {
  const int Q = 4 * (K / QK);
  if (Q <= 64) return launch_down_split<1>(W, K, N, h, out, scale, res, res_scale, stream);
  if (Q <= 128) return launch_down_split<2>(W, K, N, h, out, scale, res, res_scale, stream);
  if (Q <= 192) return launch_down_split<3>(W, K, N, h, out, scale, res, res_scale, stream);
  return launch_down_split<4>(W, K, N, h, out, scale, res, res_scale, stream);
}

}  // namespace

size_t decode_workspace_bytes(int M, int hidden, int inter) {
  (void)hidden;
  return ((size_t)(M > 0 ? M : 1) * inter * sizeof(_Float16) + 255) / 256 * 256;
}

hipError_t launch_decode(const void* wg, const void* wu, const void* wd, int hidden, int inter, const void* x, void* y,
                         int M, int inter_shift, int out_shift, void* ws, hipStream_t stream, float mlp_scale,
                         const void* res, const void* gamma, float eps, void* xn) {
  const _Float16* gm = static_cast<const _Float16*>(gamma);
  // The row kernels cover contractions up to DR_KMAX (four 64-chunk slots per
  // lane); a longer down-projection contraction takes the MFMA path, which
  // walks any K in passes.  That path normalises the activation in a kernel
  // of its own first; the row kernels do it while staging.
  if (M >= 2 || inter > DR_KMAX) {
    if (gm) {
      launch_rms_norm(static_cast<const _Float16*>(x), gm, eps, hidden, M, static_cast<_Float16*>(xn), stream);
      x = xn;
    }
    return launch_decode_mfma(wg, wu, wd, hidden, inter, x, y, M, inter_shift, out_shift, ws, stream, mlp_scale,
                              res);
  }
  const float gu_scale = ldexpf(1.0f, -inter_shift);
  const float dn_scale = ldexpf(1.0f, inter_shift - out_shift) * mlp_scale, res_scale = ldexpf(1.0f, -out_shift);
  _Float16* hbuf = static_cast<_Float16*>(ws);
  timing_begin(stream);
  hipError_t e = launch_rows_k<1, true>(wg, wu, hidden, inter, static_cast<const _Float16*>(x), M, hbuf, gu_scale,
                                        nullptr, 0.0f, gm, eps, stream);
  timing_end(stream);
  if (e != hipSuccess) return e;
  timing_begin(stream);
  e = launch_down_split_k(wd, inter, hidden, hbuf, static_cast<_Float16*>(y), dn_scale,
                          static_cast<const _Float16*>(res), res_scale, stream);
  timing_end(stream);
  return e;
}

}  // namespace zinc
