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
//   zinc_peak_mfma_valu  how much independent VALU work hides behind 16x16x32
//                        MFMAs: every step is one MFMA and `kv` packed fp16
//                        FMAs, issued by the same wave, or by a second wave on
//                        the same SIMD
//   zinc_peak_mfma32_valu  the same-wave form of zinc_peak_mfma_valu with
//                        32x32x16 MFMAs (four accumulators of 16 registers),
//                        kv up to 12
//   zinc_peak_decode_loop  the fused prefill unit's phase-1 inner loop (Q4_K
//                        decode in registers, B operands from LDS, 16x16x32
//                        MFMAs for gate and up) on L2-resident weights, with
//                        4 or 8 token groups per decoded operand, and with
//                        parts removed (the weight loads, the LDS reads, the
//                        decode) to price each
//   zinc_peak_q4k_stream   the bandwidth of three ways to read a gate/up pair
//                        of Q4_K matrices: one row per wave with the lanes
//                        along the row (the decode row kernels), 16-row tiles
//                        per wave in the MFMA lane layout walked block column
//                        by block column (the fused units, the MFMA decode),
//                        and 16-row tiles of one block column each
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../csrc/fused16.hpp"

namespace {

using zinc::half8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2p __attribute__((ext_vector_type(2)));

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

// MODE 0: every step one MFMA and KV VALU in the same wave; MODE 1: waves
// 0-3 of each 8-wave workgroup issue the MFMAs and waves 4-7 the VALU work
// (one of each per SIMD).  Operands are registers only.  AG: the accumulators
// live in AGPRs (an AGPR clobber makes the compiler select the MFMAs' AGPR
// form) instead of VGPRs.
template <int MODE, int KV, bool AG = false>
__global__ __launch_bounds__(512) void k_mfma_valu(int iters, float* __restrict__ out) {
  if constexpr (AG) asm volatile("" ::: "a0");
  const int tid = threadIdx.x, wave = tid >> 6;
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (float)((tid + e) & 7));
    b[e] = (_Float16)(0.002f * (float)e);
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  half2p v[8];
  const half2p sc = {(_Float16)0.999f, (_Float16)1.001f}, cc = {(_Float16)0.001f, (_Float16)-0.001f};
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = half2p{(_Float16)(0.1f * k), (_Float16)(tid & 3)};
  const bool do_mfma = MODE == 0 || wave < 4;
  const bool do_valu = KV > 0 && (MODE == 0 || wave >= 4);
  if (do_mfma && do_valu) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < KV; ++j) v[(k + j) & 7] = __builtin_elementwise_fma(v[(k + j) & 7], sc, cc);
      }
    }
  } else if (do_mfma) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
    }
  } else if (do_valu) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int j = 0; j < KV; ++j) v[(k + j) & 7] = __builtin_elementwise_fma(v[(k + j) & 7], sc, cc);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) r += acc[k][0] + (float)v[k][0] + (float)v[k][1];
  out[(size_t)blockIdx.x * 512 + tid] = r;
}

// Every step one 32x32x16 MFMA and KV packed fp16 FMAs of the same wave;
// registers only.
template <int KV>
__global__ __launch_bounds__(512) void k_mfma32_valu(int iters, float* __restrict__ out) {
  const int tid = threadIdx.x;
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (float)((tid + e) & 7));
    b[e] = (_Float16)(0.002f * (float)e);
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  half2p v[8];
  const half2p sc = {(_Float16)0.999f, (_Float16)1.001f}, cc = {(_Float16)0.001f, (_Float16)-0.001f};
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = half2p{(_Float16)(0.1f * k), (_Float16)(tid & 3)};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < KV; ++j) v[(k + j) & 7] = __builtin_elementwise_fma(v[(k + j) & 7], sc, cc);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) r += acc[k][0];
#pragma unroll
  for (int k = 0; k < 8; ++k) r += (float)v[k][0] + (float)v[k][1];
  out[(size_t)blockIdx.x * 512 + tid] = r;
}

// Split-K partial sinks of the fused prefill unit's phase 2, at its shape (n_wg
// workgroups of 12 waves, each writing a 64-token x 4096-row partial in 32-row
// tiles, lanes along the rows):
//   MODE 0: fp16 stores, each workgroup to its own region (the unit's partials)
//   MODE 1: fp32 stores, each workgroup to its own region
//   MODE 2: fp32 atomic adds into one accumulator per (XCD, token tile of
//           blockIdx % 4), the XCD taken from the hardware XCC id, so every
//           accumulator is updated from one XCD only
// acc: 8 * 4 * 64 * 4096 floats (zeroed by the caller for MODE 2); part:
// n_wg * 64 * 4096 floats; wg_xcc: n_wg ints (the XCC id each workgroup ran on).
constexpr int PS_TOK = 64, PS_H = 4096;
__device__ __forceinline__ int hw_xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 15;
}
template <int MODE>
__global__ __launch_bounds__(768) void k_partial_sink(float* __restrict__ acc, void* __restrict__ part,
                                                      int* __restrict__ wg_xcc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xcc = hw_xcc_id();
  if (threadIdx.x == 0) wg_xcc[blockIdx.x] = xcc;
  const int l32 = lane & 31, h = lane >> 5;
  float* const abase = acc + ((size_t)(xcc & 7) * 4 + blockIdx.x % 4) * PS_TOK * PS_H;
  _Float16* const pb = static_cast<_Float16*>(part) + (size_t)blockIdx.x * PS_TOK * PS_H;
  float* const fb = static_cast<float*>(part) + (size_t)blockIdx.x * PS_TOK * PS_H;
  for (int nt = wave; nt < PS_H / 32; nt += 12) {
    const int n = nt * 32 + l32;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t off = (size_t)(32 * t2 + 8 * q + 4 * h + e) * PS_H + n;
          if constexpr (MODE == 0) pb[off] = (_Float16)1.0f;
          else if constexpr (MODE == 1) fb[off] = 1.0f;
          else __hip_atomic_fetch_add(abase + off, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
  }
}

// The phase-1 loop of the fused unit (the lane layout, decode, scales and
// issue pattern of fused16.hpp) over nblk blocks, repeated `reps` times, with
// NG 16-token groups per decoded operand and WAVES waves of 16 rows each.
// Every workgroup reads the same rows (L2-resident); the activation column
// sits in LDS unchanged.  VAR: 0 as in the kernel; 2 without the decode (a
// fixed A operand); 4 without the weight loads (the quant words change in
// registers); 5 as 4 and with the B operands held in registers.
template <int NG, int WAVES, int VAR>
__global__ __launch_bounds__(64 * WAVES) void k_decode_loop(const uint8_t* __restrict__ wg,
                                                            const uint8_t* __restrict__ wu, int nblk, int reps,
                                                            float* __restrict__ out) {
  using namespace zinc;
  constexpr int XS = 264;
  __shared__ __attribute__((aligned(16))) _Float16 xs[NG * 16 * XS];
  for (int i = threadIdx.x; i < NG * 16 * XS; i += 64 * WAVES) xs[i] = (_Float16)(0.001f * (float)(i & 15));
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, o = lane >> 4, sel = (o >> 1) & 1;
  const uint32_t psel = sc_pair_sel(2 * sel);
  const NibbleK nk = nibble_consts_s();
  const uint32_t rowb = (uint32_t)nblk * BLOCK_BYTES;
  const uint32_t wrow_off = (uint32_t)(wave * 16 + r) * rowb;
  f32x4_16 accg[NG], accu[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) accg[g][e] = accu[g][e] = 0.0f;
  u32x4_16 hg = *reinterpret_cast<const u32x4_16*>(wg + wrow_off);
  u32x4_16 hu = *reinterpret_cast<const u32x4_16*>(wu + wrow_off);
  u32x4_16 qg0 = *reinterpret_cast<const u32x4_16*>(wg + (wrow_off + 16 + 16 * o));
  u32x4_16 qu0 = *reinterpret_cast<const u32x4_16*>(wu + (wrow_off + 16 + 16 * o));
  u32x4_16 qg1 = *reinterpret_cast<const u32x4_16*>(wg + (wrow_off + 80 + 16 * o));
  u32x4_16 qu1 = *reinterpret_cast<const u32x4_16*>(wu + (wrow_off + 80 + 16 * o));
  const int xlane = r * XS + o * 8;
  half8 bfix[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) bfix[g] = *reinterpret_cast<const half8*>(xs + xlane + g * 16 * XS);
  const half8 afix = bfix[0];
  for (int rep = 0; rep < reps; ++rep) {
    for (int kb = 0; kb < nblk; ++kb) {
      const int kn = (kb + 1 < nblk) ? kb + 1 : 0;
      const uint32_t noff = wrow_off + (uint32_t)kn * BLOCK_BYTES;
      const Lane16S sg = lane16_scales(as_u4(hg), psel), su = lane16_scales(as_u4(hu), psel);
      if constexpr (VAR < 4) {
        hg = *reinterpret_cast<const u32x4_16*>(wg + noff);
        hu = *reinterpret_cast<const u32x4_16*>(wu + noff);
      } else {
        const uint32_t d = (uint32_t)kb * 0x01010101u;
        qg0 += d;
        qu0 += d;
        qg1 += d;
        qu1 += d;
      }
      __builtin_amdgcn_sched_barrier(0);
      auto load_b = [&](int i, half8 (&b)[NG]) {
        if constexpr (VAR == 5) {
#pragma unroll
          for (int g = 0; g < NG; ++g) b[g] = bfix[g];
        } else {
#pragma unroll
          for (int g = 0; g < NG; ++g) b[g] = *reinterpret_cast<const half8*>(xs + xlane + g * 16 * XS + i * 32);
        }
      };
      auto decode = [&](int i, half8& ag, half8& au) {
        const uint32_t qg = (i < 4) ? qg0[i & 3] : qg1[i & 3];
        const uint32_t qu = (i < 4) ? qu0[i & 3] : qu1[i & 3];
        ag = dequant_dword_sc(qg, (i < 4) ? sg.r0 : sg.r1, nk);
        au = dequant_dword_sc(qu, (i < 4) ? su.r0 : su.r1, nk);
      };
      half8 bc[NG], bn[NG], agc, auc, agn, aun;
      load_b(0, bc);
      decode(0, agc, auc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < 7) {
          load_b(i + 1, bn);
          decode(i + 1, agn, aun);
        }
        if (VAR < 4 && i == 3) {
          qg0 = *reinterpret_cast<const u32x4_16*>(wg + (noff + 16 + 16 * o));
          qu0 = *reinterpret_cast<const u32x4_16*>(wu + (noff + 16 + 16 * o));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (VAR < 4 && i == 6) {
          qg1 = *reinterpret_cast<const u32x4_16*>(wg + (noff + 80 + 16 * o));
          qu1 = *reinterpret_cast<const u32x4_16*>(wu + (noff + 80 + 16 * o));
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          accg[g] = mfma16x16(VAR == 2 ? afix : agc, bc[g], accg[g]);
          accu[g] = mfma16x16(VAR == 2 ? afix : auc, bc[g], accu[g]);
        }
        if (i < 7) {
#pragma unroll
          for (int g = 0; g < NG; ++g) bc[g] = bn[g];
          agc = agn;
          auc = aun;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NG, 0);
#pragma unroll
        for (int k = 0; k < 2 * NG; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, NG >= 8 ? 2 : 3, 0);
        }
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) sum += accg[g][0] + accu[g][1];
  out[(size_t)blockIdx.x * 64 * WAVES + threadIdx.x] = sum;
}


// The same phase-1 work as k_decode_loop<4, 12, VAR> (64 tokens, gate and up
// of 192 rows) on 32x32x16 MFMAs: wave w owns one matrix (gate for even w, up
// for odd) of the 32-row tile w / 2, for both 32-token halves.  Lane (r, h) =
// (lane % 32, lane / 32) decodes row r's quant bytes [64h, 64h + 64) of each
// block, one dword per MFMA step (sixteen steps per block; chunk 2h for steps
// 0-7, 2h + 1 for 8-15), and the B operand of step s is token lane % 32's
// activation piece of that dword.  Same VAR meanings as k_decode_loop.
template <int VAR>
__global__ __launch_bounds__(768) void k_decode_loop32(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                                       int nblk, int reps, float* __restrict__ out) {
  using namespace zinc;
  constexpr int XS = 264;
  __shared__ __attribute__((aligned(16))) _Float16 xs[64 * XS];
  for (int i = threadIdx.x; i < 64 * XS; i += 768) xs[i] = (_Float16)(0.001f * (float)(i & 15));
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const NibbleK nk = nibble_consts_s();
  const uint8_t* const w = (wave & 1) ? wu : wg;
  const uint32_t rowb = (uint32_t)nblk * BLOCK_BYTES;
  const uint32_t wrow_off = (uint32_t)((wave >> 1) * 32 + r) * rowb;
  float16v acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  u32x4_16 hd = *reinterpret_cast<const u32x4_16*>(w + wrow_off);
  u32x4_16 q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = *reinterpret_cast<const u32x4_16*>(w + (wrow_off + 16 + 64 * h + 16 * i));
  const _Float16* const xl = xs + r * XS + 64 * h;   // token r of half 0; chunk 2h's first piece
  const half8 afix = *reinterpret_cast<const half8*>(xl);
  const uint32_t psel0 = sc_pair_sel(0), psel1 = sc_pair_sel(2);
  for (int rep = 0; rep < reps; ++rep) {
    for (int kb = 0; kb < nblk; ++kb) {
      const int kn = (kb + 1 < nblk) ? kb + 1 : 0;
      const uint32_t noff = wrow_off + (uint32_t)kn * BLOCK_BYTES;
      const uint4 hh = as_u4(hd);
      const half2v d2 = splat_d(hh.x);
      const half2v nd = d2 * half2v{(_Float16)-1024.0f, (_Float16)-1024.0f};
      const uint32_t scw = h ? sc47_bytes(hh) : sc03_bytes(hh);
      const half2v s0 = scale_pair(__builtin_amdgcn_perm(0x64646464u, scw, psel0), d2, nd);
      const half2v s1 = scale_pair(__builtin_amdgcn_perm(0x64646464u, scw, psel1), d2, nd);
      u32x4_16 qn[4];
      if constexpr (VAR < 4) {
        hd = *reinterpret_cast<const u32x4_16*>(w + noff);
#pragma unroll
        for (int i = 0; i < 4; ++i) qn[i] = *reinterpret_cast<const u32x4_16*>(w + (noff + 16 + 64 * h + 16 * i));
      } else {
        const uint32_t d = (uint32_t)kb * 0x01010101u;
#pragma unroll
        for (int i = 0; i < 4; ++i) qn[i] = q[i] + d;
      }
      __builtin_amdgcn_sched_barrier(0);
      auto load_b = [&](int st, half8 (&b)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) b[t] = (VAR == 5) ? afix : *reinterpret_cast<const half8*>(xl + t * 32 * XS + st * 8);
      };
      auto decode = [&](int st) -> half8 { return dequant_dword_sc(q[st >> 2][st & 3], (st < 8) ? s0 : s1, nk); };
      half8 bc[2], bn[2], ac, an;
      load_b(0, bc);
      ac = decode(0);
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        if (st < 15) {
          load_b(st + 1, bn);
          an = decode(st + 1);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma32(VAR == 2 ? afix : ac, bc[t], acc[t]);
        if (st < 15) {
          bc[0] = bn[0];
          bc[1] = bn[1];
          ac = an;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = qn[i];
    }
  }
  out[(size_t)blockIdx.x * 768 + threadIdx.x] = acc[0][0] + acc[1][1];
}

// Q4_K stream layouts (loads only, folded into a sink).  LAYOUT 0: wave per
// row, lane l = 64-weight chunk l of the row (block header + its 32 quant
// bytes); LAYOUT 1: wave per 16-row tile, lane (r, o) = row r, quant pieces
// [16o, +16) and [64 + 16o, +16) and the header of every block in turn, two
// blocks ahead.
template <int LAYOUT>
__global__ __launch_bounds__(256) void k_q4k_stream(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                                    int nb, int nrows, uint32_t* __restrict__ out) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const uint32_t rowb = (uint32_t)nb * 144u;
  u4v sink = {0u, 0u, 0u, 0u};
  if constexpr (LAYOUT == 0) {
    const uint32_t boff = (uint32_t)(lane >> 2) * 144u, qoff = boff + 16u + 32u * (uint32_t)(lane & 3);
    const bool has = (lane >> 2) < nb;
    for (int j = wave; j < nrows; j += nw) {
      if (!has) break;
      const uint32_t b = (uint32_t)j * rowb;
      sink ^= *reinterpret_cast<const u4v*>(wg + b + boff);
      sink ^= *reinterpret_cast<const u4v*>(wg + b + qoff);
      sink ^= *reinterpret_cast<const u4v*>(wg + b + qoff + 16);
      sink ^= *reinterpret_cast<const u4v*>(wu + b + boff);
      sink ^= *reinterpret_cast<const u4v*>(wu + b + qoff);
      sink ^= *reinterpret_cast<const u4v*>(wu + b + qoff + 16);
    }
  } else {
    const int r = lane & 15, o = lane >> 4;
    for (int t = wave; t < nrows / 16; t += nw) {
      const uint32_t base = (uint32_t)(t * 16 + r) * rowb;
      u4v buf[2][6];
      auto ld = [&](int a, int kb) __attribute__((always_inline)) {
        const uint32_t off = base + (uint32_t)(kb < nb ? kb : nb - 1) * 144u;
        buf[a][0] = *reinterpret_cast<const u4v*>(wg + off);
        buf[a][1] = *reinterpret_cast<const u4v*>(wg + off + 16 + 16 * o);
        buf[a][2] = *reinterpret_cast<const u4v*>(wg + off + 80 + 16 * o);
        buf[a][3] = *reinterpret_cast<const u4v*>(wu + off);
        buf[a][4] = *reinterpret_cast<const u4v*>(wu + off + 16 + 16 * o);
        buf[a][5] = *reinterpret_cast<const u4v*>(wu + off + 80 + 16 * o);
      };
      ld(0, 0);
      ld(1, 1);
      for (int kb = 0; kb < nb; kb += 2) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
          for (int m = 0; m < 6; ++m) sink ^= buf[a][m];
          ld(a, kb + a + 2);
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int m = 0; m < 6; ++m) sink ^= buf[a][m];
    }
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = sink.x ^ sink.y ^ sink.z ^ sink.w;
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

// blocks x 512 threads; `out` holds blocks * 512 floats.  Returns the MFMAs
// issued per SIMD (the step count of the MFMA waves), 0 on an error.
double zinc_peak_mfma_valu(int same_wave, int kv, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out || kv < 0 || kv > 4) return 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define ZP_MV(MODE, KV) hipLaunchKernelGGL((k_mfma_valu<MODE, KV>), dim3(blocks), dim3(512), 0, s, iters, out)
  if (same_wave) {
    switch (kv) { case 0: ZP_MV(0, 0); break; case 1: ZP_MV(0, 1); break; case 2: ZP_MV(0, 2); break;
                  case 3: ZP_MV(0, 3); break; default: ZP_MV(0, 4); break; }
  } else {
    switch (kv) { case 0: ZP_MV(1, 0); break; case 1: ZP_MV(1, 1); break; case 2: ZP_MV(1, 2); break;
                  case 3: ZP_MV(1, 3); break; default: ZP_MV(1, 4); break; }
  }
#undef ZP_MV
  if (hipGetLastError() != hipSuccess) return 0.0;
  // per SIMD (two waves of an 8-wave workgroup per SIMD, one workgroup per CU
  // and round): MFMAs issued by its MFMA-issuing waves
  return (double)iters * 8 * (same_wave ? 2 : 1);
}

// Probe 1's same-wave form with the accumulators in AGPRs; kv 0..4.
double zinc_peak_mfma_valu_agpr(int kv, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out || kv < 0 || kv > 4) return 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define ZP_MA(KV) hipLaunchKernelGGL((k_mfma_valu<0, KV, true>), dim3(blocks), dim3(512), 0, s, iters, out)
  switch (kv) { case 0: ZP_MA(0); break; case 1: ZP_MA(1); break; case 2: ZP_MA(2); break;
                case 3: ZP_MA(3); break; default: ZP_MA(4); break; }
#undef ZP_MA
  if (hipGetLastError() != hipSuccess) return 0.0;
  return (double)iters * 8 * 2;
}

// One launch of the partial-sink probe (k_partial_sink) over n_wg workgroups;
// mode 0..2.  Returns 0, or -1 on an invalid argument or a launch error.
int zinc_peak_partial_sink(int mode, int n_wg, float* acc, void* part, int* wg_xcc, void* stream) {
  if (!acc || !part || !wg_xcc || n_wg < 1 || mode < 0 || mode > 2) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0)
    hipLaunchKernelGGL(k_partial_sink<0>, dim3(n_wg), dim3(768), 0, s, acc, part, wg_xcc);
  else if (mode == 1)
    hipLaunchKernelGGL(k_partial_sink<1>, dim3(n_wg), dim3(768), 0, s, acc, part, wg_xcc);
  else
    hipLaunchKernelGGL(k_partial_sink<2>, dim3(n_wg), dim3(768), 0, s, acc, part, wg_xcc);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// blocks x 512 threads; `out` holds blocks * 512 floats; kv in {0..4, 6, 8,
// 12}.  Returns the 32x32x16 MFMAs issued per SIMD, 0 on an error.
double zinc_peak_mfma32_valu(int kv, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define ZP_M32(KV) hipLaunchKernelGGL((k_mfma32_valu<KV>), dim3(blocks), dim3(512), 0, s, iters, out)
  switch (kv) {
    case 0: ZP_M32(0); break;
    case 1: ZP_M32(1); break;
    case 2: ZP_M32(2); break;
    case 3: ZP_M32(3); break;
    case 4: ZP_M32(4); break;
    case 6: ZP_M32(6); break;
    case 8: ZP_M32(8); break;
    case 12: ZP_M32(12); break;
    default: return 0.0;
  }
#undef ZP_M32
  if (hipGetLastError() != hipSuccess) return 0.0;
  return (double)iters * 4 * 2;   // two waves per SIMD, four MFMAs per iteration each
}

// The phase-1 loop probe.  ng 4 (12 waves) or 8 (8 waves); var 0, 2, 4 or 5;
// weights: 192 rows x nblk blocks of Q4_K for each of gate and up (every row
// of both read); out holds blocks * 768 floats.  Returns the MFMAs per SIMD.
double zinc_peak_decode_loop(int ng, int var, const void* wg, const void* wu, int nblk, int reps, int blocks,
                             float* out, void* stream) {
  if (!wg || !wu || !out || nblk < 1 || reps < 1 || blocks < 1) return 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* g = static_cast<const uint8_t*>(wg);
  const uint8_t* u = static_cast<const uint8_t*>(wu);
#define ZP_DL(NG, W, V) hipLaunchKernelGGL((k_decode_loop<NG, W, V>), dim3(blocks), dim3(64 * W), 0, s, g, u, nblk, reps, out)
  if (ng == 4) {
    switch (var) { case 0: ZP_DL(4, 12, 0); break; case 2: ZP_DL(4, 12, 2); break; case 4: ZP_DL(4, 12, 4); break;
                   case 5: ZP_DL(4, 12, 5); break; default: return 0.0; }
  } else if (ng == 8) {
    switch (var) { case 0: ZP_DL(8, 8, 0); break; case 2: ZP_DL(8, 8, 2); break; case 4: ZP_DL(8, 8, 4); break;
                   case 5: ZP_DL(8, 8, 5); break; default: return 0.0; }
  } else {
    return 0.0;
  }
#undef ZP_DL
  if (hipGetLastError() != hipSuccess) return 0.0;
  const int waves = (ng == 4) ? 12 : 8;
  return (double)waves / 4 * reps * nblk * 8 * ng * 2;
}

// The phase-1 loop probe on 32x32x16 MFMAs (k_decode_loop32); var 0, 2, 4 or
// 5; weights as zinc_peak_decode_loop.  Returns the MFMAs per SIMD counted as
// 16x16x32 equivalents (two per 32x32x16), so rates compare with that probe.
double zinc_peak_decode_loop32(int var, const void* wg, const void* wu, int nblk, int reps, int blocks, float* out,
                               void* stream) {
  if (!wg || !wu || !out || nblk < 1 || reps < 1 || blocks < 1) return 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* g = static_cast<const uint8_t*>(wg);
  const uint8_t* u = static_cast<const uint8_t*>(wu);
  switch (var) {
    case 0: hipLaunchKernelGGL(k_decode_loop32<0>, dim3(blocks), dim3(768), 0, s, g, u, nblk, reps, out); break;
    case 2: hipLaunchKernelGGL(k_decode_loop32<2>, dim3(blocks), dim3(768), 0, s, g, u, nblk, reps, out); break;
    case 4: hipLaunchKernelGGL(k_decode_loop32<4>, dim3(blocks), dim3(768), 0, s, g, u, nblk, reps, out); break;
    case 5: hipLaunchKernelGGL(k_decode_loop32<5>, dim3(blocks), dim3(768), 0, s, g, u, nblk, reps, out); break;
    default: return 0.0;
  }
  if (hipGetLastError() != hipSuccess) return 0.0;
  return 3.0 * reps * nblk * 16 * 2 * 2;
}

// One launch of a Q4_K stream layout over a gate/up pair of nrows x (256 nb)
// matrices: layout 0 (row per wave, nb <= 16), 1 (16-row tiles, nrows a
// multiple of 16, nb even).  blocks x 256 threads; `out` holds blocks * 256
// words.  Returns 0, or -1 on an invalid argument.
int zinc_peak_q4k_stream(int layout, const void* wg, const void* wu, int nb, int nrows, int blocks, uint32_t* out,
                         void* stream) {
  if (!wg || !wu || !out || nb < 1 || nrows < 16 || blocks < 1) return -1;
  if (layout == 0 && nb > 16) return -1;
  if (layout == 1 && ((nrows % 16) != 0 || (nb % 2) != 0)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* g = static_cast<const uint8_t*>(wg);
  const uint8_t* u = static_cast<const uint8_t*>(wu);
  if (layout == 0)
    hipLaunchKernelGGL(k_q4k_stream<0>, dim3(blocks), dim3(256), 0, s, g, u, nb, nrows, out);
  else if (layout == 1)
    hipLaunchKernelGGL(k_q4k_stream<1>, dim3(blocks), dim3(256), 0, s, g, u, nb, nrows, out);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
