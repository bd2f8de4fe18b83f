// Device-side Q4_K helpers for gfx950 (CDNA4, wave64).
//
// Q4_K super-block (144 B, 256 weights of one row along the contraction
// dimension): bytes 0-1 fp16 d, 2-3 fp16 dmin, 4-15 the packed 6-bit scales
// and mins, 16-143 the 4-bit quants.  Weight i = d*sc_{i/32}*q_i - dmin*m_{i/32};
// quant i sits in quant byte 32*(i/64) + i%32, low nibble for i%64 < 32.
// The pages name the Q4_K block ("Fused SwiGLU MLP: ZINC RDNA4 Down-Projection
// Bandwidth", opening Q&A) and describe unpacking it in registers on the way
// into the multiply ("VGPR pressure caps the fused RDNA4 prefill GEMM at nine
// waves", "What the fused GEMM actually spends registers on").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zinc {

constexpr int QK = 256;          // weights per super-block
constexpr int BLOCK_BYTES = 144; // bytes per super-block
// The experts' other down-projection formats: Q5_K super-blocks (the Q4_K
// header, 32 bytes of fifth bits, 128 quant bytes) and Q5_1 blocks of 32
// weights (fp16 d and m, 32 fifth bits, 16 quant bytes).
constexpr int Q5K_BLOCK_BYTES = 176;
constexpr int Q5_1_BLOCK_BYTES = 24;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Header: d, dmin and the sixteen 6-bit fields.
// w1 = scale bytes S[0..3], w2 = S[4..7], w3 = S[8..11] (little-endian dwords).
// Returns four dwords holding one 6-bit value per byte:
//   sc03 = sc_0..3, sc47 = sc_4..7, m03 = m_0..3, m47 = m_4..7.
// sc_j (j>=4) takes its low nibble from S[j+4] and its top two bits from bits
// 6-7 of S[j-4]; m_j (j>=4) its low nibble from the high nibble of S[j+4] and
// its top two bits from bits 6-7 of S[j].  Shifting whole dwords moves bits
// across byte boundaries only into positions the masks clear.
// ---------------------------------------------------------------------------
struct SixBit {
  uint32_t sc03, sc47, m03, m47;
};

__device__ __forceinline__ SixBit unpack_sixbit(uint32_t w1, uint32_t w2, uint32_t w3) {
  SixBit r;
  r.sc03 = w1 & 0x3F3F3F3Fu;
  r.m03 = w2 & 0x3F3F3F3Fu;
  r.sc47 = (w3 & 0x0F0F0F0Fu) | ((w1 >> 2) & 0x30303030u);
  r.m47 = ((w3 >> 4) & 0x0F0F0F0Fu) | ((w2 >> 2) & 0x30303030u);
  return r;
}

__device__ __forceinline__ uint32_t sixbit_sc(const SixBit& s, int j) {
  uint32_t w = (j < 4) ? s.sc03 : s.sc47;
  return (w >> (8 * (j & 3))) & 0xFFu;
}
__device__ __forceinline__ uint32_t sixbit_m(const SixBit& s, int j) {
  uint32_t w = (j < 4) ? s.m03 : s.m47;
  return (w >> (8 * (j & 3))) & 0xFFu;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// ---------------------------------------------------------------------------
// Bit-exact fp32 weight: d*sc and dmin*m are exact in fp32 (11-bit x 6-bit
// significands), (d*sc)*q is exact too (21 bits), so the single rounding of the
// final subtraction gives RNE32 of the exact value whether or not the multiply
// and the subtraction are fused.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float q4k_weight_f32(float d, float dmin, uint32_t sc, uint32_t m, uint32_t q) {
  float s = d * (float)sc;
  float mm = dmin * (float)m;
  return __builtin_fmaf(s, (float)q, -mm);
}

// ---------------------------------------------------------------------------
// fp16 MFMA operands from one dword of quant bytes.
//
// A dword holds bytes b0..b3 = quants at positions l0..l0+3 of a 64-weight
// chunk: low nibbles are sub-block 2c (weights 64c+l0+e), high nibbles are
// sub-block 2c+1 (weights 64c+32+l0+e).  Exact nibble -> fp16 conversion:
//   (bits & 0x000F000F) | 0x6400 -> 1024 + q   (fp16 ulp at 1024 is 1)
//   (bits & 0x00F000F0) | 0x5400 ->   64 + q   (ulp at 64 is 1/16, q sits at bits 4-7)
// then an exact subtraction of the offset and one fused multiply-add
// w = q*s - dm rounded once to fp16.  The eight operand slots come out as
//   [lo b0, lo b2, lo b1, lo b3, hi b0, hi b2, hi b1, hi b3]
// i.e. weight offsets {0,2,1,3, 32,34,33,35} from 64c+l0; the activation side is
// stored in LDS in the same order (panel_pos), so the contraction pairs match.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2v bits_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

__device__ __forceinline__ half8 dequant_dword_f16(uint32_t Q, half2v s_lo, half2v dm_lo, half2v s_hi,
                                                   half2v dm_hi) {
  const uint32_t Q8 = Q >> 8;
  const half2v off_lo = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2v off_hi = {(_Float16)64.0f, (_Float16)64.0f};
  half2v p0 = bits_h2((Q & 0x000F000Fu) | 0x64006400u) - off_lo;
  half2v p1 = bits_h2((Q8 & 0x000F000Fu) | 0x64006400u) - off_lo;
  half2v p2 = bits_h2((Q & 0x00F000F0u) | 0x54005400u) - off_hi;
  half2v p3 = bits_h2((Q8 & 0x00F000F0u) | 0x54005400u) - off_hi;
  p0 = __builtin_elementwise_fma(p0, s_lo, -dm_lo);
  p1 = __builtin_elementwise_fma(p1, s_lo, -dm_lo);
  p2 = __builtin_elementwise_fma(p2, s_hi, -dm_hi);
  p3 = __builtin_elementwise_fma(p3, s_hi, -dm_hi);
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Per-block fp16 scale pairs for the operand dequant: s_j = fp16(d*sc_j),
// dm_j = fp16(dmin*m_j), each splatted into both halves.
struct BlockScalesF16 {
  half2v s[8];
  half2v dm[8];
};

__device__ __forceinline__ BlockScalesF16 block_scales_f16(uint4 hdr) {
  BlockScalesF16 r;
  const float d = half_bits_to_float(hdr.x & 0xFFFFu);
  const float dmin = half_bits_to_float(hdr.x >> 16);
  const SixBit sb = unpack_sixbit(hdr.y, hdr.z, hdr.w);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    _Float16 s = (_Float16)(d * (float)sixbit_sc(sb, j));
    _Float16 dm = (_Float16)(dmin * (float)sixbit_m(sb, j));
    r.s[j] = half2v{s, s};
    r.dm[j] = half2v{dm, dm};
  }
  return r;
}

// fp16 scale pairs of one 64-weight chunk c (sub-blocks 2c and 2c+1) with a
// run-time chunk index; avoids indexing a register array dynamically.
struct ChunkScalesF16 {
  half2v s_lo, dm_lo, s_hi, dm_hi;
};

__device__ __forceinline__ ChunkScalesF16 chunk_scales_f16(uint4 hdr, int c) {
  const float d = half_bits_to_float(hdr.x & 0xFFFFu);
  const float dmin = half_bits_to_float(hdr.x >> 16);
  const SixBit sb = unpack_sixbit(hdr.y, hdr.z, hdr.w);
  const int j = 2 * c;
  const _Float16 s0 = (_Float16)(d * (float)sixbit_sc(sb, j));
  const _Float16 m0 = (_Float16)(dmin * (float)sixbit_m(sb, j));
  const _Float16 s1 = (_Float16)(d * (float)sixbit_sc(sb, j + 1));
  const _Float16 m1 = (_Float16)(dmin * (float)sixbit_m(sb, j + 1));
  ChunkScalesF16 r;
  r.s_lo = half2v{s0, s0};
  r.dm_lo = half2v{m0, m0};
  r.s_hi = half2v{s1, s1};
  r.dm_hi = half2v{m1, m1};
  return r;
}

// ---------------------------------------------------------------------------
// K-slot order of a 64-wide panel (one 64-weight chunk of a block).
// MFMA substep s (K = 16 each, four per panel) gives lane half h = lane/32 the
// quant dword at byte 32c + 16h + 4s, i.e. positions l0 = 16h + 4s; its eight
// slots hold offsets {0,2,1,3,32,34,33,35} from l0.  The activation operand for
// (substep s, half h) is therefore the 8 contiguous fp16 at panel position
// (2s + h)*8, and element k (0..63) of the chunk lives at panel_pos(k).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int panel_pos(int k) {
  int hi = k >> 5, l = k & 31, h = l >> 4, s = (l >> 2) & 3, e = l & 3;
  int slot = 4 * hi + ((e == 1) ? 2 : (e == 2) ? 1 : e);
  return (2 * s + h) * 8 + slot;
}

// 32x32x16 fp16 MFMA with fp32 accumulation.  Lane l supplies row l%32 of A and
// column l%32 of B, 8 K-values each (K-half l/32); accumulator register r holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also fences
// global memory, which waits for every outstanding global load -- including
// weight prefetches meant to stay in flight across the barrier.  Here each wave
// waits for its own LDS operations, then meets the others; the memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float silu_f32(float g) {
  // g / (1 + e^-g); for g << 0 the exponential overflows to +inf and the
  // quotient is -0, the correct limit.
  return g / (1.0f + __expf(-g));
}

}  // namespace zinc
