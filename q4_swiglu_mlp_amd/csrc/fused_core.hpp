// The fused Q4_K SwiGLU work unit shared by the dense prefill kernel and the
// batched-expert kernel.
//
// One unit = (MT activation rows) x (one chunk [r0, r1) of intermediate rows,
// r1 - r0 a multiple of 64, at most ICMAX).  Activation rows are tokens given
// by a per-unit map row -> token (dense prefill: a contiguous tile; MoE: the
// (token, slot) pairs routed to one expert).
//
// Phase 1 (gate+up).  For each 256-wide super-block column kb of the hidden
//   dimension the unit's x rows are staged in LDS as fp16 in panel order
//   (panel_pos), together with the means of every 32-element sub-block.  Each
//   wave owns row tiles of 32 intermediate rows; it decodes the gate and up
//   Q4_K blocks of its rows in registers into fp16 MFMA operands w' = q*s
//   (s = d*sc, one fused multiply-add per pair of weights) and accumulates
//   32x32x16 MFMAs in fp32.  The min term of Q4_K, -dmin*m per sub-block, is
//   the same for all 32 weights of a sub-block, so it is applied by one extra
//   MFMA per two super-blocks that contracts -32*dmin*m against the sub-block
//   means of x: sum_k w_k x_k = sum_k q_k s x_k - sum_j 32 dmin m_j Xbar_j
//   (means rather than sums keep the fp16 operand in the activation's range;
//   the factor 32 is exact).  SwiGLU is
//   applied to the accumulators in registers; the result, scaled by
//   2^-inter_shift, is written as fp16 into the LDS strip [MT x chunk] with its
//   32-row means.  Row tiles beyond what the accumulators hold are done in more
//   passes over the hidden dimension.  The intermediate never leaves the chip.
// Phase 2 (down).  The strip is the B operand of the down projection over the
//   chunk's columns of W_down (same dequant and min correction, the 32-row
//   means of the strip standing in for those of x); each 32-row tile of the
//   hidden output is produced
//   from the strip held in LDS and handed to the output policy (dense: a plain
//   fp16 partial store per chunk at the output scale; MoE: see k_moe.hip).
//
// This is the dataflow of "Fused SwiGLU MLP: ZINC RDNA4 Down-Projection
// Bandwidth" ("Why this fusion is harder than the last one" and the fused row
// of Fig. 1): the kernel walks the intermediate dimension in pieces, and each
// piece is produced on chip, held in LDS and consumed at once by the down
// projection before the next piece is made.  The dequant is fused into the
// producer GEMM as on "VGPR pressure caps the fused RDNA4 prefill GEMM at nine
// waves" (scale values kept out of
// per-lane work as that page's "The recoverable registers versus the stubborn
// ones" advises).  The RDNA4 16x16 WMMA tiling there is replaced by gfx950
// 32x32x16 MFMA on 64-wide waves.
//
// fp16 operand limit: w' = (1024 + q)*s - 1024*s needs 1024*s < 65504, i.e.
// |d * sc| < 63.96 (|d| < 1.015); Q4_K super-block scales are far below it.
#pragma once

#include "q4k_device.hpp"

namespace zinc {

// Waves per workgroup.  One 32-row token tile: 12 waves, three per SIMD, so one
// wave's dequant (VALU) overlaps another's MFMA within 168 registers per lane.
// Two token tiles double the accumulators: 8 waves with 256 registers each.
template <int TT>
struct FuWaves {
  static constexpr int value = (TT == 1) ? 12 : 8;
};

// The nibble masks and fp16 exponent patterns live in VGPRs: gfx9-family VOP3
// encodings take no literal constants, and with both operands in registers
// (q & mask) | magic is a single v_and_or_b32.
struct NibbleK {
  uint32_t lo_mask, hi_mask, lo_magic, hi_magic;
};

__device__ __forceinline__ NibbleK nibble_consts() {
  NibbleK k;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.lo_mask));
  asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(k.hi_mask));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.lo_magic));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(k.hi_magic));
  return k;
}

template <int TT, int RTW, int ICMAX>
struct FusedCfg {
  static constexpr int MT = 32 * TT;                  // activation rows per unit
  static constexpr int WAVES = FuWaves<TT>::value;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int XS = QK + 8;                   // x stage row stride (halves), padded
  static constexpr int HS = ICMAX + 8;                // strip row stride (halves), padded
  static constexpr int NBMAX = (ICMAX - 64) / 256 + 2;  // W_down blocks a chunk can touch
  // strip means per row: 8 slots per touched block (block-aligned), rounded to 16
  static constexpr int HSS = ((8 * NBMAX + 15) / 16) * 16;
  static_assert(ICMAX % 64 == 0, "chunks are whole 64-wide panels");
};

template <int TT, int RTW, int ICMAX>
struct FusedSmem {
  using C = FusedCfg<TT, RTW, ICMAX>;
  _Float16 xs[2][C::MT * C::XS];  // x stage, double-buffered by super-block column
  _Float16 xsum[2][C::MT * 8];    // 32-means of the staged x, sub-block order [0,2,1,3,4,6,5,7]
  _Float16 hs[C::MT * C::HS];     // the intermediate strip
  _Float16 hsum[C::MT * C::HSS];  // 32-row means of the strip, block-aligned, zero-padded
};

// Position of sub-block j in the min-correction operands: bits 0 and 1 swapped,
// which is the order the packed scale/min unpack below produces.
__host__ __device__ constexpr int sb_slot(int j) { return (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1); }

// w' = q*s for the eight operand slots of one quant dword (see
// dequant_dword_f16 for the slot order).  (off + q)*s - off*s is exact before
// its single rounding, so each slot is RNE16(q*s).
__device__ __forceinline__ half8 dequant_dword_scaled(uint32_t Q, half2v s_lo, half2v c_lo, half2v s_hi,
                                                      half2v c_hi, const NibbleK& k) {
  const uint32_t Q8 = Q >> 8;
  half2v p0 = __builtin_elementwise_fma(bits_h2((Q & k.lo_mask) | k.lo_magic), s_lo, c_lo);
  half2v p1 = __builtin_elementwise_fma(bits_h2((Q8 & k.lo_mask) | k.lo_magic), s_lo, c_lo);
  half2v p2 = __builtin_elementwise_fma(bits_h2((Q & k.hi_mask) | k.hi_magic), s_hi, c_hi);
  half2v p3 = __builtin_elementwise_fma(bits_h2((Q8 & k.hi_mask) | k.hi_magic), s_hi, c_hi);
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight 6-bit values (bytes of lo4 = v0..v3, hi4 = v4..v7) times an fp16 factor
// f, each rounded once to fp16, as pairs (v0,v2) (v1,v3) (v4,v6) (v5,v7):
// (1024 + v)*f - 1024*f is exact before rounding.
struct Pairs8 {
  half2v p02, p13, p46, p57;
};

__device__ __forceinline__ Pairs8 scaled_pairs(uint32_t lo4, uint32_t hi4, half2v f2) {
  const half2v nf = f2 * half2v{(_Float16)-1024.0f, (_Float16)-1024.0f};
  Pairs8 r;
  r.p02 = __builtin_elementwise_fma(bits_h2((lo4 & 0x00FF00FFu) | 0x64006400u), f2, nf);
  r.p13 = __builtin_elementwise_fma(bits_h2(((lo4 >> 8) & 0x00FF00FFu) | 0x64006400u), f2, nf);
  r.p46 = __builtin_elementwise_fma(bits_h2((hi4 & 0x00FF00FFu) | 0x64006400u), f2, nf);
  r.p57 = __builtin_elementwise_fma(bits_h2(((hi4 >> 8) & 0x00FF00FFu) | 0x64006400u), f2, nf);
  return r;
}

__device__ __forceinline__ half2v splat_lo(uint32_t bits16) {
  return bits_h2((bits16 & 0xFFFFu) | (bits16 << 16));
}

// Scale registers of the decode below.  A sub-block's s = RNE16(d*sc) is
// taken as (1024 + sc)*d - 1024*d, rounded once, and then scaled exactly by a
// power of two: a register holds (1024*s_a, 64*s_b) for a low-nibble
// sub-block a and the high-nibble sub-block b of the same 64-weight chunk.
// The input is the fp16 pair (1024 + sc_a, 1024 + sc_b) as bits.
__device__ __forceinline__ half2v scale_pair(uint32_t bits, half2v d2, half2v nd2) {
  const half2v s = __builtin_elementwise_fma(bits_h2(bits), d2, nd2);
  return s * half2v{(_Float16)1024.0f, (_Float16)64.0f};
}

// d of a block header (its low half) in both halves of a register.
__device__ __forceinline__ half2v splat_d(uint32_t x) { return bits_h2(__builtin_amdgcn_perm(x, x, 0x01000100u)); }

// Six-bit scales 0..3 (masked) and 4..7 (low four bits from word 3, top two
// from bits 6..7 of word 1), one per byte.
__device__ __forceinline__ uint32_t sc03_bytes(uint4 hdr) { return hdr.y & 0x3F3F3F3Fu; }
__device__ __forceinline__ uint32_t sc47_bytes(uint4 hdr) {
  return (hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u);
}

// v_perm selector that turns bytes j and j + 1 of a word (src1) into the fp16
// pair (1024 + byte_j, 1024 + byte_j+1): each half's high byte is 0x64, taken
// from byte 0 of src0 = 0x64646464.
__host__ __device__ constexpr uint32_t sc_pair_sel(int j) {
  return 0x04000400u | ((uint32_t)(j + 1) << 16) | (uint32_t)j;
}

// The two chunks a lane decodes per block (chunk c0 = sel, c1 = 2 + sel):
// r0 for sub-blocks (2 sel, 2 sel + 1), r1 for (4 + 2 sel, 5 + 2 sel);
// psel = sc_pair_sel(2 sel).
struct Lane16S {
  half2v r0, r1;
};

__device__ __forceinline__ Lane16S lane16_scales(uint4 hdr, uint32_t psel) {
  const half2v d2 = splat_d(hdr.x);
  const half2v nd = d2 * half2v{(_Float16)-1024.0f, (_Float16)-1024.0f};
  Lane16S r;
  r.r0 = scale_pair(__builtin_amdgcn_perm(0x64646464u, sc03_bytes(hdr), psel), d2, nd);
  r.r1 = scale_pair(__builtin_amdgcn_perm(0x64646464u, sc47_bytes(hdr), psel), d2, nd);
  return r;
}

// w' = q*s for the eight operand slots of one quant dword (the slot order of
// dequant_dword_f16), from the register R = (1024*s_a, 64*s_b).  The nibble
// becomes an fp16 in [1, 2) by OR-ing in the exponent of 1.0: a low nibble
// reads 1 + q/1024, a high one (bits 4..7) 1 + q/64; fma(v, S, -S) is then
// q*s exactly before its single rounding, with -S taken by a negation
// modifier of the same register.
__device__ __forceinline__ half8 dequant_dword_sc(uint32_t Q, half2v R, const NibbleK& k) {
  const half2v S_lo = __builtin_shufflevector(R, R, 0, 0), S_hi = __builtin_shufflevector(R, R, 1, 1);
  const uint32_t Q8 = Q >> 8;
  const half2v p0 = __builtin_elementwise_fma(bits_h2((Q & k.lo_mask) | k.lo_magic), S_lo, -S_lo);
  const half2v p1 = __builtin_elementwise_fma(bits_h2((Q8 & k.lo_mask) | k.lo_magic), S_lo, -S_lo);
  const half2v p2 = __builtin_elementwise_fma(bits_h2((Q & k.hi_mask) | k.hi_magic), S_hi, -S_hi);
  const half2v p3 = __builtin_elementwise_fma(bits_h2((Q8 & k.hi_mask) | k.hi_magic), S_hi, -S_hi);
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The nibble masks in SGPRs (a VALU operation may read one), the exponent
// patterns in VGPRs: (q & mask) | magic stays one v_and_or_b32.
// Both exponent patterns are 1.0 here (dequant_dword_sc).
__device__ __forceinline__ NibbleK nibble_consts_s() {
  NibbleK k;
  asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(k.lo_mask));
  asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(k.hi_mask));
  asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(k.lo_magic));
  k.hi_magic = k.lo_magic;
  return k;
}

// s_j = RNE16(d*sc_j) of a block, in pairs.
__device__ __forceinline__ Pairs8 block_scale_pairs(uint4 hdr) {
  const SixBit sb = unpack_sixbit(hdr.y, hdr.z, hdr.w);
  return scaled_pairs(sb.sc03, sb.sc47, splat_lo(hdr.x));
}

// -32*dmin*m_j of a block in slot order sb_slot: the A operand of the min
// correction, contracted against 32-means.
__device__ __forceinline__ half8 block_neg_dm32(uint4 hdr) {
  const SixBit sb = unpack_sixbit(hdr.y, hdr.z, hdr.w);
  const half2v f = splat_lo(hdr.x >> 16) * half2v{(_Float16)-32.0f, (_Float16)-32.0f};
  const Pairs8 m = scaled_pairs(sb.m03, sb.m47, f);
  half8 r;
  r[0] = m.p02[0]; r[1] = m.p02[1]; r[2] = m.p13[0]; r[3] = m.p13[1];
  r[4] = m.p46[0]; r[5] = m.p46[1]; r[6] = m.p57[0]; r[7] = m.p57[1];
  return r;
}

// s and the offset constant (-1024*s for the low-nibble sub-block 2c, -64*s for
// the high one) of chunk c, from a block's scale pairs.
struct ChunkS {
  half2v s_lo, c_lo, s_hi, c_hi;
};

__device__ __forceinline__ ChunkS chunk_s(const Pairs8& sp, int c) {
  // chunk 0: (s0, s1); 1: (s2, s3); 2: (s4, s5); 3: (s6, s7)
  const half2v lo = (c < 2) ? sp.p02 : sp.p46;
  const half2v hi = (c < 2) ? sp.p13 : sp.p57;
  const _Float16 sl = (c & 1) ? lo[1] : lo[0];
  const _Float16 sh = (c & 1) ? hi[1] : hi[0];
  ChunkS r;
  r.s_lo = half2v{sl, sl};
  r.s_hi = half2v{sh, sh};
  r.c_lo = r.s_lo * half2v{(_Float16)-1024.0f, (_Float16)-1024.0f};
  r.c_hi = r.s_hi * half2v{(_Float16)-64.0f, (_Float16)-64.0f};
  return r;
}

// x[tok[t]][k0 .. k0+256) for the unit's MT rows: four 16-byte pieces per
// thread per 32-row token tile, loaded ahead and written to LDS later.
template <int MT>
struct XPieces {
  static constexpr int THREADS = 64 * FuWaves<MT / 32>::value;
  static constexpr int PIECES = MT * (QK / 8);                   // 16-byte pieces per column
  static constexpr int N = (PIECES + THREADS - 1) / THREADS;     // per thread (the last may be idle)
  uint4 v[N];
  bool live[N];   // false: padding row or past the tile, staged as zeros
};

template <int MT>
__device__ __forceinline__ XPieces<MT> fu_load_x(const _Float16* __restrict__ x, int H,
                                                 const int* __restrict__ tok, int k0) {
  // No branches around the loads (so the compiler's wait counts stay exact):
  // pieces past the tile or of padding rows read token 0's piece, and are
  // zeroed when staged.
  XPieces<MT> r;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int it = 0; it < XPieces<MT>::N; ++it) {
    const int ci = threadIdx.x + XPieces<MT>::THREADS * it;
    // PIECES is a multiple of 64, so whole waves are in or out: a uniform test
    const bool wave_in = wv * 64 + XPieces<MT>::THREADS * it < XPieces<MT>::PIECES;
    const int token = wave_in ? tok[min(ci, XPieces<MT>::PIECES - 1) >> 5] : -1;
    r.live[it] = token >= 0;
    r.v[it] = *reinterpret_cast<const uint4*>(x + (size_t)(token >= 0 ? token : 0) * H + k0 + 8 * (ci & 31));
  }
  return r;
}

// Write staged x pieces into xs in panel order and the 32-means into xsum.
template <int MT, int XS>
__device__ __forceinline__ void fu_store_x(const XPieces<MT>& xp, _Float16* __restrict__ xs,
                                           _Float16* __restrict__ xsum) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int it = 0; it < XPieces<MT>::N; ++it) {
    const int ci = threadIdx.x + XPieces<MT>::THREADS * it;
    // PIECES is a multiple of 64: whole waves are in range or out of it
    if (wv * 64 + XPieces<MT>::THREADS * it >= XPieces<MT>::PIECES) continue;
    const int t = ci >> 5;          // row within the unit
    const int a = ci & 31;          // 8-element group within the super-block column
    const uint4 v = xp.live[it] ? xp.v[it] : make_uint4(0, 0, 0, 0);
    const int c = a >> 3;           // 64-wide panel
    const int kl = (8 * a) & 63;    // position within the panel (multiple of 8)
    // elements e0..e3 -> slots (e0, e2, e1, e3); same for e4..e7
    const uint32_t lo0 = (v.x & 0xFFFFu) | (v.y << 16);       // e0, e2
    const uint32_t lo1 = (v.x >> 16) | (v.y & 0xFFFF0000u);   // e1, e3
    const uint32_t hi0 = (v.z & 0xFFFFu) | (v.w << 16);       // e4, e6
    const uint32_t hi1 = (v.z >> 16) | (v.w & 0xFFFF0000u);   // e5, e7
    _Float16* row = xs + t * XS + c * 64;
    *reinterpret_cast<uint2*>(row + panel_pos(kl)) = make_uint2(lo0, lo1);
    *reinterpret_cast<uint2*>(row + panel_pos(kl + 4)) = make_uint2(hi0, hi1);
    // 32-means: four consecutive pieces (lanes a, a^1, a^2, a^3) form a sub-block
    const half8 hv = __builtin_bit_cast(half8, v);
    float s8 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s8 += (float)hv[e];
    s8 += __shfl_xor(s8, 1, 64);
    s8 += __shfl_xor(s8, 2, 64);
    if ((a & 3) == 0) xsum[t * 8 + sb_slot(a >> 2)] = (_Float16)(s8 * 0.03125f);
  }
}

// One row tile's Q4_K data for a block column: gate and up headers and the
// lane's 64 quant bytes (16 per 64-weight chunk) of each.
struct RowTileData {
  uint4 hg, hu, qg[4], qu[4];
};

__device__ __forceinline__ RowTileData load_row_tile(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                                     size_t blk, int h) {
  RowTileData d;
  const uint8_t* bg = wg + blk * BLOCK_BYTES;
  const uint8_t* bu = wu + blk * BLOCK_BYTES;
  d.hg = *reinterpret_cast<const uint4*>(bg);
  d.hu = *reinterpret_cast<const uint4*>(bu);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    d.qg[c] = *reinterpret_cast<const uint4*>(bg + 16 + 32 * c + 16 * h);
    d.qu[c] = *reinterpret_cast<const uint4*>(bu + 16 + 32 * c + 16 * h);
  }
  return d;
}

// One output tile's W_down data for the chunk: the headers of the blocks the
// chunk touches (from its first block b0) and the lane's 16 quant bytes of each
// of the chunk's 64-wide panels.  OFF = the chunk's first panel within block b0,
// so panel p lives in block (p + OFF) / 4, chunk (p + OFF) % 4: compile-time.
template <int NP, int NB>
struct DownTileData {
  uint4 hdr[NB];
  uint4 qs[NP];
};

template <int NP, int NB, int OFF>
__device__ __forceinline__ DownTileData<NP, NB> load_down_tile(const uint8_t* __restrict__ blk0, int nblk, int npan,
                                                              int h) {
  DownTileData<NP, NB> d;
#pragma unroll
  for (int k = 0; k < NB; ++k)
    d.hdr[k] = (k < nblk) ? *reinterpret_cast<const uint4*>(blk0 + k * BLOCK_BYTES) : make_uint4(0, 0, 0, 0);
  const uint8_t* qb = blk0 + 16 + 16 * h;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k = (p + OFF) >> 2, c = (p + OFF) & 3;
    d.qs[p] = (p < npan) ? *reinterpret_cast<const uint4*>(qb + k * BLOCK_BYTES + 32 * c) : make_uint4(0, 0, 0, 0);
  }
  return d;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int s) {
  return (s == 0) ? q.x : (s == 1) ? q.y : (s == 2) ? q.z : q.w;
}

// Phase 2 of a unit: the down projection of the chunk [r0, r1) over all
// hidden output rows, from the strip in LDS.  OFF = (r0 / 64) % 4.
template <class C, int TT, int ICMAX, int OFF, class Out>
__device__ __forceinline__ void fu_phase2(const uint8_t* __restrict__ wd, int H, int I, const int* __restrict__ tok,
                                          const float* __restrict__ wrow, int chunk, int r0, int r1, int row0,
                                          const Out& out, const _Float16* __restrict__ hs,
                                          const _Float16* __restrict__ hsum, const NibbleK& nk) {
  constexpr int HS = C::HS, HSS = C::HSS;
  constexpr int NB = C::NBMAX;
  constexpr int NP = ICMAX / 64;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int npan = (r1 - r0) / 64;
  const int b0 = r0 >> 8;
  const int nblk = ((r1 - 1) >> 8) - b0 + 1;         // W_down blocks the chunk touches
  const size_t row_bytes = (size_t)(I / QK) * BLOCK_BYTES;
  const int NT = H / 32;                             // output row tiles
  (void)tok;
  (void)wrow;
  (void)chunk;
  (void)row0;
  const uint8_t* blk_base = wd + (size_t)l32 * row_bytes + (size_t)b0 * BLOCK_BYTES;   // row l32 of tile 0

  auto down_tile = [&](DownTileData<NP, NB>& dt, int nt, const uint8_t* nxt) {
    const uint8_t* nq = nxt + 16 + 16 * h;
    float16v acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tt][r] = 0.0f;
    Pairs8 sp[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) sp[k] = block_scale_pairs(dt.hdr[k]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p < npan) {
        const ChunkS cs = chunk_s(sp[(p + OFF) >> 2], (p + OFF) & 3);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8 a = dequant_dword_scaled(dword_of(dt.qs[p], s), cs.s_lo, cs.c_lo, cs.s_hi, cs.c_hi, nk);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const half8 bf = *reinterpret_cast<const half8*>(hs + (tt * 32 + l32) * HS + p * 64 + (2 * s + h) * 8);
            acc[tt] = mfma32(bf, a, acc[tt]);   // strip as A: accumulator rows are tokens
          }
        }
        // panel used up: refill it with the next tile's bytes
        dt.qs[p] = *reinterpret_cast<const uint4*>(nq + ((p + OFF) >> 2) * BLOCK_BYTES + 32 * ((p + OFF) & 3));
      }
    }
    // min correction: lane half h covers block k = 2g + h (block-aligned strip means)
#pragma unroll
    for (int g = 0; g < (NB + 1) / 2; ++g) {
      if (2 * g < nblk) {
        const half8 n0 = block_neg_dm32(dt.hdr[2 * g]);
        half8 n1;
        if (2 * g + 1 < NB) {
          n1 = block_neg_dm32(dt.hdr[2 * g + 1]);   // zero header -> zero operand
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) n1[e] = (_Float16)0.0f;
        }
        const half8 a = (h == 0) ? n0 : n1;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const half8 bf = *reinterpret_cast<const half8*>(hsum + (tt * 32 + l32) * HSS + 16 * g + 8 * h);
          acc[tt] = mfma32(bf, a, acc[tt]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (k < nblk) dt.hdr[k] = *reinterpret_cast<const uint4*>(nxt + k * BLOCK_BYTES);
    // a lane's sixteen accumulators of token tile tt: output row n = 32 nt +
    // (lane % 32), tokens 32 tt + 8 q + 4 (lane / 32) + {0..3} -- whole token
    // quads, which the output policy stores
    out.template store<TT>(acc, nt, l32, h);
  };

  // one rolling tile buffer: each panel's bytes and each header are refilled
  // with the next tile's (nt + WAVES) as soon as they have been consumed
  const size_t tile_step = (size_t)32 * row_bytes;
  if (wave >= NT) return;   // wave-uniform: fewer output tiles than waves
  DownTileData<NP, NB> d = load_down_tile<NP, NB, OFF>(blk_base + (size_t)wave * tile_step, nblk, npan, h);
  for (int nt = wave; nt < NT; nt += C::WAVES) {
    // refills read the next tile of this wave; after the last one, this tile
    // again (in bounds, never used)
    const int nn = (nt + C::WAVES < NT) ? nt + C::WAVES : nt;
    down_tile(d, nt, blk_base + (size_t)nn * tile_step);
  }
}

// One fused unit.  tok/wrow (LDS, MT entries) map unit rows to tokens and
// output weights and must be visible to all threads before the call.  row0 is
// the unit's first output row index handed to the output policy.  All threads
// of the block call this.
template <int TT, int RTW, int ICMAX, class Out>
__device__ __forceinline__ void fused_unit(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                           const uint8_t* __restrict__ wd, int H, int I,
                                           const _Float16* __restrict__ x, const int* __restrict__ tok,
                                           const float* __restrict__ wrow, int chunk, int r0, int r1, int row0,
                                           float inter_scale, const Out& out, FusedSmem<TT, RTW, ICMAX>& sm) {
  using C = FusedCfg<TT, RTW, ICMAX>;
  constexpr int MT = C::MT, XS = C::XS, HS = C::HS, HSS = C::HSS;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int nbH = H / QK;
  const NibbleK nk = nibble_consts();
  const int nrt = (r1 - r0) / 32;                     // row tiles in the chunk
  const int off = (r0 >> 6) & 3;                      // chunk's first panel within its W_down block
  const int rt_per_wave = (nrt + C::WAVES - 1) / C::WAVES;
  const int npass = (rt_per_wave + RTW - 1) / RTW;

  // zero the strip means (slots past the chunk must read as 0)
  for (int i = threadIdx.x; i < MT * HSS; i += C::THREADS) sm.hsum[i] = (_Float16)0.0f;

  // ---------------- phase 1: gate + up, SwiGLU into the LDS strip ----------------
  for (int pass = 0; pass < npass; ++pass) {
    // row tiles of this wave in this pass: rt = wave + C::WAVES*(pass*RTW + i), i < nv
    const int first = pass * RTW;
    const int count_w = (wave < nrt) ? (nrt - wave + C::WAVES - 1) / C::WAVES : 0;   // this wave's row tiles
    const int nv = max(0, min(RTW, count_w - first));
    float16v accg[RTW][TT], accu[RTW][TT];
    half8 dmg[RTW], dmu[RTW];
    half8 xsum_even[TT];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) accg[i][tt][r] = accu[i][tt][r] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dmg[i][e] = dmu[i][e] = (_Float16)0.0f;
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int e = 0; e < 8; ++e) xsum_even[tt][e] = (_Float16)0.0f;

    // byte offset of (row tile i of this pass, block column kb) for this lane;
    // a wave without that row tile gets the chunk's last row tile (an
    // in-bounds address: its loads are never used)
    auto row_blk = [&](int i, int kb) -> const uint8_t* {
      const int rt = min(wave + C::WAVES * (first + i), nrt - 1);
      return (const uint8_t*)0 + ((size_t)(r0 + rt * 32 + l32) * nbH + kb) * BLOCK_BYTES;
    };

    // One super-block column.  D holds this column's weight bytes (loaded one
    // column earlier); each part of D is refilled with the next column's bytes
    // as soon as it has been consumed, so a whole column stays in flight in a
    // single set of registers.
    RowTileData D[RTW];
    auto kstep = [&](int kb) {
      const int buf = kb & 1;
      const bool odd = (kb & 1) != 0;
      const bool pair_end = odd || (kb == nbH - 1);
      // refills read block column kn; on the last step that is the current
      // column again (never used): the loads stay unconditional
      const int kn = (kb + 1 < nbH) ? kb + 1 : kb;
      lds_barrier();   // x[buf] is staged; everyone is done with x[buf ^ 1]
      const XPieces<MT> xp = fu_load_x<MT>(x, H, tok, kn * QK);
      if (!odd) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          xsum_even[tt] = *reinterpret_cast<const half8*>(sm.xsum[buf] + (tt * 32 + l32) * 8);
      }
      // The refill loads are issued by every wave (a wave without a row tile
      // re-reads an in-bounds one), so no branch ever surrounds a load and the
      // compiler's wait counts stay exact; only the arithmetic is skipped.
#pragma unroll
      for (int i = 0; i < RTW; ++i) {
        const bool act = i < nv;   // wave-uniform
        const size_t nb_off = (size_t)(row_blk(i, kn) - (const uint8_t*)0);
        Pairs8 spg, spu;
        if (act) {
          spg = block_scale_pairs(D[i].hg);
          spu = block_scale_pairs(D[i].hu);
          if ((kb & 1) == h) {
            dmg[i] = block_neg_dm32(D[i].hg);
            dmu[i] = block_neg_dm32(D[i].hu);
          }
        }
        D[i].hg = *reinterpret_cast<const uint4*>(wg + nb_off);
        D[i].hu = *reinterpret_cast<const uint4*>(wu + nb_off);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const ChunkS sg = chunk_s(spg, c);
          const ChunkS su = chunk_s(spu, c);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (!act) break;
            const half8 ag = dequant_dword_scaled(dword_of(D[i].qg[c], s), sg.s_lo, sg.c_lo, sg.s_hi, sg.c_hi, nk);
            const half8 au = dequant_dword_scaled(dword_of(D[i].qu[c], s), su.s_lo, su.c_lo, su.s_hi, su.c_hi, nk);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
              const half8 b =
                  *reinterpret_cast<const half8*>(sm.xs[buf] + (tt * 32 + l32) * XS + c * 64 + (2 * s + h) * 8);
              accg[i][tt] = mfma32(ag, b, accg[i][tt]);
              accu[i][tt] = mfma32(au, b, accu[i][tt]);
            }
          }
          // this chunk's bytes are used up: refill them in place
          D[i].qg[c] = *reinterpret_cast<const uint4*>(wg + nb_off + 16 + 32 * c + 16 * h);
          D[i].qu[c] = *reinterpret_cast<const uint4*>(wu + nb_off + 16 + 32 * c + 16 * h);
        }
        if (act && pair_end) {
          // min correction for the block pair (kb-1, kb), or the lone last block:
          // lane half 0 holds the even block's -32*dmin*m and means, half 1 the odd one's
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            half8 b_odd;
#pragma unroll
            for (int e = 0; e < 8; ++e) b_odd[e] = (_Float16)0.0f;
            if (odd) b_odd = *reinterpret_cast<const half8*>(sm.xsum[buf] + (tt * 32 + l32) * 8);
            const half8 b = (h == 0) ? xsum_even[tt] : b_odd;
            accg[i][tt] = mfma32(dmg[i], b, accg[i][tt]);
            accu[i][tt] = mfma32(dmu[i], b, accu[i][tt]);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) dmg[i][e] = dmu[i][e] = (_Float16)0.0f;
        }
      }
      // next column's x into the other buffer (on the last step a harmless
      // rewrite of it: nobody reads that buffer again in this pass)
      fu_store_x<MT, XS>(xp, sm.xs[buf ^ 1], sm.xsum[buf ^ 1]);
    };

    // prologue: x of block column 0 and this wave's weights for it
    lds_barrier();   // the previous pass is done with both x buffers
    {
      const XPieces<MT> xp0 = fu_load_x<MT>(x, H, tok, 0);
      fu_store_x<MT, XS>(xp0, sm.xs[0], sm.xsum[0]);
    }
#pragma unroll
    for (int i = 0; i < RTW; ++i) D[i] = load_row_tile(wg, wu, (size_t)(row_blk(i, 0) - (const uint8_t*)0) / BLOCK_BYTES, h);
    for (int kb = 0; kb < nbH; ++kb) kstep(kb);

    // SwiGLU in registers -> fp16 strip and its 32-row means.  Accumulator r
    // of lane l is (row 8*(r/4) + 4*h + r%4 of the row tile, unit row l%32 of
    // the token tile); four consecutive rows go to four consecutive strip slots.
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
      if (i >= nv) continue;
      const int rt = wave + C::WAVES * (first + i);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        _Float16* srow = sm.hs + (tt * 32 + l32) * HS;
        float rsum = 0.0f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          _Float16 hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = accg[i][tt][4 * q4 + e];
            const float u = accu[i][tt][4 * q4 + e];
            hv[e] = (_Float16)(silu_f32(g) * u * inter_scale);
            rsum += (float)hv[e];
          }
          const int jl = rt * 32 + 8 * q4 + 4 * h;           // multiple of 4
          const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, hv[0]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, hv[2]) << 16);
          const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, hv[1]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, hv[3]) << 16);
          *reinterpret_cast<uint2*>(srow + (jl & ~63) + panel_pos(jl & 63)) = make_uint2(w0, w1);
        }
        rsum += __shfl_xor(rsum, 32, 64);
        // block-aligned slot of chunk sub-block rt: W_down block k = (rt + 2*off) / 8 of
        // the chunk, sub-block j = (rt + 2*off) % 8, stored at 8k + sb_slot(j)
        const int ga = rt + 2 * off;
        if (h == 0) sm.hsum[(tt * 32 + l32) * HSS + 8 * (ga >> 3) + sb_slot(ga & 7)] = (_Float16)(rsum * 0.03125f);
      }
    }
  }
  lds_barrier();   // the strip and its means are complete

  // ---------------- phase 2: down projection over this chunk ----------------
  switch (off) {
    case 0: fu_phase2<C, TT, ICMAX, 0>(wd, H, I, tok, wrow, chunk, r0, r1, row0, out, sm.hs, sm.hsum, nk); break;
    case 1: fu_phase2<C, TT, ICMAX, 1>(wd, H, I, tok, wrow, chunk, r0, r1, row0, out, sm.hs, sm.hsum, nk); break;
    case 2: fu_phase2<C, TT, ICMAX, 2>(wd, H, I, tok, wrow, chunk, r0, r1, row0, out, sm.hs, sm.hsum, nk); break;
    default: fu_phase2<C, TT, ICMAX, 3>(wd, H, I, tok, wrow, chunk, r0, r1, row0, out, sm.hs, sm.hsum, nk); break;
  }
}

}  // namespace zinc
