// Fused Q4_K SwiGLU unit for token tiles of MT = 64 (the dense prefill) or 80
// (the MoE, where one tile then holds a whole expert of up to 80 rows).
//
// A unit is one (MT-token tile, intermediate chunk of at most ICMAX rows)
// pair, run by one workgroup of 12 waves:
//
//   phase 1  gate and up for the chunk: each wave owns a 16-row tile of the
//            chunk and walks the whole hidden dimension one Q4_K super-block
//            column at a time with 16x16x32 fp16 MFMAs (fp32 accumulation).  A
//            lane decodes eight weights per MFMA step (its row r = l%16, octet
//            o = l/16) and that operand meets every 16-token group of the
//            tile, so each decoded weight serves MT tokens.  SwiGLU is applied
//            in registers and the fp16 strip [MT tokens x chunk] lands in LDS.
//   phase 2  the down projection of the strip (fu_phase2, 32x32x16 MFMAs, two
//            or three 32-token tiles per decoded W_down operand).
//
// Weights are decoded in registers on the way into the multiply ("VGPR
// pressure caps the fused RDNA4 prefill GEMM at nine waves", "What the fused
// GEMM actually spends registers on"); the strip never leaves the chip ("Fused
// SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth", "Why this fusion is harder
// than the last one").
//
// Lane layout of phase 1 (as in the decode MFMA kernels): per block a lane
// loads the 16-byte header and the quant runs [16o, +16) and [64+16o, +16);
// MFMA i (0..7) takes dword i%4 of the first run (i < 4) or of the second, whose
// eight slots are weights {0,2,1,3,32,34,33,35} + 64c + 16(o%2) + 4(i%4) of the
// block (c = o/2, or 2 + o/2).  The activation is staged once per call, per
// token, by k_stage_x16 in exactly that order, with the 32-element means the
// -dmin*m term is contracted against (one MFMA per four blocks, lane octet o
// supplying block 4g+o's eight -32*dmin*m values), so a unit copies the rows
// of its tokens into LDS with plain 16-byte moves: a contiguous token range
// for the dense prefill, the routed rows of one expert for the MoE.
#pragma once

#include <type_traits>

#include "fused_core.hpp"

namespace zinc {

typedef float f32x4_16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_16 __attribute__((ext_vector_type(4)));   // native 128-bit vector: no struct copies

__device__ __forceinline__ uint4 as_u4(u32x4_16 v) { return make_uint4(v.x, v.y, v.z, v.w); }

__device__ __forceinline__ f32x4_16 mfma16x16(half8 a, half8 b, f32x4_16 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Staged activation, per token and block column, X16_TP pieces of eight fp16:
// the 32 operand pieces, one piece of padding (in LDS it staggers the banks
// of consecutive tokens), then the token's eight 32-element means (sb_slot
// order).  Layout [token][column][piece]; one extra all-zero token (index M)
// stands in for the padding rows of a tile.
constexpr int X16_ROW = QK + 8;           // halves per token row in LDS
constexpr int X16_TP = X16_ROW / 8 + 1;   // pieces per token and column: 34
constexpr int X16_PIECES = 64 * X16_TP;   // pieces per 64-token column: 2176
constexpr int X16_TP_BYTES = X16_TP * 16; // bytes per token and column

// Operand slot of the eight activations 64c + 4j + {0..3} and 64c + 32 + 4j +
// {0..3} of a block: MFMA i = 4(c/2) + j%4, octet o = 2(c%2) + j/4.
__host__ __device__ constexpr int x16_slot(int c, int j) { return (4 * (c >> 1) + (j & 3)) * 4 + 2 * (c & 1) + (j >> 2); }

template <int ICMAX, int MT_ = 64>
struct Fused16Cfg {
  static constexpr int MT = MT_;                      // tokens per unit: 64, or 80 (the MoE's)
  static constexpr int NGMAX = MT / 16;               // 16-token groups
  static constexpr int MTS = (MT + 31) / 32 * 32;     // strip rows: whole 32-token halves of phase 2
  // activation columns in LDS: four (copy two ahead, a barrier every two
  // blocks) for 64 tokens; three (copy one ahead, a barrier every block) for
  // 80, which is what fits beside the unit's other LDS
  static constexpr int SLOTS = (MT <= 64) ? 4 : 3;
  static constexpr int AHEAD = SLOTS - 2;
  static constexpr int PIECES = MT * X16_TP;          // 16-byte pieces of one staged column
  static constexpr int WAVES = 12;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int XS = X16_ROW;
  static constexpr int HS = ICMAX + 8;                // strip row stride (halves)
  static constexpr int NBMAX = (ICMAX - 64) / 256 + 2;  // W_down blocks a chunk can touch
  static constexpr int HSS = ((8 * NBMAX + 15) / 16) * 16;
  static constexpr int XRING = 8;                     // block columns of means kept (two correction groups)
  static constexpr int NCOPY = (PIECES + THREADS - 1) / THREADS;
  static constexpr int NJUNK = NCOPY * THREADS - PIECES;   // copy slots past the column
  static_assert(MT % 16 == 0 && MT >= 64 && MT <= 80, "64 or 80 tokens per unit");
  static_assert(ICMAX % 64 == 0, "chunks are whole 64-row panels");
  static_assert(ICMAX / 16 <= WAVES, "one 16-row tile per wave");
};

template <int ICMAX, int MT_ = 64>
struct Fused16Smem {
  using C = Fused16Cfg<ICMAX, MT_>;
  union {
    // phase 1: activation columns in operand order, slot = column % SLOTS
    // (the column being read and the ones being staged)
    _Float16 xs[C::SLOTS][C::MT * C::XS];
    // after phase 1 (the same memory): the intermediate strip in panel order
    // and its 32-row means (block-aligned, zero-padded), MTS token rows
    struct {
      _Float16 hs[C::MTS * C::HS];
      _Float16 hsum[C::MTS * C::HSS];
    } s;
  } u;
  _Float16 xm[C::XRING][C::MT * 8];     // 32-means per block column, ring
  float hsum32[C::MT * C::HSS];         // the strip's 32-row sums while phase 1 runs
  _Float16 junk[(C::NJUNK > 0 ? C::NJUNK : 1) * 8];   // stores of the copy slots past a column
  int p2_next;                          // phase 2: next unclaimed output tile
};

// Copy plan of one thread: NCOPY 16-byte pieces per column, piece p = the
// thread's slot = (token row t = p / 34, piece j = p % 34).  src = byte offset
// of the piece in column 0 of the staged activation, dst = its offset (halves)
// in the LDS row area (j < 33), in the means area (j = 33) or in the junk
// area (slots past the column's pieces, which re-read token 0's piece 0).
template <int N>
struct X16Plan {
  uint32_t src[N];
  uint32_t dst[N];
  uint32_t kind[N];   // 0: x row area, 1: means, 2: junk
};

template <class C>
__device__ __forceinline__ X16Plan<C::NCOPY> fu16_plan(const int* __restrict__ tok, int nbH) {
  X16Plan<C::NCOPY> pl;
#pragma unroll
  for (int it = 0; it < C::NCOPY; ++it) {
    const int p = (int)threadIdx.x + C::THREADS * it;
    const int t = p / X16_TP, j = p - t * X16_TP;
    const bool in = p < C::PIECES;
    pl.src[it] = in ? ((uint32_t)tok[t] * nbH * X16_TP + j) * 16u : 0u;
    pl.kind[it] = !in ? 2u : (j < X16_TP - 1) ? 0u : 1u;
    pl.dst[it] = !in ? (uint32_t)(p - C::PIECES) * 8u : (j < X16_TP - 1) ? (uint32_t)(t * X16_ROW + j * 8) : (uint32_t)(t * 8);
  }
  return pl;
}

// One staged column in flight.  No branch surrounds a load (a load whose only
// use sits behind one is sunk to it by the compiler, with a full wait).
template <int N>
struct X16Copy {
  u32x4_16 v[N];
};

// Pieces [A, B) of a thread's share of column kb (the whole share by default).
template <class C, int A = 0, int B = C::NCOPY>
__device__ __forceinline__ void fu16_load_part(const uint8_t* __restrict__ xtok, int kb,
                                               const X16Plan<C::NCOPY>& pl, X16Copy<C::NCOPY>& r) {
  const uint8_t* col = xtok + (size_t)kb * X16_TP_BYTES;
#pragma unroll
  for (int it = A; it < B; ++it) r.v[it] = *reinterpret_cast<const u32x4_16*>(col + pl.src[it]);
}

template <class C>
__device__ __forceinline__ X16Copy<C::NCOPY> fu16_load_col(const uint8_t* __restrict__ xtok, int kb,
                                                           const X16Plan<C::NCOPY>& pl) {
  X16Copy<C::NCOPY> r;
  fu16_load_part<C>(xtok, kb, pl, r);
  return r;
}

template <class C, int A = 0, int B = C::NCOPY>
__device__ __forceinline__ void fu16_store_col(const X16Copy<C::NCOPY>& xc, const X16Plan<C::NCOPY>& pl,
                                               _Float16* __restrict__ xs, _Float16* __restrict__ xm,
                                               _Float16* __restrict__ junk) {
#pragma unroll
  for (int it = A; it < B; ++it) {
    _Float16* base = (pl.kind[it] == 0u) ? xs : (pl.kind[it] == 1u) ? xm : junk;
    *reinterpret_cast<u32x4_16*>(base + pl.dst[it]) = xc.v[it];
  }
}

namespace {

template <int CTRL>
__device__ __forceinline__ float x16_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// The staged activation: for tokens 0..M (token M all zero) and every block
// column, the 34 pieces described at X16_TP.  Grid ((M + 8) / 8, H / 256),
// 256 threads = 8 tokens x 32 pieces; piece (c, j) of a token is
// x[64c + 4j + {0..3}] and x[64c + 32 + 4j + {0..3}] of the column.
// One 256-thread group of the staging: tokens 8 bx .. 8 bx + 7 of column kb,
// thread t of the group.
__device__ __forceinline__ void stage_x16_group(const _Float16* __restrict__ x, int H, int M,
                                                uint8_t* __restrict__ xtok, int bx, int kb, int t) {
  const int nbH = H / QK;
  const int token = bx * 8 + (t >> 5);
  if (token > M) return;   // whole 32-lane groups (the DPP sums below stay within one)
  const int p = t & 31, c = p >> 3, j = p & 7;
  _Float16* col = reinterpret_cast<_Float16*>(xtok + ((size_t)token * nbH + kb) * X16_TP_BYTES);
  uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
  if (token < M) {
    const _Float16* src = x + (size_t)token * H + (size_t)kb * QK + 64 * c + 4 * j;
    lo = *reinterpret_cast<const uint2*>(src);
    hi = *reinterpret_cast<const uint2*>(src + 32);
  }
  // slot order {0,2,1,3} within each group of four
  const uint32_t l0 = (lo.x & 0xFFFFu) | (lo.y << 16), l1 = (lo.x >> 16) | (lo.y & 0xFFFF0000u);
  const uint32_t h0 = (hi.x & 0xFFFFu) | (hi.y << 16), h1 = (hi.x >> 16) | (hi.y & 0xFFFF0000u);
  *reinterpret_cast<uint4*>(col + 8 * x16_slot(c, j)) = make_uint4(l0, l1, h0, h1);
  if (p == 0) *reinterpret_cast<uint4*>(col + QK) = make_uint4(0, 0, 0, 0);
  // 32-means: the eight pieces of one (token, chunk) are eight consecutive
  // lanes; quad sums, then row_shr:4 leaves all eight in lane j == 4
  const half4 lv = __builtin_bit_cast(half4, lo), hv = __builtin_bit_cast(half4, hi);
  float sl = ((float)lv[0] + (float)lv[1]) + ((float)lv[2] + (float)lv[3]);
  float sh = ((float)hv[0] + (float)hv[1]) + ((float)hv[2] + (float)hv[3]);
  sl += x16_dpp<0xB1>(sl);
  sh += x16_dpp<0xB1>(sh);
  sl += x16_dpp<0x4E>(sl);
  sh += x16_dpp<0x4E>(sh);
  sl += x16_dpp<0x114>(sl);
  sh += x16_dpp<0x114>(sh);
  if (j == 4) {
    _Float16* m = col + X16_ROW;
    m[sb_slot(2 * c)] = (_Float16)(sl * 0.03125f);
    m[sb_slot(2 * c + 1)] = (_Float16)(sh * 0.03125f);
  }
}

__global__ __launch_bounds__(256) void k_stage_x16(const _Float16* __restrict__ x, int H, int M,
                                                   uint8_t* __restrict__ xtok) {
  stage_x16_group(x, H, M, xtok, blockIdx.x, blockIdx.y, threadIdx.x);
}

}  // namespace

inline size_t x16_staged_bytes(int M, int H) { return (size_t)(M + 1) * (H / QK) * X16_TP_BYTES; }

// Scale register of chunk CH (0..3) of a W_down block: (1024*s_2CH,
// 64*s_2CH+1), as in lane16_scales.
template <int CH>
__device__ __forceinline__ half2v panel_scales(uint4 hdr) {
  const uint32_t w = (CH < 2) ? sc03_bytes(hdr) : sc47_bytes(hdr);
  const half2v d2 = splat_d(hdr.x);
  return scale_pair(__builtin_amdgcn_perm(0x64646464u, w, sc_pair_sel(2 * (CH & 1))), d2,
                    d2 * half2v{(_Float16)-1024.0f, (_Float16)-1024.0f});
}

// Output policies of phase 2.  store<NTT>() receives the 32-row accumulator
// tiles (NTT of them hold rows) of output rows n = 32 nt + (lane % 32):
// element 4q + e of tile tt belongs to unit row 32 tt + 8 q + 4 (lane / 32) + e.
//
// Dense prefill: fp16 partials at the output scale in the token-quad layout
// P[chunk][t / 4][n][t % 4], so each element group of four is one 8-byte store
// and a store instruction writes two runs of 32 rows x 8 bytes.
struct OutQuads {
  _Float16* P;
  int Mpad;
  int H;
  float scale;
  int chunk;
  int row0;   // the unit's first token
  template <int NTT, int NA>
  __device__ __forceinline__ void store(const float16v (&acc)[NA], int nt, int l32, int h) const {
    const size_t quad_stride = (size_t)H * 4;   // halves per token quad
    _Float16* po = P + ((size_t)chunk * (Mpad / 4) + row0 / 4 + h) * quad_stride + (size_t)(nt * 32 + l32) * 4;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        half4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (_Float16)(acc[tt][4 * q + e] * scale);
        *reinterpret_cast<half4*>(po + (size_t)(8 * tt + 2 * q) * quad_stride) = v;
      }
    }
  }
};

// Formats of W_down in the unit's phase 2: Q4_K (the dense path and the
// default), and the experts' other two, Q5_K and Q5_1.
enum : int { kDownQ4K = 0, kDownQ5K = 1, kDownQ51 = 2 };

// w' = q*s for one quant dword and its fifth bits: the Q4_K operand slots of
// dequant_dword_sc, with the fifth bit of each low nibble taken from bit
// 2*CH of the same byte of QH and that of each high nibble from bit 2*CH + 1,
// OR'ed in above the nibble (1 + q/1024 and 1 + q/64 stay in [1, 2) for
// q < 32).
template <int CH>
__device__ __forceinline__ half8 dequant5_dword_sc(uint32_t Q, uint32_t QH, half2v R, const NibbleK& k) {
  const half2v S_lo = __builtin_shufflevector(R, R, 0, 0), S_hi = __builtin_shufflevector(R, R, 1, 1);
  const uint32_t Q8 = Q >> 8, QH8 = QH >> 8;
  // bytes 0 and 2 (QH) and 1 and 3 (QH8): the low-nibble bit to 4 / 20, the
  // high-nibble bit to 8 / 24 (shifting the odd bytes down first keeps byte
  // 3's high-nibble bit inside the word)
  auto lo_bits = [](uint32_t v) { return (4 - 2 * CH >= 0) ? (v << (4 - 2 * CH)) : (v >> (2 * CH - 4)); };
  auto hi_bits = [](uint32_t v) { return v << (7 - 2 * CH); };
  const half2v p0 =
      __builtin_elementwise_fma(bits_h2((Q & k.lo_mask) | k.lo_magic | (lo_bits(QH) & 0x00100010u)), S_lo, -S_lo);
  const half2v p1 =
      __builtin_elementwise_fma(bits_h2((Q8 & k.lo_mask) | k.lo_magic | (lo_bits(QH8) & 0x00100010u)), S_lo, -S_lo);
  const half2v p2 =
      __builtin_elementwise_fma(bits_h2((Q & k.hi_mask) | k.hi_magic | (hi_bits(QH) & 0x01000100u)), S_hi, -S_hi);
  const half2v p3 =
      __builtin_elementwise_fma(bits_h2((Q8 & k.hi_mask) | k.hi_magic | (hi_bits(QH8) & 0x01000100u)), S_hi, -S_hi);
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Q5_1 quant bytes of a block (bytes 8..23, 8-byte aligned).
__device__ __forceinline__ uint4 load_q51_quants(const uint8_t* blk) {
  const uint2 a = *reinterpret_cast<const uint2*>(blk + 8), b = *reinterpret_cast<const uint2*>(blk + 16);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// One 32-row output tile's W_down data for a lane, per format.
template <int FMT, int NP, int NB>
struct DownTile;

template <int NP, int NB>
struct DownTile<kDownQ4K, NP, NB> {
  using type = DownTileData<NP, NB>;
  template <int OFF>
  __device__ __forceinline__ static type load(const uint8_t* blk0, int nblk, int npan, int h) {
    return load_down_tile<NP, NB, OFF>(blk0, nblk, npan, h);
  }
};

template <int NP, int NB>
struct DownTileQ5K {
  uint4 hdr[NB];   // block headers (Q4_K layout)
  uint4 qh[NB];    // fifth bits of the lane's half: bytes 16 + 16h .. +16
  uint4 qs[NP];    // the lane's 16 quant bytes per panel
};

template <int NP, int NB>
struct DownTile<kDownQ5K, NP, NB> {
  using type = DownTileQ5K<NP, NB>;
  template <int OFF>
  __device__ __forceinline__ static type load(const uint8_t* blk0, int nblk, int npan, int h) {
    type d;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      d.hdr[k] = (k < nblk) ? *reinterpret_cast<const uint4*>(blk0 + k * Q5K_BLOCK_BYTES) : make_uint4(0, 0, 0, 0);
      d.qh[k] = (k < nblk) ? *reinterpret_cast<const uint4*>(blk0 + k * Q5K_BLOCK_BYTES + 16 + 16 * h)
                           : make_uint4(0, 0, 0, 0);
    }
    const uint8_t* qb = blk0 + 48 + 16 * h;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int k = (p + OFF) >> 2, c = (p + OFF) & 3;
      d.qs[p] = (p < npan) ? *reinterpret_cast<const uint4*>(qb + k * Q5K_BLOCK_BYTES + 32 * c) : make_uint4(0, 0, 0, 0);
    }
    return d;
  }
};

template <int NP, int NB>
struct DownTileQ51 {
  uint2 ha[NP], hb[NP];   // per panel, blocks A and B: (d | m << 16, fifth bits)
  uint4 qa[NP], qb[NP];   // their 16 quant bytes
};

template <int NP, int NB>
struct DownTile<kDownQ51, NP, NB> {
  using type = DownTileQ51<NP, NB>;
  // blk0: the row's first block of the chunk's first 256-column group; panel
  // p's blocks are 2 (p + OFF) and the one after it
  template <int OFF>
  __device__ __forceinline__ static type load(const uint8_t* blk0, int nblk, int npan, int h) {
    (void)nblk;
    (void)h;
    type d;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint8_t* a = blk0 + (size_t)(2 * (p + OFF)) * Q5_1_BLOCK_BYTES;
      if (p < npan) {
        d.ha[p] = *reinterpret_cast<const uint2*>(a);
        d.hb[p] = *reinterpret_cast<const uint2*>(a + Q5_1_BLOCK_BYTES);
        d.qa[p] = load_q51_quants(a);
        d.qb[p] = load_q51_quants(a + Q5_1_BLOCK_BYTES);
      } else {
        d.ha[p] = d.hb[p] = make_uint2(0, 0);
        d.qa[p] = d.qb[p] = make_uint4(0, 0, 0, 0);
      }
    }
    return d;
  }
};

// Phase 2 of the unit: the down projection of the chunk [r0, r1) for
// all hidden output rows, from the strip in LDS.  The same contraction as
// fu_phase2 (32x32x16 MFMAs, one decoded W_down operand for both 32-token
// halves, the min correction against the strip's 32-row means), with the
// strip as the A operand: a lane's sixteen accumulators of a token half are
// then one output row n and the tokens 8q + 4(l/32) + {0..3}, which the
// output policy stores.  OFF = (r0 / 64) % 4.
template <class C, int ICMAX, int OFF, int NTT, class Out, int FMT = kDownQ4K>
__device__ __forceinline__ void fu16_phase2(const uint8_t* __restrict__ wd, int H, int I, int r0, int r1,
                                            const Out& out, const _Float16* __restrict__ hs,
                                            const _Float16* __restrict__ hsum, const NibbleK& nk,
                                            int* __restrict__ next_tile) {
  constexpr int HS = C::HS, HSS = C::HSS;
  constexpr int NB = C::NBMAX;
  constexpr int NP = ICMAX / 64;
  constexpr int BB = (FMT == kDownQ5K) ? Q5K_BLOCK_BYTES : BLOCK_BYTES;   // super-block bytes (Q4_K, Q5_K)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int npan = (r1 - r0) / 64;
  const int b0 = r0 >> 8;
  const int nblk = ((r1 - 1) >> 8) - b0 + 1;         // W_down blocks the chunk touches
  // row l32 of tile 0: from the chunk's first 256-column group (Q5_1: its
  // first 32-weight block)
  const size_t row_bytes =
      (FMT == kDownQ51) ? (size_t)(I / 32) * Q5_1_BLOCK_BYTES : (size_t)(I / QK) * BB;
  const int NT = H / 32;                             // output row tiles
  const uint8_t* blk_base = wd + (size_t)l32 * row_bytes +
                            ((FMT == kDownQ51) ? (size_t)b0 * 8 * Q5_1_BLOCK_BYTES : (size_t)b0 * BB);
  using TD = typename DownTile<FMT, NP, NB>::type;

  auto zero_acc = [&](float16v (&acc)[C::MTS / 32]) {
#pragma unroll
    for (int tt = 0; tt < C::MTS / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tt][e] = 0.0f;
  };
  // the strip's 32-row means of block group 2g + h against the lane's
  // min-correction operand
  auto min_mfma = [&](float16v (&acc)[C::MTS / 32], int g, const half8& b) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const half8 a = *reinterpret_cast<const half8*>(hsum + (tt * 32 + l32) * HSS + 16 * g + 8 * h);
      acc[tt] = mfma32(a, b, acc[tt]);
    }
  };
  auto strip_mfma = [&](float16v (&acc)[C::MTS / 32], int P, int s, const half8& b) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const half8 a = *reinterpret_cast<const half8*>(hs + (tt * 32 + l32) * HS + P * 64 + (2 * s + h) * 8);
      acc[tt] = mfma32(a, b, acc[tt]);
    }
  };
  (void)zero_acc;
  (void)min_mfma;
  (void)strip_mfma;

  auto down_tile_q4k = [&](DownTileData<NP, NB>& dt, int nt, const uint8_t* nxt) {
    const uint8_t* nq = nxt + 16 + 16 * h;
    float16v acc[C::MTS / 32];
#pragma unroll
    for (int tt = 0; tt < C::MTS / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tt][e] = 0.0f;
    auto panel = [&](auto pc) {
      constexpr int P = decltype(pc)::value;
      if (P < NP && P < npan) {
        const half2v ps = panel_scales<(P + OFF) & 3>(dt.hdr[(P + OFF) >> 2]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8 b = dequant_dword_sc(dword_of(dt.qs[P], s), ps, nk);
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) {
            const half8 a = *reinterpret_cast<const half8*>(hs + (tt * 32 + l32) * HS + P * 64 + (2 * s + h) * 8);
            acc[tt] = mfma32(a, b, acc[tt]);
          }
        }
        // panel used up: refill it with the next tile's bytes
        dt.qs[P] = *reinterpret_cast<const uint4*>(nq + ((P + OFF) >> 2) * BLOCK_BYTES + 32 * ((P + OFF) & 3));
      }
    };
    panel(std::integral_constant<int, 0>{});
    if constexpr (NP > 1) panel(std::integral_constant<int, 1>{});
    if constexpr (NP > 2) panel(std::integral_constant<int, 2>{});
    if constexpr (NP > 3) panel(std::integral_constant<int, 3>{});
    static_assert(NP <= 4, "panels per chunk");
    // min correction: lane half h covers block 2g + h (block-aligned strip means)
#pragma unroll
    for (int g = 0; g < (NB + 1) / 2; ++g) {
      if (2 * g < nblk) {
        uint4 hd = dt.hdr[2 * g];
        if (2 * g + 1 < NB) {
          if (h) hd = dt.hdr[2 * g + 1];   // zero header past the chunk's blocks -> zero operand
        } else if (h) {
          hd = make_uint4(0, 0, 0, 0);
        }
        const half8 b = block_neg_dm32(hd);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          const half8 a = *reinterpret_cast<const half8*>(hsum + (tt * 32 + l32) * HSS + 16 * g + 8 * h);
          acc[tt] = mfma32(a, b, acc[tt]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (k < nblk) dt.hdr[k] = *reinterpret_cast<const uint4*>(nxt + k * BLOCK_BYTES);
    out.template store<NTT>(acc, nt, l32, h);
  };

  auto down_tile = [&](TD& dt, int nt, const uint8_t* nxt) {
    if constexpr (FMT == kDownQ4K) {
      down_tile_q4k(dt, nt, nxt);
    } else if constexpr (FMT == kDownQ5K) {
      // Q5_K: Q4_K's panels and headers, plus the fifth bits of the lane's
      // half (bytes 16 + 16h .. +16 of each block: bit 2c / 2c+1 for chunk c)
      float16v acc[C::MTS / 32];
      zero_acc(acc);
      const uint8_t* nq = nxt + 48 + 16 * h;
      auto panel = [&](auto pc) {
        constexpr int P = decltype(pc)::value;
        constexpr int CH = (P + OFF) & 3, K = (P + OFF) >> 2;
        if (P < NP && P < npan) {
          const half2v ps = panel_scales<CH>(dt.hdr[K]);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const half8 b = dequant5_dword_sc<CH>(dword_of(dt.qs[P], s), dword_of(dt.qh[K], s), ps, nk);
            strip_mfma(acc, P, s, b);
          }
          dt.qs[P] = *reinterpret_cast<const uint4*>(nq + K * BB + 32 * CH);
        }
      };
      panel(std::integral_constant<int, 0>{});
      if constexpr (NP > 1) panel(std::integral_constant<int, 1>{});
      if constexpr (NP > 2) panel(std::integral_constant<int, 2>{});
      if constexpr (NP > 3) panel(std::integral_constant<int, 3>{});
#pragma unroll
      for (int g = 0; g < (NB + 1) / 2; ++g) {
        if (2 * g < nblk) {
          uint4 hd = dt.hdr[2 * g];
          if (2 * g + 1 < NB) {
            if (h) hd = dt.hdr[2 * g + 1];
          } else if (h) {
            hd = make_uint4(0, 0, 0, 0);
          }
          min_mfma(acc, g, block_neg_dm32(hd));
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (k < nblk) {
          dt.hdr[k] = *reinterpret_cast<const uint4*>(nxt + k * BB);
          dt.qh[k] = *reinterpret_cast<const uint4*>(nxt + k * BB + 16 + 16 * h);
        }
      out.template store<NTT>(acc, nt, l32, h);
    } else {
      // Q5_1: a 64-row panel is two 32-weight blocks A, B; the lane half h
      // takes nibble h of both, repacked into the Q4_K operand order (A's
      // weights 16h + 4s + e in the low-nibble slots, B's in the high ones)
      // with the fifth bits as bits 0 (A) and 1 (B) of each byte, and the
      // blocks' own d as the two scales
      float16v acc[C::MTS / 32];
      zero_acc(acc);
      auto panel = [&](auto pc) {
        constexpr int P = decltype(pc)::value;
        if (P < NP && P < npan) {
          // (1024 * d_A, 64 * d_B): the scale register of dequant5_dword_sc
          const half2v sab = bits_h2((dt.ha[P].x & 0xFFFFu) | (dt.hb[P].x << 16)) *
                             half2v{(_Float16)1024.0f, (_Float16)64.0f};
          const uint32_t fa = dt.ha[P].y >> (16 * h), fb = dt.hb[P].y >> (16 * h);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t A = dword_of(dt.qa[P], s), Bq = dword_of(dt.qb[P], s);
            const uint32_t Q = h ? (((A >> 4) & 0x0F0F0F0Fu) | (Bq & 0xF0F0F0F0u))
                                 : ((A & 0x0F0F0F0Fu) | ((Bq & 0x0F0F0F0Fu) << 4));
            // four fifth bits to bit 0 of four bytes: x * 0x204081 puts bit e at 8e
            const uint32_t QH = ((((fa >> (4 * s)) & 0xFu) * 0x00204081u) & 0x01010101u) |
                                (((((fb >> (4 * s)) & 0xFu) * 0x00204081u) & 0x01010101u) << 1);
            strip_mfma(acc, P, s, dequant5_dword_sc<0>(Q, QH, sab, nk));
          }
          const uint8_t* nb = nxt + (size_t)(2 * (P + OFF)) * Q5_1_BLOCK_BYTES;
          dt.qa[P] = load_q51_quants(nb);
          dt.qb[P] = load_q51_quants(nb + Q5_1_BLOCK_BYTES);
        }
      };
      panel(std::integral_constant<int, 0>{});
      if constexpr (NP > 1) panel(std::integral_constant<int, 1>{});
      if constexpr (NP > 2) panel(std::integral_constant<int, 2>{});
      if constexpr (NP > 3) panel(std::integral_constant<int, 3>{});
      // min term +m per block: +32 m_j against the 32-row means, block j of
      // group 2g + h sits in panel 4(2g + h) + j/2 - OFF (A for even j);
      // blocks outside the chunk's panels meet zero means and take 0
#pragma unroll
      for (int g = 0; g < (NB + 1) / 2; ++g) {
        if (2 * g < nblk) {
          half8 b;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            _Float16 v[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int P = 4 * (2 * g + hh) + j / 2 - OFF;
              v[hh] = (_Float16)0.0f;
              if (P >= 0 && P < NP) {
                if (P < npan) {
                  const uint32_t mb = ((j & 1) ? dt.hb[P < NP ? P : 0].x : dt.ha[P < NP ? P : 0].x) >> 16;
                  v[hh] = (_Float16)32.0f * __builtin_bit_cast(_Float16, (uint16_t)mb);
                }
              }
            }
            b[sb_slot(j)] = h ? v[1] : v[0];
          }
          min_mfma(acc, g, b);
        }
      }
#pragma unroll
      for (int P = 0; P < NP; ++P)
        if (P < npan) {
          const uint8_t* nb = nxt + (size_t)(2 * (P + OFF)) * Q5_1_BLOCK_BYTES;
          dt.ha[P] = *reinterpret_cast<const uint2*>(nb);
          dt.hb[P] = *reinterpret_cast<const uint2*>(nb + Q5_1_BLOCK_BYTES);
        }
      out.template store<NTT>(acc, nt, l32, h);
    }
  };
  // Two rolling tile buffers, so a wave's loads run two tiles ahead: each
  // panel's bytes and each header are refilled with the wave's tile after
  // next as soon as they have been consumed.  Wave w starts on tiles w and
  // w + WAVES; every later tile is claimed from an LDS counter (starting at
  // 2 WAVES) when the tile two before it starts, so waves that issue faster
  // (the scheduler favours older waves) take more tiles and the unit's
  // waves finish together.  Claims only grow, so a wave's tiles ascend and
  // the first one past the last tile ends its loop.
  constexpr int W = C::WAVES;
  const size_t tile_step = (size_t)32 * row_bytes;
  if (wave >= NT) return;   // wave-uniform: fewer output tiles than waves
  // loads past the last tile re-read the last one (in bounds, never used)
  auto clamp_tile = [&](int t) { return t < NT ? t : NT - 1; };
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(next_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int t0 = wave, t1 = wave + W;
  TD d0 = DownTile<FMT, NP, NB>::template load<OFF>(blk_base + (size_t)t0 * tile_step, nblk, npan, h);
  TD d1 = DownTile<FMT, NP, NB>::template load<OFF>(blk_base + (size_t)clamp_tile(t1) * tile_step, nblk, npan, h);
  while (t0 < NT) {
    const int t2 = claim();
    down_tile(d0, t0, blk_base + (size_t)clamp_tile(t2) * tile_step);
    if (t1 >= NT) break;
    const int t3 = claim();
    down_tile(d1, t1, blk_base + (size_t)clamp_tile(t3) * tile_step);
    t0 = t2;
    t1 = t3;
  }
}

// What a unit runs: the fused form, or one half of the staged comparison
// baseline, in which the intermediate crosses device memory as the unfused
// dataflow of "The MLP is two trips up to a wider width" has it (gate and up
// written and read back, the intermediate written and read back):
//   kUnitGateUp  phase 1 only; G and U stored as fp16 [M x I] (token-major)
//   kUnitDown    no phase 1; the strip is read from the fp16 intermediate
//                [M x I], then phase 2 as in the fused form
enum : int { kUnitFused = 0, kUnitGateUp = 1, kUnitDown = 2 };

struct StagedIO {
  _Float16* g = nullptr;          // kUnitGateUp outputs
  _Float16* u = nullptr;
  const _Float16* h = nullptr;    // kUnitDown input
  int t0 = 0;                     // the unit's first token
};

// One fused MT-token unit.  xtok = the staged activation (k_stage_x16); tok =
// the unit's MT token indices (LDS, visible to all threads before the call;
// the zero token M for padding rows); rows = how many of them are real (1..MT,
// the rest are padding: 16-token groups and 32-token halves wholly past it
// are skipped); out = the phase-2 output policy.
template <int ICMAX, class Out, int MT_, int MODE = kUnitFused, int FMT = kDownQ4K>
__device__ __forceinline__ void fused_unit16(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                             const uint8_t* __restrict__ wd, int H, int I,
                                             const uint8_t* __restrict__ xtok, const int* __restrict__ tok,
                                             int rows, int r0, int r1, float inter_scale, const Out& out,
                                             Fused16Smem<ICMAX, MT_>& sm, StagedIO sio = StagedIO{}) {
  using C = Fused16Cfg<ICMAX, MT_>;
  constexpr int NGMAX = C::NGMAX, SLOTS = C::SLOTS, AHEAD = C::AHEAD, MTS = C::MTS;
  constexpr int XS = C::XS, HS = C::HS, HSS = C::HSS, MT = C::MT;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, o = lane >> 4, sel = (o >> 1) & 1;
  const uint32_t psel = sc_pair_sel(2 * sel);   // lane16_scales
  const int nbH = H / QK;
  const size_t rowb = (size_t)nbH * BLOCK_BYTES;
  const NibbleK nk = nibble_consts_s();
  const int nrt = (r1 - r0) / 16;                 // 16-row tiles in the chunk (<= WAVES)
  const int off = (r0 >> 6) & 3;                  // chunk's first panel within its W_down block
  const int rt = wave;
  const bool act = rt < nrt;                      // wave-uniform
  const int rtc = act ? rt : nrt - 1;             // idle waves stream an in-bounds tile (never used)
  // weight rows as 32-bit offsets from the (uniform) matrix bases, so loads
  // take the scalar-base form
  const uint32_t wrow_off = (uint32_t)((size_t)(r0 + rtc * 16 + r) * rowb);

  for (int i = threadIdx.x; i < MT * HSS; i += C::THREADS) sm.hsum32[i] = 0.0f;
  // the means ring: octets past the last block of a short final group read
  // slots never written in this unit; zero operands need finite partners
  for (int i = threadIdx.x; i < C::XRING * MT * 8; i += C::THREADS) (&sm.xm[0][0])[i] = (_Float16)0.0f;

  f32x4_16 accg[NGMAX], accu[NGMAX];
#pragma unroll
  for (int g = 0; g < NGMAX; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) accg[g][e] = accu[g][e] = 0.0f;

  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using IG = std::integral_constant<int, NGMAX>;

  if constexpr (MODE != kUnitDown) {
  // prologue: columns 0 .. AHEAD-1 staged
  const X16Plan<C::NCOPY> xplan = fu16_plan<C>(tok, nbH);
  {
    const X16Copy<C::NCOPY> x0 = fu16_load_col<C>(xtok, 0, xplan);
    const int c1 = nbH > 1 ? 1 : 0;
    if constexpr (AHEAD == 2) {
      const X16Copy<C::NCOPY> x1 = fu16_load_col<C>(xtok, c1, xplan);
      lds_barrier();   // ring zeroed before the means land in it
      fu16_store_col<C>(x0, xplan, sm.u.xs[0], sm.xm[0], sm.junk);
      fu16_store_col<C>(x1, xplan, sm.u.xs[1], sm.xm[c1], sm.junk);
    } else {
      lds_barrier();
      fu16_store_col<C>(x0, xplan, sm.u.xs[0], sm.xm[0], sm.junk);
    }
  }

  // The column loop, once for waves with a row tile (ACT) and once for idle
  // waves, which only help stage the activation; both meet the same barriers.
  //
  // Staging.  Column c is copied into slot c % SLOTS during block c - AHEAD
  // (MFMA step 4), SLOTS = AHEAD + 2.  A barrier at the top of every AHEAD-th
  // block publishes the columns copied before it; the slot written in block
  // kb held column kb - 2, which every wave finished reading before the last
  // barrier.
  //
  // Pipeline.  Within a block an active wave's MFMA steps are
  // software-pipelined: the B operands and the decoded A operands of step i+1
  // are fetched while step i's eight MFMAs run.
  auto column_loop = [&](auto act_tag, auto ng_tag) {
    constexpr bool ACT = decltype(act_tag)::value;
    constexpr int NG = decltype(ng_tag)::value;   // 16-token groups holding rows
    constexpr int VPM = (NG >= 3) ? 3 : (NG == 2) ? 5 : 9;   // decode VALU per MFMA slot
    u32x4_16 hg, hu, qg0, qu0, qg1, qu1;
    u32x4_16 cg = {0u, 0u, 0u, 0u}, cu = {0u, 0u, 0u, 0u};   // headers for the min correction
    if constexpr (ACT) {
      hg = *reinterpret_cast<const u32x4_16*>(wg + wrow_off);
      hu = *reinterpret_cast<const u32x4_16*>(wu + wrow_off);
      qg0 = *reinterpret_cast<const u32x4_16*>(wg + (wrow_off + 16 + 16 * o));
      qu0 = *reinterpret_cast<const u32x4_16*>(wu + (wrow_off + 16 + 16 * o));
      qg1 = *reinterpret_cast<const u32x4_16*>(wg + (wrow_off + 80 + 16 * o));
      qu1 = *reinterpret_cast<const u32x4_16*>(wu + (wrow_off + 80 + 16 * o));
    }
    const int xlane = r * XS + o * 8;   // lane's token r of group 0, octet o
    for (int kb = 0; kb < nbH; ++kb) {
      // weight refills read column kn, the staging copy column kx; past the
      // end they re-read the last column (never used), so no branch ever
      // surrounds a load
      const int kn = (kb + 1 < nbH) ? kb + 1 : kb;
      const int kx = (kb + AHEAD < nbH) ? kb + AHEAD : nbH - 1;
      const uint32_t noff = wrow_off + (uint32_t)kn * BLOCK_BYTES;
      if (kb % AHEAD == 0) lds_barrier();
      // an 80-token column is copied in two halves (the second loaded once
      // the first is stored), which keeps half the copy registers live
      constexpr bool SPLIT = C::NCOPY >= 4;
      constexpr int HALF = SPLIT ? (C::NCOPY + 1) / 2 : C::NCOPY;
      X16Copy<C::NCOPY> xc;
      fu16_load_part<C, 0, HALF>(xtok, kx, xplan, xc);
      _Float16* const xs_next = sm.u.xs[(kb + AHEAD) % SLOTS];
      _Float16* const xm_next = sm.xm[kx & (C::XRING - 1)];
      if constexpr (ACT) {
        const Lane16S sg = lane16_scales(as_u4(hg), psel), su = lane16_scales(as_u4(hu), psel);
        // octet o keeps block (kb & ~3) + o's headers for the correction
        const bool mine = o == (kb & 3);
        cg = mine ? hg : cg;
        cu = mine ? hu : cu;
        hg = *reinterpret_cast<const u32x4_16*>(wg + noff);
        hu = *reinterpret_cast<const u32x4_16*>(wu + noff);
        // keep the column's loads here, a whole block step ahead of their use
        // (left alone, the scheduler sinks them below the MFMAs)
        __builtin_amdgcn_sched_barrier(0);
        const _Float16* xb = sm.u.xs[kb % SLOTS] + xlane;
        auto load_b = [&](int i, half8 (&b)[NGMAX]) {
#pragma unroll
          for (int g = 0; g < NG; ++g) b[g] = *reinterpret_cast<const half8*>(xb + g * 16 * XS + i * 32);
        };
        auto decode = [&](int i, half8& ag, half8& au) {
          const uint32_t qg = (i < 4) ? qg0[i & 3] : qg1[i & 3];
          const uint32_t qu = (i < 4) ? qu0[i & 3] : qu1[i & 3];
          ag = dequant_dword_sc(qg, (i < 4) ? sg.r0 : sg.r1, nk);
          au = dequant_dword_sc(qu, (i < 4) ? su.r0 : su.r1, nk);
        };
        // Five token groups leave no room for a second set of B operands:
        // there each group's B is refilled in place right after its two
        // MFMAs, a whole step ahead of its next use.
        constexpr bool INPLACE = NG > 4;
        half8 bc[NGMAX], bn[INPLACE ? 1 : NGMAX], agc, auc, agn, aun;
        load_b(0, bc);
        decode(0, agc, auc);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i < 7) {
            if constexpr (!INPLACE) load_b(i + 1, bn);
            decode(i + 1, agn, aun);
          }
          if (i == 3) {   // the first quant run is decoded: refill it in place
            qg0 = *reinterpret_cast<const u32x4_16*>(wg + (noff + 16 + 16 * o));
            qu0 = *reinterpret_cast<const u32x4_16*>(wu + (noff + 16 + 16 * o));
            __builtin_amdgcn_sched_barrier(0);
          }
          // column kx into its slot and the means ring: the last barrier
          // released that slot, and the ring slot written is none of the
          // four the corrections of blocks up to kb+1 read (past the end a
          // rewrite of data nobody reads again, or of the same values)
          if (i == 4) {
            fu16_store_col<C, 0, HALF>(xc, xplan, xs_next, xm_next, sm.junk);
            if constexpr (SPLIT) fu16_load_part<C, HALF, C::NCOPY>(xtok, kx, xplan, xc);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (SPLIT) {
            if (i == 7) {
              fu16_store_col<C, HALF, C::NCOPY>(xc, xplan, xs_next, xm_next, sm.junk);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if (i == 6) {   // and the second
            qg1 = *reinterpret_cast<const u32x4_16*>(wg + (noff + 80 + 16 * o));
            qu1 = *reinterpret_cast<const u32x4_16*>(wu + (noff + 80 + 16 * o));
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            accg[g] = mfma16x16(agc, bc[g], accg[g]);
            accu[g] = mfma16x16(auc, bc[g], accu[g]);
            if constexpr (INPLACE) {
              if (i < 7) bc[g] = *reinterpret_cast<const half8*>(xb + g * 16 * XS + (i + 1) * 32);
            }
          }
          if (i < 7) {
            if constexpr (!INPLACE) {
#pragma unroll
              for (int g = 0; g < NG; ++g) bc[g] = bn[g];
            }
            agc = agn;
            auc = aun;
          }
          if constexpr (INPLACE) {
            // issue order: per group its two MFMAs with decode VALU work
            // between them, then that group's B refill
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
          } else {
            // issue order of the step: the next B reads, then the MFMAs with
            // the next decode's VALU work threaded between them
            __builtin_amdgcn_sched_group_barrier(0x100, NG, 0);
#pragma unroll
            for (int k = 0; k < 2 * NG; ++k) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
            }
          }
        }
        // min correction once per four blocks (or at the last): octet o holds
        // block (kb & ~3) + o's headers (zero past the last block: zero
        // operand), contracted with that block's means
        if ((kb & 3) == 3 || kb == nbH - 1) {
          const half8 dmg = block_neg_dm32(as_u4(cg)), dmu = block_neg_dm32(as_u4(cu));
          const _Float16* mb = sm.xm[((kb & ~3) + o) & (C::XRING - 1)] + r * 8;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const half8 b = *reinterpret_cast<const half8*>(mb + g * 16 * 8);
            accg[g] = mfma16x16(dmg, b, accg[g]);
            accu[g] = mfma16x16(dmu, b, accu[g]);
          }
          cg = u32x4_16{0u, 0u, 0u, 0u};
          cu = u32x4_16{0u, 0u, 0u, 0u};
        }
      } else {
        if constexpr (SPLIT) fu16_load_part<C, HALF, C::NCOPY>(xtok, kx, xplan, xc);
        fu16_store_col<C>(xc, xplan, xs_next, xm_next, sm.junk);
      }
    }
  };
  // token groups past the unit's rows stay zero and are skipped
  const int ng = (rows + 15) >> 4;   // uniform, 1..NGMAX
  if (!act)
    column_loop(std::false_type{}, IG{});
  else if (ng >= NGMAX)
    column_loop(std::true_type{}, IG{});
  else if (NGMAX > 4 && ng == 4)
    column_loop(std::true_type{}, I4{});
  else if (ng == 3)
    column_loop(std::true_type{}, I3{});
  else if (ng == 2)
    column_loop(std::true_type{}, I2{});
  else
    column_loop(std::true_type{}, I1{});
  }   // MODE != kUnitDown
  if constexpr (MODE == kUnitGateUp) {
    // staged baseline: G and U to device memory; accumulator e of lane (r, o)
    // in group g is row 4o + e of the wave's tile, token 16g + r
    if (act) {
      const int n = r0 + rt * 16 + 4 * o;
#pragma unroll
      for (int g = 0; g < NGMAX; ++g) {
        const int t = g * 16 + r;
        if (t < rows) {
          half4 gv, uv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[e] = (_Float16)accg[g][e];
            uv[e] = (_Float16)accu[g][e];
          }
          *reinterpret_cast<half4*>(sio.g + (size_t)(sio.t0 + t) * I + n) = gv;
          *reinterpret_cast<half4*>(sio.u + (size_t)(sio.t0 + t) * I + n) = uv;
        }
      }
    }
    return;
  }
  lds_barrier();   // the strip below overwrites the activation slots
  if constexpr (MTS > MT) {   // token rows past the unit's MT: a zero strip (phase 2 reads whole 32-token halves)
    for (int i = threadIdx.x; i < (MTS - MT) * HS; i += C::THREADS) sm.u.s.hs[MT * HS + i] = (_Float16)0.0f;
  }

  if constexpr (MODE == kUnitDown) {
    // staged baseline: the strip and its 32-row sums from the intermediate in
    // device memory (zero rows past the unit's tokens)
    // one thread per (token, 32-row group): the group's sum is taken in a
    // fixed order, so the staged call's result does not depend on scheduling
    const int n32 = (r1 - r0) >> 5;
    for (int idx = threadIdx.x; idx < MT * n32; idx += C::THREADS) {
      const int t = idx / n32, j32 = (idx - t * n32) * 32;
      float s32 = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int jl = j32 + 4 * k;
        uint2 v = make_uint2(0u, 0u);
        if (t < rows) v = *reinterpret_cast<const uint2*>(sio.h + (size_t)(sio.t0 + t) * I + r0 + jl);
        const half4 hv = __builtin_bit_cast(half4, v);
        const uint32_t w0 = (v.x & 0xFFFFu) | (v.y << 16);
        const uint32_t w1 = (v.x >> 16) | (v.y & 0xFFFF0000u);
        *reinterpret_cast<uint2*>(sm.u.s.hs + t * HS + (jl & ~63) + panel_pos(jl & 63)) = make_uint2(w0, w1);
        s32 += ((float)hv[0] + (float)hv[1]) + ((float)hv[2] + (float)hv[3]);
      }
      const int jg = off * 64 + j32;
      sm.hsum32[t * HSS + 8 * (jg >> 8) + sb_slot((jg >> 5) & 7)] = s32;
    }
  }
  // SwiGLU in registers -> fp16 strip (panel order) and the 32-row sums.
  // Accumulator e of lane (r, o) in group g: row 4o + e of the tile, token 16g + r.
  if (MODE == kUnitFused && act) {
    const int jl = rt * 16 + 4 * o;                     // chunk-local row, multiple of 4
    const int jg = off * 64 + rt * 16;                  // row from the start of the chunk's first W_down block
    const int slot = 8 * (jg >> 8) + sb_slot((jg >> 5) & 7);
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) {
      _Float16 hv[4];
      float s4 = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[e] = (_Float16)(silu_f32(accg[g][e]) * accu[g][e] * inter_scale);
        s4 += (float)hv[e];
      }
      const int t = g * 16 + r;
      // rows jl..jl+3 sit at panel_pos(jl % 64) + {0, 2, 1, 3}
      const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, hv[0]) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, hv[2]) << 16);
      const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, hv[1]) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, hv[3]) << 16);
      *reinterpret_cast<uint2*>(sm.u.s.hs + t * HS + (jl & ~63) + panel_pos(jl & 63)) = make_uint2(w0, w1);
      // the tile's 16 rows of token t: octets of lanes r, r+16, r+32, r+48
      s4 += __shfl_xor(s4, 16, 64);
      s4 += __shfl_xor(s4, 32, 64);
      if (o == 0) atomicAdd(&sm.hsum32[t * HSS + slot], s4);
    }
  }
  if (threadIdx.x == 0) sm.p2_next = 2 * C::WAVES;
  lds_barrier();   // strip and sums complete
  for (int i = threadIdx.x; i < MTS * HSS; i += C::THREADS)
    sm.u.s.hsum[i] = (i < MT * HSS) ? (_Float16)(sm.hsum32[i] * 0.03125f) : (_Float16)0.0f;
  lds_barrier();

  // ---------------- phase 2: down projection over this chunk ----------------
  auto phase2 = [&](auto ntt_tag) {
    constexpr int NTT = decltype(ntt_tag)::value;
    switch (off) {
      case 0: fu16_phase2<C, ICMAX, 0, NTT, Out, FMT>(wd, H, I, r0, r1, out, sm.u.s.hs, sm.u.s.hsum, nk, &sm.p2_next); break;
      case 1: fu16_phase2<C, ICMAX, 1, NTT, Out, FMT>(wd, H, I, r0, r1, out, sm.u.s.hs, sm.u.s.hsum, nk, &sm.p2_next); break;
      case 2: fu16_phase2<C, ICMAX, 2, NTT, Out, FMT>(wd, H, I, r0, r1, out, sm.u.s.hs, sm.u.s.hsum, nk, &sm.p2_next); break;
      default: fu16_phase2<C, ICMAX, 3, NTT, Out, FMT>(wd, H, I, r0, r1, out, sm.u.s.hs, sm.u.s.hsum, nk, &sm.p2_next); break;
    }
  };
  if constexpr (MTS > 64) {
    if (rows > 64) {
      phase2(std::integral_constant<int, 3>{});
      return;
    }
  }
  if (rows > 32)
    phase2(I2{});
  else
    phase2(I1{});
}

}  // namespace zinc
