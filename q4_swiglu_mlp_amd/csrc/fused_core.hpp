// The fused Q4_K SwiGLU work unit shared by the dense prefill kernel and the
// batched-expert kernel.
//
// One unit = (MT rows of activations) x (IC intermediate rows of one expert).
// The rows are tokens given by a per-unit map row -> token (dense prefill: a
// contiguous tile; MoE: the (token, slot) pairs routed to one expert), each
// with an output weight (1 for dense, the mixing weight for MoE).
//   Phase 1 (gate+up): for every 256-wide super-block column of the hidden
//     dimension the unit's x rows are staged in LDS (fp16, panel_pos order) and
//     each wave decodes the gate and up Q4_K blocks of its rows in registers
//     straight into fp16 MFMA operands; 32x32x16 MFMAs accumulate in fp32.
//     SwiGLU is applied to the accumulators in registers and the result, scaled
//     by 2^-inter_shift, is written as fp16 into the LDS strip [MT x IC]: the
//     intermediate never leaves the chip.
//   Phase 2 (down): the strip is the B operand of the down projection over the
//     unit's IC columns of W_down; each 32-row tile of the hidden output is
//     produced from the strip held in LDS, scaled by the row's output weight and
//     added in fp32 into Y32t [hidden x Mpad] with hardware float atomics (the
//     reduction over intermediate chunks and, for MoE, over a token's experts).
//
// This is the dataflow of "Fused SwiGLU MLP: ZINC RDNA4 Down-Projection
// Bandwidth" ("Why this fusion is harder than the last one": compute a block of
// the intermediate for a set of columns, stage it in the LDS, feed the down
// projection's accumulation for those columns, advance; the fused row of
// Fig. 1), with the dequant fused into the producer GEMM as on "VGPR pressure
// caps the fused RDNA4 prefill GEMM at nine waves".  The RDNA4 16x16 WMMA
// tiling there is replaced by gfx950 32x32x16 MFMA on 64-wide waves.
#pragma once

#include "q4k_device.hpp"

namespace zinc {

constexpr int FU_WAVES = 4;
constexpr int FU_THREADS = 64 * FU_WAVES;

template <int TT, int RT>
struct FusedCfg {
  static constexpr int MT = 32 * TT;             // activation rows per unit
  static constexpr int IC = 32 * RT * FU_WAVES;  // intermediate rows per unit
  static constexpr int XS = QK + 8;              // x stage row stride (halves), padded
  static constexpr int HS = IC + 8;              // strip row stride (halves), padded
};

// Stage x[tok[t]][k0 .. k0+256) for the unit's MT rows into xs in panel order;
// rows whose token is negative are zero.
template <int MT, int XS>
__device__ __forceinline__ void fu_stage_x(_Float16* __restrict__ xs, const _Float16* __restrict__ x, int H,
                                           const int* __restrict__ tok, int k0) {
  constexpr int PIECES = MT * (QK / 8);  // 16-byte pieces
#pragma unroll
  for (int it = 0; it < PIECES / FU_THREADS; ++it) {
    const int ci = threadIdx.x + FU_THREADS * it;
    const int t = ci >> 5;          // row within the unit
    const int a = ci & 31;          // 8-element group within the super-block column
    const int token = tok[t];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (token >= 0) v = *reinterpret_cast<const uint4*>(x + (size_t)token * H + k0 + 8 * a);
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
  }
}

// One fused unit.  tok/wrow (LDS, MT entries) map unit rows to tokens and
// output weights; must be visible to all threads before the call.  xs, hs are
// the LDS stage and strip.  All threads of the block call this.
template <int TT, int RT>
__device__ __forceinline__ void fused_unit(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                           const uint8_t* __restrict__ wd, int H, int I,
                                           const _Float16* __restrict__ x, const int* __restrict__ tok,
                                           const float* __restrict__ wrow, int chunk, float* __restrict__ y32t,
                                           int Mpad, float inter_scale, _Float16* __restrict__ xs,
                                           _Float16* __restrict__ hs) {
  using C = FusedCfg<TT, RT>;
  constexpr int MT = C::MT, IC = C::IC, XS = C::XS, HS = C::HS;
  (void)MT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int nbH = H / QK;
  const int jbase = chunk * IC;

  // ---------------- phase 1: gate + up, SwiGLU into the LDS strip ----------------
  float16v accg[RT][TT], accu[RT][TT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) accg[rt][tt][r] = accu[rt][tt][r] = 0.0f;

  for (int kb = 0; kb < nbH; ++kb) {
    __syncthreads();
    fu_stage_x<C::MT, XS>(xs, x, H, tok, kb * QK);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rbase = jbase + (wave * RT + rt) * 32;
      if (rbase >= I) continue;   // wave-uniform: row tile past the last intermediate row
      const int row = rbase + l32;
      const uint8_t* bg = wg + ((size_t)row * nbH + kb) * BLOCK_BYTES;
      const uint8_t* bu = wu + ((size_t)row * nbH + kb) * BLOCK_BYTES;
      const BlockScalesF16 sg = block_scales_f16(*reinterpret_cast<const uint4*>(bg));
      const BlockScalesF16 su = block_scales_f16(*reinterpret_cast<const uint4*>(bu));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 qg = *reinterpret_cast<const uint4*>(bg + 16 + 32 * c + 16 * h);
        const uint4 qu = *reinterpret_cast<const uint4*>(bu + 16 + 32 * c + 16 * h);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t dg = (s == 0) ? qg.x : (s == 1) ? qg.y : (s == 2) ? qg.z : qg.w;
          const uint32_t du = (s == 0) ? qu.x : (s == 1) ? qu.y : (s == 2) ? qu.z : qu.w;
          const half8 ag = dequant_dword_f16(dg, sg.s[2 * c], sg.dm[2 * c], sg.s[2 * c + 1], sg.dm[2 * c + 1]);
          const half8 au = dequant_dword_f16(du, su.s[2 * c], su.dm[2 * c], su.s[2 * c + 1], su.dm[2 * c + 1]);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const half8 b = *reinterpret_cast<const half8*>(xs + (tt * 32 + l32) * XS + c * 64 + (2 * s + h) * 8);
            accg[rt][tt] = mfma32(ag, b, accg[rt][tt]);
            accu[rt][tt] = mfma32(au, b, accu[rt][tt]);
          }
        }
      }
    }
  }

  // SwiGLU in registers -> fp16 strip.  Accumulator r of lane l is
  // (row 8*(r/4) + 4*h + r%4 of the row tile, unit row l%32 of the token tile);
  // each group of four consecutive rows goes to four consecutive strip slots.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rtile = (wave * RT + rt) * 32;
    if (jbase + rtile >= I) continue;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      _Float16* srow = hs + (tt * 32 + l32) * HS;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        _Float16 hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = accg[rt][tt][4 * q4 + e];
          const float u = accu[rt][tt][4 * q4 + e];
          hv[e] = (_Float16)(silu_f32(g) * u * inter_scale);
        }
        const int jl = rtile + 8 * q4 + 4 * h;           // multiple of 4
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, hv[0]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hv[2]) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, hv[1]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hv[3]) << 16);
        *reinterpret_cast<uint2*>(srow + (jl & ~63) + panel_pos(jl & 63)) = make_uint2(w0, w1);
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: down projection over this chunk ----------------
  const int nbI = I / QK;
  const int jcount = min(IC, I - jbase);     // multiple of 128
  const int npan = jcount / 64;
  int tokc[TT];
  float wc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    tokc[tt] = tok[tt * 32 + l32];
    wc[tt] = wrow[tt * 32 + l32];
  }
  for (int nt = wave; nt < H / 32; nt += FU_WAVES) {
    float16v acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tt][r] = 0.0f;
    const uint8_t* rowp = wd + (size_t)(nt * 32 + l32) * nbI * BLOCK_BYTES;
    for (int p = 0; p < npan; ++p) {
      const int j0 = jbase + 64 * p;
      const int b = j0 >> 8, c = (j0 >> 6) & 3;
      const uint8_t* bp = rowp + (size_t)b * BLOCK_BYTES;
      const ChunkScalesF16 sc = chunk_scales_f16(*reinterpret_cast<const uint4*>(bp), c);
      const uint4 qd = *reinterpret_cast<const uint4*>(bp + 16 + 32 * c + 16 * h);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t dw = (s == 0) ? qd.x : (s == 1) ? qd.y : (s == 2) ? qd.z : qd.w;
        const half8 a = dequant_dword_f16(dw, sc.s_lo, sc.dm_lo, sc.s_hi, sc.dm_hi);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const half8 bf = *reinterpret_cast<const half8*>(hs + (tt * 32 + l32) * HS + p * 64 + (2 * s + h) * 8);
          acc[tt] = mfma32(a, bf, acc[tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tokc[tt] >= 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = nt * 32 + mfma32_row(r, lane);
          unsafeAtomicAdd(y32t + (size_t)n * Mpad + tokc[tt], wc[tt] * acc[tt][r]);
        }
      }
    }
  }
}

}  // namespace zinc
