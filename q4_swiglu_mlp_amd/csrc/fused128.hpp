// Fused Q4_K SwiGLU unit for 128-token tiles: the large-prefill form of the
// 64-token unit of fused16.hpp, with every decoded weight serving twice the
// tokens.
//
// Why.  On this chip the dequant VALU work of a fused unit does not hide behind
// its MFMAs: a SIMD spends roughly 16 cycles per 16x16x32 MFMA plus the issue
// time of every VALU instruction.  Decoding eight weights costs about nine
// VALU instructions whatever the tile, so the decode cost per flop falls with
// the tokens that share each decoded operand: a wave here owns 16 rows and
// eight 16-token groups, so one decoded A operand feeds 16 MFMAs (8 groups x
// gate/up) instead of 8.
//
// A unit is one (128-token tile, chunk of up to NPASS x 128 intermediate rows)
// pair, run by one workgroup of 8 waves (two per SIMD: the accumulators of 8
// groups x gate/up take 64 registers):
//
//   phase 1  NPASS passes of 128 rows.  In each, wave w owns rows 16w..16w+15
//            of the pass and walks the hidden dimension one Q4_K block column at
//            a time: the same lane layout, decode and min correction as the
//            64-token unit.  SwiGLU in registers; the pass's fp16 strip columns
//            land in LDS.  Passes keep the chunk wide (fewer split-K partials,
//            whose size is tokens x hidden per chunk) while a wave still holds
//            accumulators for only 16 rows.
//   phase 2  the down projection of the [128 x chunk] strip (fu16_phase2, four
//            32-token halves per decoded W_down operand).
//
// The activation (staged once per call by k_stage_x16, operand order) is
// copied into LDS half a block column at a time (128 of its 256 K values, 64
// KB per 128 tokens would not fit twice beside the strip): two slots, slot 0
// for MFMA steps 0-3 and slot 1 for steps 4-7.  A barrier at the top of step 3
// publishes slot 1 and frees slot 0; one at the top of step 7 publishes slot 0
// (the next column's first half) and frees slot 1.  Each half is loaded right
// after the barrier that frees its slot and stored three steps later.
#pragma once

#include "fused16.hpp"

namespace zinc {

template <int NPASS>
struct Fused128Cfg {
  static constexpr int MT = 128;
  static constexpr int NGMAX = 8;                     // 16-token groups
  static constexpr int MTS = 128;                     // strip rows (four 32-token halves)
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ICMAX = 128 * NPASS;           // rows per chunk
  static constexpr int XSH = QK / 2 + 8;              // halves per token row of a half-column slot
  static constexpr int HP = 16;                       // operand pieces per token and half-column
  static constexpr int NCOPY = MT * HP / THREADS;     // pieces per thread and half-column: 4
  static constexpr int HS = ICMAX + 8;                // strip row stride (halves)
  static constexpr int NBMAX = (ICMAX - 64) / 256 + 2;  // W_down blocks a chunk can touch
  static constexpr int HSS = ((8 * NBMAX + 15) / 16) * 16;
  static constexpr int XRING = 8;                     // block columns of means kept (a power of two)
  static_assert(MT * HP % THREADS == 0, "whole pieces per thread");
  static_assert(NPASS >= 1 && NPASS <= 2, "one or two passes fit the LDS");
};

template <int NPASS>
struct Fused128Smem {
  using C = Fused128Cfg<NPASS>;
  union {
    _Float16 xs[2][C::MT * C::XSH];       // phase 1: the two half-column slots
    _Float16 hsum[C::MTS * C::HSS];       // after phase 1: the strip's 32-row means
  } u;
  _Float16 hs[C::MTS * C::HS];            // the strip, panel order, all passes
  _Float16 xm[C::XRING][C::MT * 8];       // 32-means per block column, ring
  float hsum32[C::MT * C::HSS];           // the strip's 32-row sums while phase 1 runs
  int p2_next;                            // phase 2: next unclaimed output tile
};

// One half-column in flight: NCOPY operand pieces per thread, and the means
// piece (first halves only, threads 0..127).
template <int N>
struct X128Copy {
  u32x4_16 v[N];
  u32x4_16 m;
};

// One unit.  tok = the tile's 128 token indices in LDS (the zero token M for
// padding rows), r0/r1 = the chunk's intermediate rows (multiples of 64).
template <int NPASS, class Out>
__device__ __forceinline__ void fused_unit128(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                              const uint8_t* __restrict__ wd, int H, int I,
                                              const uint8_t* __restrict__ xtok, const int* __restrict__ tok, int rows,
                                              int r0, int r1, float inter_scale, const Out& out,
                                              Fused128Smem<NPASS>& sm) {
  using C = Fused128Cfg<NPASS>;
  constexpr int NG = C::NGMAX, XSH = C::XSH, HS = C::HS, HSS = C::HSS, MT = C::MT, NC = C::NCOPY;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, o = lane >> 4, sel = (o >> 1) & 1;
  const uint32_t psel = sc_pair_sel(2 * sel);   // lane16_scales
  const int tid = threadIdx.x;
  const int nbH = H / QK;
  const uint32_t rowb = (uint32_t)nbH * BLOCK_BYTES;
  const NibbleK nk = nibble_consts_s();
  const int off = (r0 >> 6) & 3;                  // chunk's first panel within its W_down block

  for (int i = tid; i < MT * HSS; i += C::THREADS) sm.hsum32[i] = 0.0f;
  for (int i = tid; i < C::XRING * MT * 8; i += C::THREADS) (&sm.xm[0][0])[i] = (_Float16)0.0f;

  // copy plan: thread slot q = tid + THREADS*it -> token q / 16, piece q % 16
  uint32_t csrc[NC], cdst[NC];
#pragma unroll
  for (int it = 0; it < NC; ++it) {
    const int q = tid + C::THREADS * it, t = q >> 4, p = q & 15;
    csrc[it] = ((uint32_t)tok[t] * nbH * X16_TP + p) * 16u;
    cdst[it] = (uint32_t)(t * XSH + p * 8);
  }
  const bool mwave = wave < MT / 64;              // waves 0-1 carry the means pieces (wave-uniform)
  const uint32_t msrc = mwave ? ((uint32_t)tok[tid & (MT - 1)] * nbH * X16_TP + (X16_TP - 1)) * 16u : 0u;
  const uint32_t mdst = (uint32_t)((tid & (MT - 1)) * 8);

  // half-column hc = 2 * column + part; past the last column re-read the last
  // (in bounds; what it stores is never read)
  auto load_half = [&](int hc, X128Copy<NC>& xc) {
    const int kb = (hc >> 1) < nbH ? (hc >> 1) : nbH - 1;
    const uint8_t* col = xtok + (size_t)kb * X16_TP_BYTES + (hc & 1) * (C::HP * 16);
#pragma unroll
    for (int it = 0; it < NC; ++it) xc.v[it] = *reinterpret_cast<const u32x4_16*>(col + csrc[it]);
    if (mwave) xc.m = *reinterpret_cast<const u32x4_16*>(xtok + (size_t)kb * X16_TP_BYTES + msrc);
  };
  auto store_half = [&](int hc, const X128Copy<NC>& xc) {
    _Float16* slot = sm.u.xs[hc & 1];
#pragma unroll
    for (int it = 0; it < NC; ++it) *reinterpret_cast<u32x4_16*>(slot + cdst[it]) = xc.v[it];
    if (mwave && !(hc & 1)) {
      const int kb = hc >> 1;
      *reinterpret_cast<u32x4_16*>(&sm.xm[kb & (C::XRING - 1)][0] + mdst) = xc.m;
    }
  };

  for (int pass = 0; pass < NPASS; ++pass) {
    const int pr0 = r0 + pass * 128;              // the pass's first row
    if (pr0 >= r1) break;                         // a chunk of at most 128 rows: one pass (uniform)
    const bool act = pr0 + wave * 16 < r1;        // wave-uniform
    const uint32_t wrow_off = (uint32_t)((size_t)(act ? pr0 + wave * 16 + r : r0 + r) * rowb);

    f32x4_16 accg[NG], accu[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) accg[g][e] = accu[g][e] = 0.0f;

    // prologue: half-columns 0 and 1 staged; the loop's first store (step 2)
    // writes half 1, loaded here
    X128Copy<NC> xc;
    load_half(0, xc);
    lds_barrier();   // the previous pass (or the ring zeroing) is done with the slots
    store_half(0, xc);
    load_half(1, xc);

    u32x4_16 hg = {0u, 0u, 0u, 0u}, hu = hg, qg0 = hg, qu0 = hg, qg1 = hg, qu1 = hg;
    u32x4_16 cg = {0u, 0u, 0u, 0u}, cu = {0u, 0u, 0u, 0u};   // headers for the min correction
    if (act) {
      hg = *reinterpret_cast<const u32x4_16*>(wg + wrow_off);
      hu = *reinterpret_cast<const u32x4_16*>(wu + wrow_off);
      qg0 = *reinterpret_cast<const u32x4_16*>(wg + (wrow_off + 16 + 16 * o));
      qu0 = *reinterpret_cast<const u32x4_16*>(wu + (wrow_off + 16 + 16 * o));
      qg1 = *reinterpret_cast<const u32x4_16*>(wg + (wrow_off + 80 + 16 * o));
      qu1 = *reinterpret_cast<const u32x4_16*>(wu + (wrow_off + 80 + 16 * o));
    }
    lds_barrier();   // half 0 published
    const int xlane = r * XSH + o * 8;

    for (int kb = 0; kb < nbH; ++kb) {
      const int kn = (kb + 1 < nbH) ? kb + 1 : kb;
      const uint32_t noff = wrow_off + (uint32_t)kn * BLOCK_BYTES;
      if (act) {
        const Lane16S sg = lane16_scales(as_u4(hg), psel), su = lane16_scales(as_u4(hu), psel);
        const bool mine = o == (kb & 3);
        cg = mine ? hg : cg;
        cu = mine ? hu : cu;
        hg = *reinterpret_cast<const u32x4_16*>(wg + noff);
        hu = *reinterpret_cast<const u32x4_16*>(wu + noff);
        __builtin_amdgcn_sched_barrier(0);
        auto load_b = [&](int i, half8 (&b)[NG]) {
          const _Float16* xb = sm.u.xs[i >> 2] + xlane + (i & 3) * 32;
#pragma unroll
          for (int g = 0; g < NG; ++g) b[g] = *reinterpret_cast<const half8*>(xb + g * 16 * XSH);
        };
        (void)load_b;
        auto decode = [&](int i, half8& ag, half8& au) {
          const uint32_t qg = (i < 4) ? qg0[i & 3] : qg1[i & 3];
          const uint32_t qu = (i < 4) ? qu0[i & 3] : qu1[i & 3];
          ag = dequant_dword_sc(qg, (i < 4) ? sg.r0 : sg.r1, nk);
          au = dequant_dword_sc(qu, (i < 4) ? su.r0 : su.r1, nk);
        };
        // Eight token groups leave no room for a second set of B operands:
        // each group's B is refilled in place right after its two MFMAs, a
        // whole step ahead of its next use.
        half8 bc[NG], agc, auc, agn, aun;
        load_b(0, bc);
        decode(0, agc, auc);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i == 3 || i == 7) {
            // i == 3: slot 1 (half 2kb+1) published, slot 0 free -> load half 2kb+2
            // i == 7: slot 0 (half 2kb+2) published, slot 1 free -> load half 2kb+3
            lds_barrier();
            load_half(2 * kb + (i == 3 ? 2 : 3), xc);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (i < 7) decode(i + 1, agn, aun);
          if (i == 3) {   // the first quant run is decoded: refill it in place
            qg0 = *reinterpret_cast<const u32x4_16*>(wg + (noff + 16 + 16 * o));
            qu0 = *reinterpret_cast<const u32x4_16*>(wu + (noff + 16 + 16 * o));
            __builtin_amdgcn_sched_barrier(0);
          }
          if (i == 2 || i == 6) {   // the half loaded three steps ago into its slot
            store_half(2 * kb + (i == 2 ? 1 : 2), xc);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (i == 6) {   // and the second quant run
            qg1 = *reinterpret_cast<const u32x4_16*>(wg + (noff + 80 + 16 * o));
            qu1 = *reinterpret_cast<const u32x4_16*>(wu + (noff + 80 + 16 * o));
            __builtin_amdgcn_sched_barrier(0);
          }
          const _Float16* xbn = sm.u.xs[(i + 1) >> 2] + xlane + ((i + 1) & 3) * 32;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            accg[g] = mfma16x16(agc, bc[g], accg[g]);
            accu[g] = mfma16x16(auc, bc[g], accu[g]);
            if (i < 7) bc[g] = *reinterpret_cast<const half8*>(xbn + g * 16 * XSH);
          }
          if (i < 7) {
            agc = agn;
            auc = aun;
          }
          // issue order: per group its two MFMAs with decode VALU work between
          // them, then that group's B refill
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
        // min correction once per four blocks (or at the last): octet o holds
        // block (kb & ~3) + o's headers (zero past the last block)
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
        // idle waves only stage, meeting the same barriers
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i == 3 || i == 7) {
            lds_barrier();
            load_half(2 * kb + (i == 3 ? 2 : 3), xc);
          }
          if (i == 2 || i == 6) store_half(2 * kb + (i == 2 ? 1 : 2), xc);
        }
      }
    }
    // the last half loaded (past the end) goes to its free slot; then every
    // wave is done with this pass's slots and ring
    store_half(2 * nbH + 1, xc);

    // SwiGLU in registers -> fp16 strip (panel order) and the 32-row sums.
    // Accumulator e of lane (r, o) in group g: row 4o + e of the wave's tile, token 16g + r.
    if (act) {
      const int jl = pass * 128 + wave * 16 + 4 * o;      // chunk-local row, multiple of 4
      const int jg = off * 64 + pass * 128 + wave * 16;   // from the start of the chunk's first W_down block
      const int slot = 8 * (jg >> 8) + sb_slot((jg >> 5) & 7);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        _Float16 hv[4];
        float s4 = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[e] = (_Float16)(silu_f32(accg[g][e]) * accu[g][e] * inter_scale);
          s4 += (float)hv[e];
        }
        const int t = g * 16 + r;
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, hv[0]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hv[2]) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, hv[1]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hv[3]) << 16);
        *reinterpret_cast<uint2*>(sm.hs + t * HS + (jl & ~63) + panel_pos(jl & 63)) = make_uint2(w0, w1);
        s4 += __shfl_xor(s4, 16, 64);
        s4 += __shfl_xor(s4, 32, 64);
        // two 16-row tiles meet in each 32-row sum: two adds onto zero, so the
        // order does not change the value
        if (o == 0) atomicAdd(&sm.hsum32[t * HSS + slot], s4);
      }
    }
  }
  if (threadIdx.x == 0) sm.p2_next = 2 * C::WAVES;
  lds_barrier();   // strip and sums complete, slots free
  for (int i = tid; i < C::MTS * HSS; i += C::THREADS) sm.u.hsum[i] = (_Float16)(sm.hsum32[i] * 0.03125f);
  lds_barrier();

  // phase 2: the down projection over this chunk; token halves past the tile's
  // rows are skipped
  auto phase2 = [&](auto ntt_tag) {
    constexpr int NTT = decltype(ntt_tag)::value;
    switch (off) {
      case 0: fu16_phase2<C, C::ICMAX, 0, NTT, Out>(wd, H, I, r0, r1, out, sm.hs, sm.u.hsum, nk, &sm.p2_next); break;
      case 1: fu16_phase2<C, C::ICMAX, 1, NTT, Out>(wd, H, I, r0, r1, out, sm.hs, sm.u.hsum, nk, &sm.p2_next); break;
      case 2: fu16_phase2<C, C::ICMAX, 2, NTT, Out>(wd, H, I, r0, r1, out, sm.hs, sm.u.hsum, nk, &sm.p2_next); break;
      default: fu16_phase2<C, C::ICMAX, 3, NTT, Out>(wd, H, I, r0, r1, out, sm.hs, sm.u.hsum, nk, &sm.p2_next); break;
    }
  };
  if (rows > 96)
    phase2(std::integral_constant<int, 4>{});
  else if (rows > 64)
    phase2(std::integral_constant<int, 3>{});
  else if (rows > 32)
    phase2(std::integral_constant<int, 2>{});
  else
    phase2(std::integral_constant<int, 1>{});
}

}  // namespace zinc
