// Decode for 2 <= M <= 8 tokens (one launch per pass, up to eight token
// columns of the MFMA): the two HBM-bound Q4_K passes on 16x16x32
// MFMAs, so the Q4_K decode work (the VALU cost) does not grow with M.
//
//   k_decode<GATEUP=true>  streams W_gate and W_up once against one staging of
//     the activation (the same-input gate/up pair fusion of "Four bottlenecks,
//     one CUDA backend", "Bottleneck 3"), applies SwiGLU and writes the
//     per-token intermediate fp16(h * 2^-inter_shift) [M x inter].
//   k_decode<GATEUP=false> streams W_down against it and writes y.
//
// Shape.  A workgroup owns one 16-row tile of the output and KS waves; wave w
// takes an even share of the tile's super-block columns and walks them in
// passes of NBW columns.  Per pass it stages its slice of the activation in
// its own LDS area, then issues the pass's weight loads (consecutive lanes read
// consecutive 16-byte pieces of the rows' blocks, packed across the pass's
// columns) and passes each block column through LDS into the MFMA lane layout
// as it arrives; the KS partial sums meet through LDS at the end.
//
// Arithmetic.  Lane l holds row l%16 of the weight tile and token l%16 of the
// activation, eight K values each (octet o = l/16); token columns beyond M are
// computed and dropped.  A lane's operands per block are the header and the
// quant runs [16o, +16) and [64+16o, +16): chunk o/2 and chunk 2+o/2.  Dword
// i%4 of the first run (i < 4) or the second (i >= 4) feeds MFMA i; its eight
// slots are the chunk offsets {0,2,1,3,32,34,33,35} + 16(o%2) + 4(i%4).  Each
// wave stages its K range of the activation in LDS in exactly that order
// ("pieces" of eight fp16), with the 32-element sub-block means the -dmin*m
// term is contracted against: one more MFMA per four blocks.
#include <utility>

#include "fused_core.hpp"
#include "launch.hpp"

namespace zinc {

namespace {

typedef float float4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // a native 128-bit vector (no struct copies)

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

__device__ __forceinline__ float4v_t mfma16(half8 a, half8 b, float4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// f(integral_constant<int, I>) for I = 0 .. N-1, fully unrolled, so register
// arrays indexed by I stay in registers.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Cross-lane adds on the VALU (DPP): quad swaps and a shift by four lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHR4 = 0x114;   // row_shr:4 (lanes 0-3 of each row of 16 read 0)

// Launch shapes: KS waves per workgroup, at most NBW super-blocks per wave per
// pass.  Eight tokens take half the blocks per pass, so that their staged
// activation still fits LDS (60 KB for gate/up, two workgroups per CU; 134 KB
// for down).
template <int MM, bool GATEUP>
struct DecShape {
  static constexpr int KS = GATEUP ? 4 : 11;
  static constexpr int NBW = MM > 4 ? 2 : 4;
};

// Orders one wave's LDS accesses for the compiler (the hardware already runs
// them in program order); emits no instruction.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

struct DecBlock {
  uint4 hdr, q0, q1;
};

// Piece p of a wave's staged activation: token n, local block bl, chunk c,
// 4-byte step j (quant byte 4j of the chunk's first 32).  Its LDS slot is the
// (MFMA i, octet o) whose operand it is: i = 4*(c/2) + j%4, o = 2*(c%2) + j/4.
__device__ __forceinline__ int piece_slot(int bl, int c, int j) {
  const int i = 4 * (c >> 1) + (j & 3);
  const int o = 2 * (c & 1) + (j >> 2);
  return (bl * 8 + i) * 4 + o;
}

// Three waves per SIMD (at most 168 VGPRs): with 53 KB of LDS, three 4-wave
// gate/up workgroups share a CU, so the 688 tiles of an 11,008-row pass are
// all resident at once instead of 512 and a second round of 176.
template <int MM, bool GATEUP, int KS, int NBW>
__global__ __launch_bounds__(64 * KS, 3) void k_decode(const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
                                                    int K, int N, const _Float16* __restrict__ xin, int M,
                                                    _Float16* out, float scale, const _Float16* res,
                                                    float res_scale) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int TSTRIDE = NBW * 256 + 32;     // halves per staged token (+64 B against bank conflicts)
  constexpr int NPIECE = MM * NBW * 32;       // pieces of 8 halves per pass
  constexpr int NPIT = (NPIECE + 63) / 64;
  constexpr int NG = (NBW + 3) / 4;           // min-correction groups per pass
  constexpr int NPC = NBW * 144;              // 16-byte weight pieces per matrix and pass
  constexpr int NLD = (NPC + 63) / 64;        // coalesced loads per matrix and pass
  __shared__ __attribute__((aligned(16))) _Float16 xs_all[KS][MM * TSTRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 xm_all[KS][MM * NBW * 8];
  // per wave and matrix: one block column of the tile (16 rows x 9 pieces of
  // 16 B), written in load order and read back in the MFMA lane layout.  After
  // its last block a wave leaves its partial sums for wave 0 in its own area
  // (NMAT x 4 x 64 floats), which no other wave touches.
  __shared__ __attribute__((aligned(16))) u32x4 wt_all[KS][NMAT][16 * 9];
  static_assert(sizeof(wt_all[0]) >= NMAT * 4 * 64 * sizeof(float), "partial sums fit a wave's weight area");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches below
  const int r = lane & 15, o = lane >> 4, sel = (o >> 1) & 1;
  const uint32_t psel = sc_pair_sel(2 * sel);   // lane16_scales: chunks sel and 2 + sel
  // B-operand column: token r.  Columns r >= M are computed and discarded, so
  // they may read any staged token's (finite) data.
  const int tb = r & (MM - 1);
  const int tile = blockIdx.x;
  const int nb = K / QK;
  const int b0 = (int)((long long)wave * nb / KS), b1 = (int)((long long)(wave + 1) * nb / KS);
  const int per_wave_max = (nb + KS - 1) / KS;
  const int npass = (per_wave_max + NBW - 1) / NBW;   // the same for every wave of the block
  const uint32_t row_bytes = (uint32_t)nb * BLOCK_BYTES;
  const uint8_t* tile0 = W0 + (size_t)tile * 16 * row_bytes;
  const uint8_t* tile1 = GATEUP ? W1 + (size_t)tile * 16 * row_bytes : nullptr;
  u32x4* wt0 = wt_all[wave][0];
  u32x4* wt1 = wt_all[wave][NMAT - 1];
  _Float16* xs = xs_all[wave];
  _Float16* xm = xm_all[wave];
  const NibbleK nk = nibble_consts_s();

  float4v_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  for (int pass = 0; pass < npass; ++pass) {
    const int pb = b0 + pass * NBW;                   // first block of this pass
    const int cnt = max(0, min(NBW, b1 - pb));        // wave-uniform
    // 1. the activation loads of the pass.  Every load of a pass is issued,
    //    whatever cnt is: a block past the wave's range reads the wave's last
    //    block (or block 0 when the range is empty) instead, and its result is
    //    discarded below, so the compiler can count the loads in flight.
    const int blast = max(b1 - 1, 0);
    uint2 xl[NPIT], xh[NPIT];
#pragma unroll
    for (int it = 0; it < NPIT; ++it) {
      const int p = lane + 64 * it;
      const int j = p & 7, c = (p >> 3) & 3, bl = (p >> 5) % NBW, n = p / (32 * NBW);
      const _Float16* src = xin + (size_t)min(n, M - 1) * K + (size_t)min(pb + bl, blast) * QK + 64 * c + 4 * j;
      xl[it] = *reinterpret_cast<const uint2*>(src);
      xh[it] = *reinterpret_cast<const uint2*>(src + 32);
    }
    // 2. stage this pass's activation pieces and sub-block means.  The LDS
    //    areas of the pass loop belong to one wave each, whose LDS accesses
    //    complete in program order, so no workgroup barrier is needed; the
    //    fence below only keeps the compiler from moving accesses across it.
    wave_lds_order();
#pragma unroll
    for (int it = 0; it < NPIT; ++it) {
      const int p = lane + 64 * it;
      const int j = p & 7, c = (p >> 3) & 3, bl = (p >> 5) % NBW, n = p / (32 * NBW);
      const bool live = (p < NPIECE) && (bl < cnt);
      const uint2 lo = xl[it], hi = xh[it];
      // slot order {0,2,1,3}: swap the middle two halves of each group of four
      const uint32_t l0 = (lo.x & 0xFFFFu) | (lo.y << 16), l1 = (lo.x >> 16) | (lo.y & 0xFFFF0000u);
      const uint32_t h0 = (hi.x & 0xFFFFu) | (hi.y << 16), h1 = (hi.x >> 16) | (hi.y & 0xFFFF0000u);
      if (live) *reinterpret_cast<uint4*>(xs + n * TSTRIDE + piece_slot(bl, c, j) * 8) = make_uint4(l0, l1, h0, h1);
      const half4 lv = __builtin_bit_cast(half4, lo), hv = __builtin_bit_cast(half4, hi);
      float sl = ((float)lv[0] + (float)lv[1]) + ((float)lv[2] + (float)lv[3]);
      float sh = ((float)hv[0] + (float)hv[1]) + ((float)hv[2] + (float)hv[3]);
      // the eight pieces of one (token, block, chunk) are eight consecutive
      // lanes; after the quad sums and the shift by four, lane j == 4 holds all eight
      sl += dpp_f<DPP_QUAD_XOR1>(sl);
      sh += dpp_f<DPP_QUAD_XOR1>(sh);
      sl += dpp_f<DPP_QUAD_XOR2>(sl);
      sh += dpp_f<DPP_QUAD_XOR2>(sh);
      sl += dpp_f<DPP_ROW_SHR4>(sl);
      sh += dpp_f<DPP_ROW_SHR4>(sh);
      if (live && j == 4) {
        xm[(n * NBW + bl) * 8 + sb_slot(2 * c)] = (_Float16)(sl * 0.03125f);
        xm[(n * NBW + bl) * 8 + sb_slot(2 * c + 1)] = (_Float16)(sh * 0.03125f);
      }
    }
    wave_lds_order();

    // 3. the weight loads, issued only once the activation is staged.  Issued
    //    together, the activation loads queue behind every tile's weight
    //    loads (they landed 4 to 14 us after a wave's start), and a wave
    //    cannot start on block columns that have already arrived.  The
    //    scheduling barriers keep the loads here.
    __builtin_amdgcn_sched_barrier(0);
    // The NBW block columns of a pass are NPC pieces of 16 B per matrix, read
    // by NLD coalesced loads: piece p = 64k + lane is block p/144 of the pass,
    // row (p%144)/9, bytes [16*(p%9), +16) of that row's block.  Pieces past
    // NPC re-read the last one (in bounds, unused).
    u32x4 w0[NLD], w1[NLD];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int pc = min(64 * k + lane, NPC - 1);
      const int bl = pc / 144, q = pc - 144 * bl;
      const uint32_t off = (uint32_t)(q / 9) * row_bytes + 16u * (uint32_t)(q % 9) +
                           (uint32_t)min(pb + bl, blast) * BLOCK_BYTES;
      w0[k] = *reinterpret_cast<const u32x4*>(tile0 + off);
      if (GATEUP) w1[k] = *reinterpret_cast<const u32x4*>(tile1 + off);
    }
    // headers of the min correction (octet o of group g takes block 4g+o),
    // picked from the LDS copy of each block column as it is read below; an
    // octet past the pass's blocks keeps a zero header, hence a zero A operand
    uint4 ch0[NG], ch1[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) ch0[g] = ch1[g] = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // 4. MFMAs: 8 per block and matrix, then the min correction per 4 blocks
    const _Float16* xb = xs + tb * TSTRIDE + o * 8;
    static_for<NBW>([&](auto blc) {
      constexpr int bl = decltype(blc)::value;
      if (bl >= cnt) return;   // wave-uniform
      // through LDS into the MFMA layout: lane (r, o) takes row r's header and
      // quant runs [16o, +16) and [64+16o, +16)
      static_for<(144 * bl + 143) / 64 - (144 * bl) / 64 + 1>([&](auto kc) {
        constexpr int k = (144 * bl) / 64 + decltype(kc)::value;
        const int q = 64 * k + lane - 144 * bl;
        if (q >= 0 && q < 144) {
          wt0[q] = w0[k];
          if (GATEUP) wt1[q] = w1[k];
        }
      });
      DecBlock db0, db1;
      db0.hdr = as_uint4(wt0[9 * r]);
      db0.q0 = as_uint4(wt0[9 * r + 1 + o]);
      db0.q1 = as_uint4(wt0[9 * r + 5 + o]);
      if (GATEUP) {
        db1.hdr = as_uint4(wt1[9 * r]);
        db1.q0 = as_uint4(wt1[9 * r + 1 + o]);
        db1.q1 = as_uint4(wt1[9 * r + 5 + o]);
      }
      if (o == (bl & 3)) {
        ch0[bl >> 2] = db0.hdr;
        if (GATEUP) ch1[bl >> 2] = db1.hdr;
      }
      const Lane16S s0 = lane16_scales(db0.hdr, psel);
      Lane16S s1;
      if (GATEUP) s1 = lane16_scales(db1.hdr, psel);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const half8 b = *reinterpret_cast<const half8*>(xb + (bl * 8 + i) * 32);
        const uint32_t q = (i < 4) ? dword_of(db0.q0, i & 3) : dword_of(db0.q1, i & 3);
        const half8 a = dequant_dword_sc(q, (i < 4) ? s0.r0 : s0.r1, nk);
        acc0 = mfma16(a, b, acc0);
        if (GATEUP) {
          const uint32_t qu = (i < 4) ? dword_of(db1.q0, i & 3) : dword_of(db1.q1, i & 3);
          const half8 au = dequant_dword_sc(qu, (i < 4) ? s1.r0 : s1.r1, nk);
          acc1 = mfma16(au, b, acc1);
        }
      }
    });
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (4 * g >= cnt) continue;   // wave-uniform
      const int bl = 4 * g + o;
      // octets past the pass's blocks (zero headers) read the means of a staged
      // block (finite)
      const half8 b = *reinterpret_cast<const half8*>(xm + (tb * NBW + min(bl, cnt - 1)) * 8);
      acc0 = mfma16(block_neg_dm32(ch0[g]), b, acc0);
      if (GATEUP) acc1 = mfma16(block_neg_dm32(ch1[g]), b, acc1);
    }
  }

  // 5. the KS partial sums meet in wave 0
  if (KS > 1) {
    wave_lds_order();   // the wave's last weight reads stay before these writes
    if (wave > 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float* red = reinterpret_cast<float*>(wt_all[wave]);
        red[e * 64 + lane] = acc0[e];
        if (GATEUP) red[(4 + e) * 64 + lane] = acc1[e];
      }
    }
    lds_barrier();
    if (wave > 0) return;
    for (int w = 1; w < KS; ++w) {
      const float* red = reinterpret_cast<const float*>(wt_all[w]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0[e] += red[e * 64 + lane];
        if (GATEUP) acc1[e] += red[(4 + e) * 64 + lane];
      }
    }
  }
  // accumulator e of lane l: row 4*(l/16) + e of the tile, token l%16
  if (r < M) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = GATEUP ? silu_f32(acc0[e]) * acc1[e] * scale : acc0[e] * scale;
      // the residual (down pass only; it may be out itself: read, then written, here)
      if (!GATEUP && res) v += (float)res[(size_t)r * N + tile * 16 + 4 * o + e] * res_scale;
      out[(size_t)r * N + tile * 16 + 4 * o + e] = (_Float16)v;
    }
  }
}

template <int MM>
void launch_group_mfma(const void* wg, const void* wu, const void* wd, int hidden, int inter, const _Float16* x,
                       _Float16* y, _Float16* h, int M, float gu_scale, float dn_scale, const _Float16* res,
                       float res_scale, int stage, hipStream_t stream) {
  typedef DecShape<MM, true> GU;
  typedef DecShape<MM, false> DN;
  if (stage == 0) {
    hipLaunchKernelGGL((k_decode<MM, true, GU::KS, GU::NBW>), dim3(inter / 16), dim3(64 * GU::KS), 0, stream,
                       static_cast<const uint8_t*>(wg), static_cast<const uint8_t*>(wu), hidden, inter, x, M, h,
                       gu_scale, (const _Float16*)nullptr, 0.0f);
  } else {
    hipLaunchKernelGGL((k_decode<MM, false, DN::KS, DN::NBW>), dim3(hidden / 16), dim3(64 * DN::KS), 0, stream,
                       static_cast<const uint8_t*>(wd), static_cast<const uint8_t*>(nullptr), inter, hidden, h, M,
                       y, dn_scale, res, res_scale);
  }
}

void launch_tokens_mfma(const void* wg, const void* wu, const void* wd, int hidden, int inter, const _Float16* x,
                        _Float16* y, _Float16* h, int M, float gu_scale, float dn_scale, const _Float16* res,
                        float res_scale, int stage, hipStream_t stream) {
  if (M <= 1)
    launch_group_mfma<1>(wg, wu, wd, hidden, inter, x, y, h, M, gu_scale, dn_scale, res, res_scale, stage, stream);
  else if (M <= 2)
    launch_group_mfma<2>(wg, wu, wd, hidden, inter, x, y, h, M, gu_scale, dn_scale, res, res_scale, stage, stream);
  else if (M <= 4)
    launch_group_mfma<4>(wg, wu, wd, hidden, inter, x, y, h, M, gu_scale, dn_scale, res, res_scale, stage, stream);
  else
    launch_group_mfma<8>(wg, wu, wd, hidden, inter, x, y, h, M, gu_scale, dn_scale, res, res_scale, stage, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const void* wg, const void* wu, const void* wd, int hidden, int inter, const void* x,
                              void* y, int M, int inter_shift, int out_shift, void* ws, hipStream_t stream,
                              float mlp_scale, const void* res) {
  const _Float16* xh = static_cast<const _Float16*>(x);
  _Float16* yh = static_cast<_Float16*>(y);
  const _Float16* rh = static_cast<const _Float16*>(res);
  _Float16* hbuf = static_cast<_Float16*>(ws);
  const float gu_scale = ldexpf(1.0f, -inter_shift);
  const float dn_scale = ldexpf(1.0f, inter_shift - out_shift) * mlp_scale, res_scale = ldexpf(1.0f, -out_shift);
  // groups of at most eight tokens (the 16 columns of the MFMA hold them all,
  // so each weight is read once per call)
  for (int stage = 0; stage < 2; ++stage) {
    timing_begin(stream);
    for (int t0 = 0; t0 < M; t0 += 8) {
      const int mg = min(8, M - t0);
      launch_tokens_mfma(wg, wu, wd, hidden, inter, xh + (size_t)t0 * hidden, yh + (size_t)t0 * hidden,
                         hbuf + (size_t)t0 * inter, mg, gu_scale, dn_scale, rh ? rh + (size_t)t0 * hidden : nullptr,
                         res_scale, stage, stream);
    }
    timing_end(stream);
  }
  return hipGetLastError();
}

}  // namespace zinc
