// Batched-expert MoE MLP: y[t] = sum_s p[t,s] * MLP_{ids[t,s]}(x[t]).
//
// The expert ids and mixing weights stay on the GPU.  The host launches a
// fixed sequence of kernels sized only by (M, top_k, n_experts) -- never by the
// routing -- so nothing is read back mid-call.  This is the batched-expert
// design of "Four bottlenecks, one CUDA backend", "Bottleneck 2": the device
// kernels look up which experts each token uses and address those experts'
// weights on their own, with no host round trip in between:
//   1. k_moe_count    per-expert slot counts; invalid ids set *dev_error
//   2. k_moe_plan     exclusive scan of the counts -> list offsets, and the tile
//                     table (expert, first list entry, rows) of MT-slot tiles
//   3. k_moe_scatter  slot indices grouped by expert, and each slot's position
//   4. k_stage_x16    the activation per token in the fused unit's operand
//                     order (fused16.hpp), plus an all-zero token
//   5. k_moe_fused16  one 80-token fused unit (fused16.hpp) per (tile of up
//                     to 80 routed rows of one expert, intermediate chunk):
//                     192-row chunks, or 128-row chunks for every tile of an
//                     expert whose remainder tile is small; blocks past the
//                     device-side unit count exit at once.  Each row's expert
//                     output (fp16 at the output scale) is stored at its
//                     slot: Q[chunk][slot][hidden]
//   6. k_moe_combine  y[t] = fp16(sum over the token's slots of p[t,s] times
//                     the sum over chunks), in fp32
// Every partial has exactly one writer, all tiles of an expert share one
// chunking (so a row's arithmetic does not depend on which of its expert's
// tiles the scatter put it in), and the combine order is fixed, so the result
// is deterministic (the atomics only count and place).
#include <algorithm>

#include "fused16.hpp"
#include "launch.hpp"
#include "util_kernels.hpp"

namespace zinc {

namespace {

// Bytes of one [H x I] W_down matrix in the given format.
__host__ __device__ inline size_t down_matrix_bytes(int fmt, int H, int I) {
  return (fmt == kDownQ51) ? (size_t)H * (I / 32) * Q5_1_BLOCK_BYTES
                           : (size_t)H * (I / QK) * ((fmt == kDownQ5K) ? Q5K_BLOCK_BYTES : BLOCK_BYTES);
}

constexpr int ICMAX_MOE = 192;  // intermediate rows per chunk (three 64-row panels)
constexpr int MT_MOE = 80;      // routed rows per tile: an expert of up to 80 rows is one tile
using MoeCfg = Fused16Cfg<ICMAX_MOE, MT_MOE>;

struct MoePlan {
  int* counts;       // [E]
  int* cursor;       // [E]
  int* offsets;      // [E + 1]
  int* tile_expert;  // [max_tiles]
  int* tile_start;   // [max_tiles]
  int* tile_rows;    // [max_tiles]
  int* n_tiles;      // [2]: tiles, tiles of 192-row-chunk experts (listed first)
  int* slots;        // [M * top_k] slot indices grouped by expert
  int* pos;          // [M * top_k] list position of each slot (| kPosSmall: 128-row chunks), -1 if its id is invalid
  _Float16* Q;       // [n_chunks][M * top_k + 1][H], fp16 at the output scale (last row: junk)
  uint8_t* xtok;     // staged activation, x16_staged_bytes(M, H)
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int max_tiles_for(int M, int top_k, int E) {
  const long long pairs = (long long)M * top_k;
  return (int)((pairs + MT_MOE - 1) / MT_MOE + (pairs < E ? pairs : E));
}

// Chunks of the intermediate dimension: 192-row chunks (three 64-row panels),
// or 128-row chunks (eight busy waves instead of twelve) for every tile of an
// expert whose remainder tile has at most kSmallRows rows.  Such a remainder
// tile costs most of a unit for a few rows (the weight decode dominates); cut
// into more, shorter units, the expert's tiles fill the last round of units
// more evenly.  A whole expert takes one chunking, so a row's partial sums do
// not depend on which of the expert's tiles the scatter put it in.
constexpr int kSmallRows = 16;

__host__ __device__ inline bool small_expert(int count, int MT) {
  const int rem = count % MT;
  return rem > 0 && rem <= kSmallRows;
}

int chunks_for(int I) {
  const int npan = I / 64;
  return (npan + ICMAX_MOE / 64 - 1) / (ICMAX_MOE / 64);
}

int chunks_small_for(int I) {
  const int npan = I / 64;
  return std::max(chunks_for(I), (npan + 1) / 2);
}

// A slot's list position carries this bit when its expert takes 128-row
// chunks (positions are below 2^24), so the combine knows its chunk count.
constexpr int kPosSmall = 1 << 30;

MoePlan carve(void* ws, int M, int top_k, int E, int H, int I, size_t* total) {
  MoePlan p;
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  const int mt = max_tiles_for(M, top_k, E);
  const size_t pairs = (size_t)M * top_k;
  auto take = [&](size_t bytes) { char* r = base ? base + off : nullptr; off += align256(bytes); return r; };
  p.counts = reinterpret_cast<int*>(take(sizeof(int) * E));
  p.cursor = reinterpret_cast<int*>(take(sizeof(int) * E));
  p.offsets = reinterpret_cast<int*>(take(sizeof(int) * (E + 1)));
  p.tile_expert = reinterpret_cast<int*>(take(sizeof(int) * mt));
  p.tile_start = reinterpret_cast<int*>(take(sizeof(int) * mt));
  p.tile_rows = reinterpret_cast<int*>(take(sizeof(int) * mt));
  p.n_tiles = reinterpret_cast<int*>(take(sizeof(int) * 2));
  p.slots = reinterpret_cast<int*>(take(sizeof(int) * pairs));
  p.pos = reinterpret_cast<int*>(take(sizeof(int) * pairs));
  p.Q = reinterpret_cast<_Float16*>(take(sizeof(_Float16) * (size_t)chunks_small_for(I) * (pairs + 1) * H));
  p.xtok = reinterpret_cast<uint8_t*>(take(x16_staged_bytes(M, H)));
  if (total) *total = off;
  return p;
}

// Tile table from per-expert counts, by thread e of a 1024-thread block (E <=
// 1024): the tiles of 192-row-chunk experts first (full tiles, then
// remainders), then those of 128-row-chunk experts (full, then remainders), so
// the longest units start first.  Also the list offsets (exclusive scan of the
// counts), n_tiles[0] = all tiles and n_tiles[1] = the tiles of 192-row-chunk
// experts.  s0..s4: LDS scratch of 1024 ints each.  Returns the expert's list
// offset.
__device__ int build_tile_table(int e, int E, int c, int MT, int* s0, int* s1, int* s2, int* s3, int* s4,
                                int* __restrict__ offsets, int* __restrict__ tile_expert,
                                int* __restrict__ tile_start, int* __restrict__ tile_rows,
                                int* __restrict__ n_tiles) {
  const int nf = c / MT, rem = c - nf * MT;
  const bool sm = small_expert(c, MT);
  const int fa = sm ? 0 : nf, ra = (!sm && rem > 0) ? 1 : 0;   // 192-row-chunk expert
  const int fb = sm ? nf : 0, rb = sm ? 1 : 0;                 // 128-row-chunk expert
  // inclusive scans over the first P entries, P the power of two at or above
  // E (the entries from E on are zero, so entry P - 1 holds the totals and
  // later entries are never read)
  int P = 1;
  while (P < E) P <<= 1;
  if (P <= 64) {
    // one wave holds every entry: scan in registers, then publish
    if (e < 64) {
      int v0 = c, v1 = fa, v2 = ra, v3 = fb, v4 = rb;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int a0 = __shfl_up(v0, d, 64), a1 = __shfl_up(v1, d, 64), a2 = __shfl_up(v2, d, 64);
        const int a3 = __shfl_up(v3, d, 64), a4 = __shfl_up(v4, d, 64);
        if (e >= d) {
          v0 += a0;
          v1 += a1;
          v2 += a2;
          v3 += a3;
          v4 += a4;
        }
      }
      s0[e] = v0;
      s1[e] = v1;
      s2[e] = v2;
      s3[e] = v3;
      s4[e] = v4;
    }
    lds_barrier();
  } else {
  s0[e] = c;
  s1[e] = fa;
  s2[e] = ra;
  s3[e] = fb;
  s4[e] = rb;
  lds_barrier();
  for (int d = 1; d < P; d <<= 1) {
    const int a0 = (e >= d) ? s0[e - d] : 0;
    const int a1 = (e >= d) ? s1[e - d] : 0;
    const int a2 = (e >= d) ? s2[e - d] : 0;
    const int a3 = (e >= d) ? s3[e - d] : 0;
    const int a4 = (e >= d) ? s4[e - d] : 0;
    lds_barrier();
    s0[e] += a0;
    s1[e] += a1;
    s2[e] += a2;
    s3[e] += a3;
    s4[e] += a4;
    lds_barrier();
  }
  }
  const int off = s0[e] - c;   // exclusive
  const int tfa = s1[P - 1], tra = s2[P - 1], tfb = s3[P - 1], trb = s4[P - 1];
  if (e < E) offsets[e] = off;
  if (e == E - 1) {
    offsets[E] = s0[e];
    n_tiles[0] = tfa + tra + tfb + trb;
    n_tiles[1] = tfa + tra;
  }
  const int t0 = sm ? tfa + tra + s3[e] - fb : s1[e] - fa;   // first full tile of this expert
  for (int i = 0; i < nf; ++i) {
    tile_expert[t0 + i] = e;
    tile_start[t0 + i] = off + i * MT;
    tile_rows[t0 + i] = MT;
  }
  if (rem > 0) {
    const int t = sm ? tfa + tra + tfb + s4[e] - 1 : tfa + s2[e] - 1;
    tile_expert[t] = e;
    tile_start[t] = off + nf * MT;
    tile_rows[t] = rem;
  }
  return off;
}

__global__ __launch_bounds__(256) void k_moe_count(const int32_t* __restrict__ ids, int n_slots, int E,
                                                  int* __restrict__ counts, int32_t* __restrict__ dev_error) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_slots) return;
  const int e = ids[i];
  if (e >= 0 && e < E) {
    atomicAdd(counts + e, 1);
  } else if (dev_error) {
    atomicOr(dev_error, 1);
  }
}

// One block of 1024 threads: list offsets and the tile table (build_tile_table).
__global__ __launch_bounds__(1024) void k_moe_plan(const int* __restrict__ counts, int E, int* __restrict__ offsets,
                                                  int* __restrict__ tile_expert, int* __restrict__ tile_start,
                                                  int* __restrict__ tile_rows, int* __restrict__ n_tiles, int MT) {
  __shared__ int s0[1024], s1[1024], s2[1024], s3[1024], s4[1024];
  const int e = threadIdx.x;
  const int cnt = (e < E) ? counts[e] : 0;
  build_tile_table(e, E, cnt, MT, s0, s1, s2, s3, s4, offsets, tile_expert, tile_start, tile_rows, n_tiles);
}

__global__ __launch_bounds__(256) void k_moe_scatter(const int32_t* __restrict__ ids, int n_slots, int E, int MT,
                                                    const int* __restrict__ offsets, int* __restrict__ cursor,
                                                    int* __restrict__ slots, int* __restrict__ pos) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_slots) return;
  const int e = ids[i];
  if (e < 0 || e >= E) {
    pos[i] = -1;
    return;
  }
  const int o = offsets[e];
  const int q = o + atomicAdd(cursor + e, 1);
  slots[q] = i;
  pos[i] = q | (small_expert(offsets[e + 1] - o, MT) ? kPosSmall : 0);
}

// Steps 1-3 in one workgroup of 1024 threads when the slot count is small
// (the usual case): counts with LDS atomics, the scans and the tile table
// (build_tile_table's order), then the scatter with LDS cursors.
constexpr int kRouteOneBlockSlots = 1 << 16;

// Block 0 routes (the one-workgroup path); every other block stages the
// activation, four 256-thread staging groups per block (group g = 4 (b - 1) +
// threadIdx.x / 256 of the grid ((M + 8) / 8) x (H / 256)), so the two run side
// by side in one launch.
__global__ __launch_bounds__(1024) void k_moe_route(const int32_t* __restrict__ ids, int n_slots, int E,
                                                   int32_t* __restrict__ dev_error, int* __restrict__ offsets,
                                                   int* __restrict__ tile_expert, int* __restrict__ tile_start,
                                                   int* __restrict__ tile_rows, int* __restrict__ n_tiles,
                                                   int* __restrict__ slots, int* __restrict__ pos, int MT,
                                                   const _Float16* __restrict__ x, int H, int M,
                                                   uint8_t* __restrict__ xtok) {
  if (blockIdx.x > 0) {
    const int gx = (M + 8) / 8, g = 4 * ((int)blockIdx.x - 1) + ((int)threadIdx.x >> 8);
    if (g < gx * (H / QK)) stage_x16_group(x, H, M, xtok, g % gx, g / gx, threadIdx.x & 255);
    return;
  }
  __shared__ int cnt[1024];
  __shared__ int s0[1024], s1[1024], s2[1024], s3[1024], s4[1024];
  const int e = threadIdx.x;
  cnt[e] = 0;
  lds_barrier();
  bool bad = false;
  // the first four ids of this thread stay in registers for the scatter pass
  constexpr int KEEP = 4;
  int idk[KEEP];
#pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    const int i = (int)threadIdx.x + 1024 * k;
    idk[k] = (i < n_slots) ? ids[i] : 0;
  }
#pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    if ((int)threadIdx.x + 1024 * k < n_slots) {
      const int x = idk[k];
      if (x >= 0 && x < E)
        atomicAdd(&cnt[x], 1);
      else
        bad = true;
    }
  }
  for (int i = threadIdx.x + 1024 * KEEP; i < n_slots; i += 1024) {
    const int x = ids[i];
    if (x >= 0 && x < E)
      atomicAdd(&cnt[x], 1);
    else
      bad = true;
  }
  if (bad && dev_error) atomicOr(dev_error, 1);
  lds_barrier();
  const int c = (e < E) ? cnt[e] : 0;
  const int off = build_tile_table(e, E, c, MT, s0, s1, s2, s3, s4, offsets, tile_expert, tile_start, tile_rows,
                                   n_tiles);
  lds_barrier();
  s1[e] = small_expert(c, MT) ? kPosSmall : 0;   // the expert's position flag
  lds_barrier();
  cnt[e] = off;   // the expert's cursor
  lds_barrier();
  auto scatter = [&](int i, int x) {
    if (x >= 0 && x < E) {
      const int q = atomicAdd(&cnt[x], 1);
      slots[q] = i;
      pos[i] = q | s1[x];
    } else {
      pos[i] = -1;
    }
  };
#pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    const int i = (int)threadIdx.x + 1024 * k;
    if (i < n_slots) scatter(i, idk[k]);
  }
  for (int i = threadIdx.x + 1024 * KEEP; i < n_slots; i += 1024) scatter(i, ids[i]);
}

// MoE output of the 80-token unit: unit row r belongs to slot slot_of_row[r];
// the fp16 partial, at the output scale, goes to Q[chunk][slot][n].  Padding
// rows carry slot = pairs, a junk row after the chunk's pairs (no branch
// around the stores).  Lanes run along n, so a store instruction writes two
// runs of 32 rows x 2 bytes; its address is a 32-bit offset (row offsets read
// once per unit) from the chunk's base.
struct OutSlots {
  _Float16* Q;
  size_t pairs;
  int H;
  float scale;
  int chunk;
  const int* slot_of_row;   // LDS, one entry per strip row (96)
  template <int NTT, int NA>
  __device__ __forceinline__ void store(const float16v (&acc)[NA], int nt, int l32, int h) const {
    const size_t rows_bytes = (pairs + 1) * (size_t)H * sizeof(_Float16);   // < 4 GiB (checked by the caller)
    const __amdgpu_buffer_rsrc_t qc = __builtin_amdgcn_make_buffer_rsrc(Q + (size_t)chunk * (pairs + 1) * H, (short)0,
                                                                       (int)rows_bytes, 0x00020000);
    const uint32_t nb = (uint32_t)(nt * 32 + l32) * 2u;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t row = (uint32_t)slot_of_row[32 * tt + 8 * q + 4 * h + e] * (uint32_t)H * 2u;
          const _Float16 v = (_Float16)(acc[tt][4 * q + e] * scale);
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, v), qc, row + nb, 0, 0);
        }
      }
    }
  }
};

template <int FMT>
__global__ __launch_bounds__(MoeCfg::THREADS) void k_moe_fused16(
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, const uint8_t* __restrict__ wd, int H, int I,
    int M, const uint8_t* __restrict__ xtok, int top_k, const int* __restrict__ n_tiles,
    const int* __restrict__ tile_expert, const int* __restrict__ tile_start, const int* __restrict__ tile_rows,
    const int* __restrict__ slots, _Float16* __restrict__ Q, int pairs, float inter_scale, float out_scale,
    int n_chunks, int n_chunks_small) {
  __shared__ __attribute__((aligned(16))) Fused16Smem<ICMAX_MOE, MT_MOE> sm;
  __shared__ int tok[MT_MOE];
  __shared__ int slot_of_row[MoeCfg::MTS];   // rows past MT_MOE (phase 2's last 32-token half): the junk row

  // Units: the chunks of the 192-row-chunk experts' tiles (listed first), then
  // those of the others' tiles.  Workgroups go to the eight XCDs round-robin
  // by block id, and every chunk of tile ti runs on XCD ti % 8: the chunks of
  // one expert tile read neighbouring W_down column slices, which share cache
  // lines at their boundary (144-byte Q4_K blocks do not align with 128-byte
  // lines), and the tile's gathered activation rows, under one L2.  Each of
  // the two segments takes 8 * chunks * ceil(tiles / 8) block ids.
  const int nbig = n_tiles[1];
  const int seg_big = 8 * n_chunks * ((nbig + 7) / 8);
  const bool big = (int)blockIdx.x < seg_big;
  const int nc = big ? n_chunks : n_chunks_small;
  const int u = big ? (int)blockIdx.x : (int)blockIdx.x - seg_big;
  const int x = u & 7, s = u >> 3;
  const int q = s / nc;
  const int chunk = s - q * nc;
  const int ti = (big ? 0 : nbig) + 8 * q + x;
  if (big ? ti >= nbig : ti >= n_tiles[0]) return;
  const int e = tile_expert[ti];
  const int start = tile_start[ti], rows = tile_rows[ti];
  if (threadIdx.x < MoeCfg::MTS) {
    int t = M, sl = pairs;   // padding rows: the zero token, the junk row
    if ((int)threadIdx.x < rows) {
      sl = slots[start + threadIdx.x];
      t = sl / top_k;
    }
    if (threadIdx.x < MT_MOE) tok[threadIdx.x] = t;
    slot_of_row[threadIdx.x] = sl;
  }
  lds_barrier();
  const int npan = I / 64;
  const int r0 = (int)((long long)chunk * npan / nc) * 64;
  const int r1 = (int)((long long)(chunk + 1) * npan / nc) * 64;
  const size_t gu_bytes = (size_t)I * (H / QK) * BLOCK_BYTES;   // one expert's gate (or up) matrix
  const size_t d_bytes = down_matrix_bytes(FMT, H, I);          // one expert's down matrix
  const OutSlots out{Q, (size_t)pairs, H, out_scale, chunk, slot_of_row};
  fused_unit16<ICMAX_MOE, OutSlots, MT_MOE, kUnitFused, FMT>(wg + e * gu_bytes, wu + e * gu_bytes, wd + e * d_bytes,
                                                             H, I, xtok, tok, rows, r0, r1, inter_scale, out, sm);
}

// y[t][n] = fp16(sum_s p[t*k+s] * sum_c Q[c][t*k+s][n]) over the token's valid
// slots; one block per token, eight outputs (one 16-byte load) per thread.  A
// slot's chunk count is n_chunks_small if its position carries kPosSmall.
__global__ __launch_bounds__(256) void k_moe_combine(const _Float16* __restrict__ Q, const int* __restrict__ pos,
                                                    const float* __restrict__ p, int top_k, int n_chunks,
                                                    int n_chunks_small, int pairs, int H,
                                                    _Float16* __restrict__ y) {
  const int t = blockIdx.x;
  for (int n = threadIdx.x * 8; n < H; n += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int s = 0; s < top_k; ++s) {
      const int slot = t * top_k + s;
      const int q = pos[slot];
      if (q < 0) continue;   // invalid expert id: no contribution
      const int nc = (q & kPosSmall) ? n_chunks_small : n_chunks;
      float part[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) part[e] = 0.0f;
      const _Float16* base = Q + (size_t)slot * H + n;
      const size_t cstride = (size_t)(pairs + 1) * H;
      int c = 0;
      // four chunks' loads in flight at a time (a slot has 4 or 6 chunks);
      // the sum keeps chunk order
      for (; c + 4 <= nc; c += 4) {
        half8 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const half8*>(base + (size_t)(c + u) * cstride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) part[e] += (float)v[u][e];
      }
      for (; c < nc; ++c) {
        const half8 v = *reinterpret_cast<const half8*>(base + (size_t)c * cstride);
#pragma unroll
        for (int e = 0; e < 8; ++e) part[e] += (float)v[e];
      }
      const float w = p[slot];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w * part[e];
    }
    half8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)acc[e];
    *reinterpret_cast<half8*>(y + (size_t)t * H + n) = o;
  }
}

}  // namespace

size_t moe_workspace_bytes(int M, int top_k, int n_experts, int hidden, int inter) {
  size_t total = 0;
  carve(nullptr, M, top_k, n_experts, hidden, inter, &total);
  return total;
}

hipError_t launch_moe(const void* wg, const void* wu, const void* wd, int n_experts, int hidden, int inter,
                      const void* x, int M, const int32_t* ids, const float* p, int top_k, void* y, int inter_shift,
                      int out_shift, void* ws, int32_t* dev_error, hipStream_t stream, int down_fmt) {
  const int E = n_experts;
  const int n_slots = M * top_k;
  MoePlan pl = carve(ws, M, top_k, E, hidden, inter, nullptr);
  const bool one_block = n_slots <= kRouteOneBlockSlots;
  const _Float16* xh = static_cast<const _Float16*>(x);
  if (one_block) {
    // routing and staging in one launch (block 0 routes)
    const int groups = ((M + 8) / 8) * (hidden / QK);
    hipLaunchKernelGGL(k_moe_route, dim3(1 + (groups + 3) / 4), dim3(1024), 0, stream, ids, n_slots, E, dev_error,
                       pl.offsets, pl.tile_expert, pl.tile_start, pl.tile_rows, pl.n_tiles, pl.slots, pl.pos, MT_MOE,
                       xh, hidden, M, pl.xtok);
  } else {
    // counts and cursor are adjacent 256-byte-aligned arrays; zero both
    launch_fill_zero(reinterpret_cast<float*>(pl.counts),
                     (size_t)(reinterpret_cast<char*>(pl.offsets) - reinterpret_cast<char*>(pl.counts)) / 4, stream);
    const int sblocks = (n_slots + 255) / 256;
    hipLaunchKernelGGL(k_moe_count, dim3(sblocks), dim3(256), 0, stream, ids, n_slots, E, pl.counts, dev_error);
    hipLaunchKernelGGL(k_moe_plan, dim3(1), dim3(1024), 0, stream, pl.counts, E, pl.offsets, pl.tile_expert,
                       pl.tile_start, pl.tile_rows, pl.n_tiles, MT_MOE);
    hipLaunchKernelGGL(k_moe_scatter, dim3(sblocks), dim3(256), 0, stream, ids, n_slots, E, MT_MOE, pl.offsets, pl.cursor,
                       pl.slots, pl.pos);
    hipLaunchKernelGGL(k_stage_x16, dim3(M / 8 + 1, hidden / QK), dim3(256), 0, stream, xh, hidden, M, pl.xtok);
  }
  const int n_chunks = chunks_for(inter), n_chunks_small = chunks_small_for(inter);
  const int max_tiles = max_tiles_for(M, top_k, E);
  // both unit segments (tile counts known on the device only) padded to whole
  // groups of eight tiles: at most max_tiles * n_chunks_small + 8 * (n_chunks +
  // n_chunks_small) block ids
  const int grid = max_tiles * n_chunks_small + 8 * (n_chunks + n_chunks_small);
  auto fused = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(MoeCfg::THREADS), 0, stream,
                       static_cast<const uint8_t*>(wg), static_cast<const uint8_t*>(wu),
                       static_cast<const uint8_t*>(wd), hidden, inter, M, pl.xtok, top_k, pl.n_tiles, pl.tile_expert,
                       pl.tile_start, pl.tile_rows, pl.slots, pl.Q, n_slots, ldexpf(1.0f, -inter_shift),
                       ldexpf(1.0f, inter_shift - out_shift), n_chunks, n_chunks_small);
  };
  timing_begin(stream);
  if (down_fmt == kDownQ5K)
    fused(k_moe_fused16<kDownQ5K>);
  else if (down_fmt == kDownQ51)
    fused(k_moe_fused16<kDownQ51>);
  else
    fused(k_moe_fused16<kDownQ4K>);
  timing_end(stream);
  hipLaunchKernelGGL(k_moe_combine, dim3(M), dim3(256), 0, stream, pl.Q, pl.pos, p, top_k, n_chunks, n_chunks_small,
                     n_slots, hidden, static_cast<_Float16*>(y));
  return hipGetLastError();
}

}  // namespace zinc
