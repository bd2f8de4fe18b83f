// Batched-expert MoE MLP: y[t] = sum_s p[t,s] * MLP_{ids[t,s]}(x[t]).
//
// The expert ids and mixing weights stay on the GPU.  The host launches a
// fixed sequence of kernels sized only by (M, top_k, n_experts) -- never by the
// routing -- so nothing is read back mid-call ("Four bottlenecks, one CUDA
// backend", "Bottleneck 2": batched-expert kernels read the chosen expert ids
// from a GPU buffer and index the expert weights themselves):
//   1. k_moe_count    per-expert slot counts; invalid ids set *dev_error
//   2. k_moe_plan     exclusive scan of the counts -> list offsets, and the tile
//                     table (expert, first list entry, rows) of MT-slot tiles
//   3. k_moe_scatter  slot indices grouped by expert, and each slot's position
//   4. k_moe_fused    one fused unit per (tile, intermediate chunk); blocks past
//                     the device-side tile count exit at once.  Each row's
//                     expert output, times p[t,s], is stored (fp32) at the
//                     row's list position: Q[chunk][position][hidden]
//   5. k_moe_combine  y[t] = fp16(sum over chunks and the token's slots)
// No atomics: every partial has exactly one writer, and the combine order is
// fixed, so the result is deterministic.
#include "fused_core.hpp"
#include "launch.hpp"
#include "util_kernels.hpp"

namespace zinc {

namespace {

constexpr int TT_MOE = 1;       // 32 (token, slot) rows per unit
constexpr int RTW_MOE = 1;      // row tiles per wave per pass
constexpr int ICMAX_MOE = 384;  // intermediate rows per chunk
using MoeCfg = FusedCfg<TT_MOE, RTW_MOE, ICMAX_MOE>;

struct MoePlan {
  int* counts;       // [E]
  int* cursor;       // [E]
  int* offsets;      // [E + 1]
  int* tile_expert;  // [max_tiles]
  int* tile_start;   // [max_tiles]
  int* tile_rows;    // [max_tiles]
  int* n_tiles;      // [1]
  int* slots;        // [M * top_k] slot indices grouped by expert
  int* pos;          // [M * top_k] list position of each slot, -1 if its id is invalid
  float* Q;          // [n_chunks][M * top_k][H]
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int max_tiles_for(int M, int top_k, int E) {
  const long long pairs = (long long)M * top_k;
  return (int)((pairs + MoeCfg::MT - 1) / MoeCfg::MT + (pairs < E ? pairs : E));
}

int chunks_for(int I) {
  const int npan = I / 64;
  return (npan + ICMAX_MOE / 64 - 1) / (ICMAX_MOE / 64);
}

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
  p.n_tiles = reinterpret_cast<int*>(take(sizeof(int)));
  p.slots = reinterpret_cast<int*>(take(sizeof(int) * pairs));
  p.pos = reinterpret_cast<int*>(take(sizeof(int) * pairs));
  p.Q = reinterpret_cast<float*>(take(sizeof(float) * (size_t)chunks_for(I) * pairs * H));
  if (total) *total = off;
  return p;
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

// One block of 1024 threads; E <= 1024.
__global__ __launch_bounds__(1024) void k_moe_plan(const int* __restrict__ counts, int E, int* __restrict__ offsets,
                                                  int* __restrict__ tile_expert, int* __restrict__ tile_start,
                                                  int* __restrict__ tile_rows, int* __restrict__ n_tiles, int MT) {
  __shared__ int sc[1024];
  __shared__ int st[1024];
  const int e = threadIdx.x;
  const int cnt = (e < E) ? counts[e] : 0;
  const int nt = (cnt + MT - 1) / MT;
  sc[e] = cnt;
  st[e] = nt;
  __syncthreads();
  // inclusive Hillis-Steele scans of counts and tile counts
  for (int d = 1; d < 1024; d <<= 1) {
    const int a = (e >= d) ? sc[e - d] : 0;
    const int b = (e >= d) ? st[e - d] : 0;
    __syncthreads();
    sc[e] += a;
    st[e] += b;
    __syncthreads();
  }
  const int off = sc[e] - cnt;      // exclusive
  const int tb = st[e] - nt;
  if (e < E) offsets[e] = off;
  if (e == E - 1) {
    offsets[E] = sc[e];
    *n_tiles = st[e];
  }
  for (int i = 0; i < nt; ++i) {
    tile_expert[tb + i] = e;
    tile_start[tb + i] = off + i * MT;
    tile_rows[tb + i] = min(MT, cnt - i * MT);
  }
}

__global__ __launch_bounds__(256) void k_moe_scatter(const int32_t* __restrict__ ids, int n_slots, int E,
                                                    const int* __restrict__ offsets, int* __restrict__ cursor,
                                                    int* __restrict__ slots, int* __restrict__ pos) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_slots) return;
  const int e = ids[i];
  if (e < 0 || e >= E) {
    pos[i] = -1;
    return;
  }
  const int q = offsets[e] + atomicAdd(cursor + e, 1);
  slots[q] = i;
  pos[i] = q;
}

// MoE output: row r of a unit is list position row0 + r; store w * v at Q[chunk][position][n].
struct OutPairs {
  float* Q;
  size_t pairs;
  int H;
  __device__ __forceinline__ void put(int chunk, int n, int position, int tok, float w, float v) const {
    if (tok >= 0) Q[((size_t)chunk * pairs + position) * H + n] = w * v;
  }
};

__global__ __launch_bounds__(MoeCfg::THREADS) void k_moe_fused(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
                                                          const uint8_t* __restrict__ wd, int H, int I,
                                                          const _Float16* __restrict__ x, const float* __restrict__ p,
                                                          int top_k, const int* __restrict__ n_tiles,
                                                          const int* __restrict__ tile_expert,
                                                          const int* __restrict__ tile_start,
                                                          const int* __restrict__ tile_rows,
                                                          const int* __restrict__ slots, float* __restrict__ Q,
                                                          int pairs, float inter_scale, int n_chunks) {
  __shared__ __attribute__((aligned(16))) FusedSmem<TT_MOE, RTW_MOE, ICMAX_MOE> sm;
  __shared__ int tok[MoeCfg::MT];
  __shared__ float wrow[MoeCfg::MT];

  // A tile's chunks have consecutive block ids and so spread over the XCDs
  // (ids go round-robin over them); with n_chunks a multiple of 8, one chunk of
  // every tile lands on the same XCD, whose L2 then serves that slice of an
  // expert's weights to all of the expert's tiles.
  const int ti = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x % n_chunks;
  if (ti >= *n_tiles) return;
  const int e = tile_expert[ti];
  const int start = tile_start[ti], rows = tile_rows[ti];
  if (threadIdx.x < MoeCfg::MT) {
    int t = -1;
    float w = 0.0f;
    if ((int)threadIdx.x < rows) {
      const int slot = slots[start + threadIdx.x];
      t = slot / top_k;
      w = p[slot];
    }
    tok[threadIdx.x] = t;
    wrow[threadIdx.x] = w;
  }
  __syncthreads();
  const int npan = I / 64;
  const int r0 = (int)((long long)chunk * npan / n_chunks) * 64;
  const int r1 = (int)((long long)(chunk + 1) * npan / n_chunks) * 64;
  const size_t gu_bytes = (size_t)I * (H / QK) * BLOCK_BYTES;   // one expert's gate (or up) matrix
  const size_t d_bytes = (size_t)H * (I / QK) * BLOCK_BYTES;    // one expert's down matrix
  OutPairs out{Q, (size_t)pairs, H};
  fused_unit<TT_MOE, RTW_MOE, ICMAX_MOE>(wg + e * gu_bytes, wu + e * gu_bytes, wd + e * d_bytes, H, I, x, tok, wrow,
                                         chunk, r0, r1, start, inter_scale, out, sm);
}

// y[t][n] = fp16(scale * sum_c sum_s Q[c][pos[t*k+s]][n]); one block per token.
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ Q, const int* __restrict__ pos,
                                                    int top_k, int n_chunks, int pairs, int H,
                                                    _Float16* __restrict__ y, float scale) {
  const int t = blockIdx.x;
  for (int n = threadIdx.x * 4; n < H; n += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < top_k; ++s) {
      const int q = pos[t * top_k + s];
      if (q < 0) continue;
      for (int c = 0; c < n_chunks; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(Q + ((size_t)c * pairs + q) * H + n);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
    }
    _Float16* yr = y + (size_t)t * H + n;
    yr[0] = (_Float16)(acc.x * scale);
    yr[1] = (_Float16)(acc.y * scale);
    yr[2] = (_Float16)(acc.z * scale);
    yr[3] = (_Float16)(acc.w * scale);
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
                      int out_shift, void* ws, int32_t* dev_error, hipStream_t stream) {
  const int E = n_experts;
  const int n_slots = M * top_k;
  MoePlan pl = carve(ws, M, top_k, E, hidden, inter, nullptr);
  // counts and cursor are adjacent 256-byte-aligned arrays; zero both
  launch_fill_zero(reinterpret_cast<float*>(pl.counts),
                   (size_t)(reinterpret_cast<char*>(pl.offsets) - reinterpret_cast<char*>(pl.counts)) / 4, stream);
  const int sblocks = (n_slots + 255) / 256;
  hipLaunchKernelGGL(k_moe_count, dim3(sblocks), dim3(256), 0, stream, ids, n_slots, E, pl.counts, dev_error);
  hipLaunchKernelGGL(k_moe_plan, dim3(1), dim3(1024), 0, stream, pl.counts, E, pl.offsets, pl.tile_expert,
                     pl.tile_start, pl.tile_rows, pl.n_tiles, MoeCfg::MT);
  hipLaunchKernelGGL(k_moe_scatter, dim3(sblocks), dim3(256), 0, stream, ids, n_slots, E, pl.offsets, pl.cursor,
                     pl.slots, pl.pos);
  const int n_chunks = chunks_for(inter);
  const int max_tiles = max_tiles_for(M, top_k, E);
  timing_begin(stream);
  hipLaunchKernelGGL(k_moe_fused, dim3(max_tiles * n_chunks), dim3(MoeCfg::THREADS), 0, stream,
                     static_cast<const uint8_t*>(wg), static_cast<const uint8_t*>(wu),
                     static_cast<const uint8_t*>(wd), hidden, inter, static_cast<const _Float16*>(x), p, top_k,
                     pl.n_tiles, pl.tile_expert, pl.tile_start, pl.tile_rows, pl.slots, pl.Q, n_slots,
                     ldexpf(1.0f, -inter_shift), n_chunks);
  timing_end(stream);
  hipLaunchKernelGGL(k_moe_combine, dim3(M), dim3(256), 0, stream, pl.Q, pl.pos, top_k, n_chunks, n_slots, hidden,
                     static_cast<_Float16*>(y), ldexpf(1.0f, inter_shift - out_shift));
  return hipGetLastError();
}

}  // namespace zinc
