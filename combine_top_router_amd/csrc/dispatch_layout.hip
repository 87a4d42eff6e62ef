// Per-rank deduplicated dispatch layout.
//
// DeepEP computes, from topk_idx and the expert count and before any data
// moves, the tokens per rank, the tokens per expert and a token-in-rank
// table that its dispatch consumes (DeepEP issue #272, the maintainer's
// example around get_dispatch_layout). A token goes once to each rank that
// holds at least one of its experts; rank r holds experts
// [r*E/ep, (r+1)*E/ep). Outputs:
//   is_token_in_rank [T, ep] uint8, num_tokens_per_rank [ep],
//   num_tokens_per_expert [E], token_rank_pos [T, ep] (position of t among
//   the tokens rank r receives, in token order; -1 if not sent).
//
// Three launches on one stream, one thread per token:
//   count  per tile of 256 tokens: each rank's tokens (wavefront ballots over
//          the token's rank mask) and an LDS histogram of expert ids;
//   scan   one workgroup: per-rank exclusive scan over tiles, per-expert sums;
//   place  per tile: the token's position = tile base + tokens of the tile
//          before it (ballot prefix within the wavefront + earlier wavefronts).
// Integer sums only, no atomics across workgroups: the result does not
// depend on scheduling.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTile = 256;  // tokens per workgroup, one per thread
constexpr int kTileWaves = kTile / kWave;

struct DlArgs {
  const int32_t* idx;
  int64_t T;
  int E, k, ep, el;
  int tiles;
  int32_t* tile_rank;    // [tiles, ep]  counts, then exclusive bases
  int32_t* tile_expert;  // [tiles, E]
};

__device__ __forceinline__ uint64_t rank_mask(const DlArgs& a, int64_t t) {
  uint64_t m = 0;
  if (t < a.T) {
    for (int s = 0; s < a.k; ++s) {
      const int e = a.idx[t * a.k + s];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(a.E)) m |= 1ull << (e / a.el);
    }
  }
  return m;
}

__global__ __launch_bounds__(kTile) void dl_count_kernel(DlArgs a) {
  __shared__ int32_t hist[1024];
  __shared__ int32_t wave_cnt[kTileWaves][64];
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int tile = blockIdx.x;
  for (int e = tid; e < a.E; e += kTile) hist[e] = 0;
  __syncthreads();
  const int64_t t = int64_t(tile) * kTile + tid;
  if (t < a.T)
    for (int s = 0; s < a.k; ++s) {
      const int e = a.idx[t * a.k + s];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(a.E)) atomicAdd(&hist[e], 1);
    }
  const uint64_t m = rank_mask(a, t);
  for (int r = 0; r < a.ep; ++r) {
    const uint64_t b = __ballot((m >> r) & 1);
    if (lane == 0) wave_cnt[w][r] = __popcll(b);
  }
  __syncthreads();
  for (int r = tid; r < a.ep; r += kTile) {
    int c = 0;
    for (int q = 0; q < kTileWaves; ++q) c += wave_cnt[q][r];
    a.tile_rank[size_t(tile) * a.ep + r] = c;
  }
  for (int e = tid; e < a.E; e += kTile) a.tile_expert[size_t(tile) * a.E + e] = hist[e];
}

// Threads per row when `rows` rows share 1024 threads over `n` tiles each: the
// fewest (a power of two) that leave every thread at most one batch of 8.
__device__ __forceinline__ int group_size(int rows, int n) {
  int P = 1;
  while (P * 2 * rows <= 1024 && P * 8 < n) P *= 2;
  return P;
}

// One workgroup: rank r's tile counts become exclusive bases over the tiles in
// order, and expert e's tile counts are summed. Each rank (then each expert)
// gets a group of P threads (group_size), each thread a contiguous run of
// tiles loaded in batches of independent loads; the run sums are then scanned
// (ranks) or reduced (experts) across the group in LDS.
__global__ __launch_bounds__(1024) void dl_scan_kernel(DlArgs a, int32_t* per_rank,
                                                      int32_t* per_expert) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  {
    const int P = group_size(a.ep, a.tiles);
    const int r = tid / P, p = tid % P;
    const int C = (a.tiles + P - 1) / P;
    const int j0 = min(a.tiles, p * C), j1 = min(a.tiles, j0 + C);
    int sum = 0;
    if (r < a.ep)
      batched_run(j0, j1, [&](int j) { return a.tile_rank[size_t(j) * a.ep + r]; },
                  [&](int, int c) { sum += c; });
    part[tid] = sum;
    __syncthreads();
    // inclusive prefix of the run sums within each group (Hillis-Steele)
    for (int off = 1; off < P; off <<= 1) {
      const int v = p >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    if (r < a.ep) {
      int run = part[tid] - sum;
      batched_run(j0, j1, [&](int j) { return a.tile_rank[size_t(j) * a.ep + r]; },
                  [&](int j, int c) {
                    a.tile_rank[size_t(j) * a.ep + r] = run;
                    run += c;
                  });
      if (p == P - 1) per_rank[r] = part[tid];
    }
    __syncthreads();
  }
  {
    const int P = group_size(a.E, a.tiles);
    const int e = tid / P, p = tid % P;
    const int C = (a.tiles + P - 1) / P;
    const int j0 = min(a.tiles, p * C), j1 = min(a.tiles, j0 + C);
    int sum = 0;
    if (e < a.E)
      batched_run(j0, j1, [&](int j) { return a.tile_expert[size_t(j) * a.E + e]; },
                  [&](int, int c) { sum += c; });
    part[tid] = sum;
    __syncthreads();
    for (int off = P / 2; off >= 1; off >>= 1) {
      if (p < off) part[tid] += part[tid + off];
      __syncthreads();
    }
    if (e < a.E && p == 0) per_expert[e] = part[tid];
  }
}

__global__ __launch_bounds__(kTile) void dl_place_kernel(DlArgs a, uint8_t* in_rank,
                                                       int32_t* pos) {
  __shared__ int32_t wave_cnt[kTileWaves][64];
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int tile = blockIdx.x;
  const int64_t t = int64_t(tile) * kTile + tid;
  const uint64_t m = rank_mask(a, t);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  for (int r = 0; r < a.ep; ++r) {
    const uint64_t b = __ballot((m >> r) & 1);
    if (lane == 0) wave_cnt[w][r] = __popcll(b);
  }
  __syncthreads();
  for (int r = 0; r < a.ep; ++r) {
    // every lane takes part in the ballot; only tokens < T write
    const uint64_t b = __ballot((m >> r) & 1);
    const bool sent = (m >> r) & 1;
    int before = a.tile_rank[size_t(tile) * a.ep + r] + __popcll(b & below);
    for (int q = 0; q < w; ++q) before += wave_cnt[q][r];
    if (t < a.T) {
      in_rank[t * a.ep + r] = sent ? 1 : 0;
      pos[t * a.ep + r] = sent ? before : -1;
    }
  }
}

}  // namespace

size_t dispatch_layout_workspace_bytes(int64_t T, int E, int ep) {
  const int64_t tiles = (T + kTile - 1) / kTile;
  return size_t(tiles) * size_t(ep + E) * sizeof(int32_t);
}

hipError_t launch_dispatch_layout(const int32_t* idx, int64_t T, int E, int k, int ep,
                                  int32_t* per_rank, int32_t* per_expert, uint8_t* in_rank,
                                  int32_t* pos, void* ws, hipStream_t s) {
  DlArgs a{};
  a.idx = idx, a.T = T, a.E = E, a.k = k, a.ep = ep, a.el = E / ep;
  a.tiles = static_cast<int>((T + kTile - 1) / kTile);
  a.tile_rank = static_cast<int32_t*>(ws);
  a.tile_expert = a.tile_rank + size_t(a.tiles) * ep;
  if (a.tiles > 0) dl_count_kernel<<<a.tiles, kTile, 0, s>>>(a);
  dl_scan_kernel<<<1, 1024, 0, s>>>(a, per_rank, per_expert);
  if (a.tiles > 0) dl_place_kernel<<<a.tiles, kTile, 0, s>>>(a, in_rank, pos);
  return hipGetLastError();
}

}  // namespace moe
