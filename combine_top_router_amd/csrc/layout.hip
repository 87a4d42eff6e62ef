// Dispatch layout: per-expert histogram, split plan, alignment-padded offsets
// and the stable expert-major permutation, all on the device with no host
// sync.
//
// What is computed follows the pages: the layout comes from topk_idx before
// any data moves (DeepEP issue #272, dispatch example: get_dispatch_layout);
// the histogram must not force a host sync (xtuner PR #2056, review
// comments: histc over bincount); the split plan is derived from the
// per-(source rank, expert) count matrix alone, whose row sums are the splits
// (DeepSpeed PR #8190, sections "Redundancy" and "Fix"); each local expert's
// rows are padded to the grouped-GEMM alignment (DeepSpeed AutoEP commit
// text, section "Attribution"); rows are named by the flat index
// token*top_k + slot (DeepSpeed PR #8847, section "Change").
//
// Up to 4096 assignments one workgroup does everything in one launch (see
// layout_fused_kernel): one CU is then as fast as the whole chip and two
// launches are saved. Beyond that, three kernels on one stream:
//   count   one workgroup per tile of flat assignments (tiles never cross a
//           source-rank boundary): LDS histogram over all experts.
//   scan    one workgroup: per-rank and per-expert totals, split matrix,
//           receive counts, padded offsets, and each tile's exclusive base
//           row per local expert.
//   scatter one workgroup per tile: ranks inside the tile from wavefront
//           ballots (lanes holding the same local expert find each other
//           with key_bits ballots, then popcount below their lane), in
//           flat-index order, so the permutation is stable and does not
//           depend on scheduling; writes dst_row and src_row, then marks the
//           padding and tail rows of src_row with -1.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

struct Ws {
  int32_t* tile_hist;  // [num_tiles, E]
  int32_t* tile_base;  // [num_tiles, e_loc]
  int32_t* lcount;     // [e_loc]
};

__host__ __device__ inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

Ws carve(const LayoutPlan& p, void* base) {
  char* c = static_cast<char*>(base);
  Ws w;
  w.tile_hist = reinterpret_cast<int32_t*>(c);
  c += round256(sizeof(int32_t) * size_t(p.num_tiles) * p.E);
  w.tile_base = reinterpret_cast<int32_t*>(c);
  c += round256(sizeof(int32_t) * size_t(p.num_tiles) * p.e_loc);
  w.lcount = reinterpret_cast<int32_t*>(c);
  return w;
}

__device__ __forceinline__ void tile_range(const LayoutPlan& p, int b, int64_t& start,
                                           int64_t& end) {
  const int s = b / p.tiles_per_rank, j = b % p.tiles_per_rank;
  start = s * p.chunk + int64_t(j) * p.tile;
  end = min(start + p.tile, int64_t(s + 1) * p.chunk);
}

__global__ __launch_bounds__(kThreads) void layout_count_kernel(LayoutPlan p,
                                                                const int32_t* __restrict__ idx,
                                                                int32_t* __restrict__ tile_hist) {
  extern __shared__ int32_t hist[];  // [E]
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < p.E; e += kThreads) hist[e] = 0;
  __syncthreads();
  int64_t start, end;
  tile_range(p, b, start, end);
  for (int64_t i = start + threadIdx.x; i < end; i += kThreads) {
    const int e = idx[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(p.E)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += kThreads) tile_hist[size_t(b) * p.E + e] = hist[e];
}

// Inclusive scan over a workgroup of 1024 threads (16 wavefronts).
__device__ int block_inclusive_scan_1024(int v, int* wave_tot) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) wave_tot[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) {
      const int t = wave_tot[i];
      wave_tot[i] = run;
      run += t;
    }
  }
  __syncthreads();
  return v + wave_tot[w];
}

__global__ __launch_bounds__(1024) void layout_scan_kernel(
    LayoutPlan p, const int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_base,
    int32_t* __restrict__ lcount_ws, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ send_counts, int32_t* __restrict__ split_matrix,
    int32_t* __restrict__ recv_counts, int32_t* __restrict__ output_splits,
    int32_t* __restrict__ offsets) {
  extern __shared__ int32_t sm[];
  int32_t* send = sm;                      // [ep, E]
  int32_t* lcount = send + p.ep * p.E;     // [e_loc]
  int32_t* wave_tot = lcount + p.e_loc;    // [16]
  const int tpr = p.tiles_per_rank;

  for (int e = threadIdx.x; e < p.E; e += 1024) {
    const bool loc = e >= p.first && e < p.first + p.e_loc;
    const int el = e - p.first;
    int total = 0;
    for (int s = 0; s < p.ep; ++s) {
      int rs = 0;
      int j = 0;
      for (; j + 4 <= tpr; j += 4) {  // four independent loads in flight
        const int b = s * tpr + j;
        int c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c[u] = tile_hist[size_t(b + u) * p.E + e];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (loc) tile_base[size_t(b + u) * p.e_loc + el] = total + rs;
          rs += c[u];
        }
      }
      for (; j < tpr; ++j) {
        const int b = s * tpr + j;
        const int c = tile_hist[size_t(b) * p.E + e];
        if (loc) tile_base[size_t(b) * p.e_loc + el] = total + rs;
        rs += c;
      }
      send[s * p.E + e] = rs;
      if (send_counts) send_counts[s * p.E + e] = rs;
      total += rs;
    }
    if (expert_counts) expert_counts[e] = total;
    if (loc) {
      lcount[el] = total;
      lcount_ws[el] = total;
    }
  }
  __syncthreads();

  if (recv_counts)
    for (int q = threadIdx.x; q < p.ep * p.e_loc; q += 1024)
      recv_counts[q] = send[(q / p.e_loc) * p.E + p.first + q % p.e_loc];
  if (output_splits)
    for (int s = threadIdx.x; s < p.ep; s += 1024) {
      int sum = 0;
      for (int el = 0; el < p.e_loc; ++el) sum += send[s * p.E + p.first + el];
      output_splits[s] = sum;
    }
  if (split_matrix) {
    const int eper = p.E / p.ep;
    for (int q = threadIdx.x; q < p.ep * p.ep; q += 1024) {
      const int s = q / p.ep, d = q % p.ep;
      int sum = 0;
      for (int e = 0; e < eper; ++e) sum += send[s * p.E + d * eper + e];
      split_matrix[q] = sum;
    }
  }

  // padded offsets over local experts (e_loc <= 1024)
  int padded = 0;
  if (threadIdx.x < p.e_loc) {
    const int c = lcount[threadIdx.x];
    padded = (c + p.align - 1) / p.align * p.align;
  }
  const int incl = block_inclusive_scan_1024(padded, wave_tot);
  if (threadIdx.x == 0) offsets[0] = 0;
  if (threadIdx.x < p.e_loc) offsets[threadIdx.x + 1] = incl;
}

template <int R>
__global__ __launch_bounds__(kThreads) void layout_scatter_kernel(
    LayoutPlan p, const int32_t* __restrict__ idx, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ lcount, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row, int64_t m_cap) {
  extern __shared__ int32_t sm[];
  const int el_n = p.e_loc;
  int32_t* cnt = sm;               // [4, e_loc]: running count per wavefront
  int32_t* wbase = sm + 4 * el_n;  // [4, e_loc]: exclusive prefix over wavefronts
  const int b = blockIdx.x;
  const int w = threadIdx.x / kWave, lane = lane_id();

  if (b < p.num_tiles) {
    for (int q = threadIdx.x; q < 4 * el_n; q += kThreads) cnt[q] = 0;
    __syncthreads();

    int64_t start, end;
    tile_range(p, b, start, end);
    const int64_t sub_start = start + int64_t(w) * (kWave * R);
    const int64_t sub_end = min(sub_start + kWave * R, end);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    int key[R], pre[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = sub_start + kWave * r + lane;
      const bool valid = i < sub_end;
      const int e = valid ? idx[i] : -1;
      const int el = (e >= p.first && e < p.first + el_n) ? e - p.first : el_n;
      key[r] = el;
      // lanes holding the same key: intersect ballots of each key bit
      uint64_t m = __ballot(valid);
      for (int bit = 0; bit < p.key_bits; ++bit) {
        const bool set = (el >> bit) & 1;
        const uint64_t bb = __ballot(set);
        m &= set ? bb : ~bb;
      }
      pre[r] = 0;
      if (el < el_n) {
        const int old = cnt[w * el_n + el];
        const int rank = __popcll(m & below);
        pre[r] = old + rank;
        if (rank == 0) cnt[w * el_n + el] = old + __popcll(m);
      }
    }
    __syncthreads();
    for (int el = threadIdx.x; el < el_n; el += kThreads) {
      int run = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wbase[q * el_n + el] = run;
        run += cnt[q * el_n + el];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = sub_start + kWave * r + lane;
      if (i >= sub_end) continue;
      const int el = key[r];
      if (el < el_n) {
        const int64_t row = int64_t(offsets[el]) + tile_base[size_t(b) * el_n + el] +
                            wbase[w * el_n + el] + pre[r];
        dst_row[i] = static_cast<int32_t>(row);
        if (row >= 0 && row < m_cap) src_row[row] = static_cast<int32_t>(i);
      } else {
        dst_row[i] = -1;
      }
    }
  }

  // padding rows of each local expert and the tail up to m_cap: -1
  for (int el = b; el < el_n; el += gridDim.x) {
    const int64_t hi = min(int64_t(offsets[el + 1]), m_cap);
    for (int64_t r = int64_t(offsets[el]) + lcount[el] + threadIdx.x; r < hi; r += kThreads)
      src_row[r] = -1;
  }
  for (int64_t r = int64_t(offsets[el_n]) + int64_t(b) * kThreads + threadIdx.x; r < m_cap;
       r += int64_t(gridDim.x) * kThreads)
    src_row[r] = -1;
}

// ---------------------------------------------------------------------------
// Single-workgroup layout for up to kFusedMaxN assignments: one launch does
// the histogram, the scan and the scatter. 16 wavefronts each own a
// contiguous segment of flat assignments. Pass 1 builds the per-(source
// rank, expert) histogram with LDS atomics and each wavefront's count per
// local expert with ballots; pass 2 turns them into totals, splits, padded
// offsets and each wavefront's first row per local expert; pass 3 re-reads
// the segment and assigns rows in flat-index order (ballot rank + the
// wavefront's running row), so the order is the same stable order as the
// tiled path.
constexpr int kFusedThreads = 1024, kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedMaxN = 4096;  // beyond this the tiled path is faster
constexpr int kFusedMaxHist = 16384, kFusedMaxLocal = 1024;
constexpr int kFusedBatch = 8;

__device__ __forceinline__ uint64_t match_mask(int key, int bits, bool valid) {
  uint64_t m = __ballot(valid);
  for (int bit = 0; bit < bits; ++bit) {
    const bool set = (key >> bit) & 1;
    const uint64_t bb = __ballot(set);
    m &= set ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(kFusedThreads) void layout_fused_kernel(
    LayoutPlan p, const int32_t* __restrict__ idx, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ send_counts, int32_t* __restrict__ split_matrix,
    int32_t* __restrict__ recv_counts, int32_t* __restrict__ output_splits,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row,
    int64_t m_cap) {
  __shared__ int32_t hist[kFusedMaxHist];                  // [ep, E]
  __shared__ int32_t wcnt[kFusedWaves * kFusedMaxLocal];   // [wave, e_loc]
  __shared__ int32_t lcnt[kFusedMaxLocal];
  __shared__ int32_t off[kFusedMaxLocal + 1];
  __shared__ int32_t wave_tot[kFusedWaves];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int el_n = p.e_loc, E = p.E;
  const int64_t N = p.T * p.k;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

  for (int q = tid; q < p.ep * E; q += kFusedThreads) hist[q] = 0;
  for (int q = tid; q < kFusedWaves * el_n; q += kFusedThreads) wcnt[q] = 0;
  __syncthreads();

  const int64_t seg = ((N + kFusedWaves - 1) / kFusedWaves + kWave - 1) / kWave * kWave;
  const int64_t s0 = int64_t(w) * seg, s1 = min(s0 + seg, N);
  int32_t* mycnt = wcnt + w * el_n;
  const uint32_t chunk32 = static_cast<uint32_t>(p.chunk);  // N < 2^31 on this path

  // pass 1: histograms. kBatch loads per lane are issued before any is used,
  // so a wavefront waits for one memory latency per kBatch*64 assignments.
  for (int64_t base = s0; base < s1; base += kWave * kFusedBatch) {
    int ev[kFusedBatch];
#pragma unroll
    for (int v = 0; v < kFusedBatch; ++v) {
      const int64_t i = base + v * kWave + lane;
      ev[v] = i < s1 ? idx[i] : -1;
    }
#pragma unroll
    for (int v = 0; v < kFusedBatch; ++v) {
      const int64_t i = base + v * kWave + lane;
      const bool valid = i < s1;
      const int e = ev[v];
      if (valid && static_cast<unsigned>(e) < static_cast<unsigned>(E))
        atomicAdd(&hist[int(uint32_t(i) / chunk32) * E + e], 1);
      const int el = (e >= p.first && e < p.first + el_n) ? e - p.first : el_n;
      const uint64_t m = match_mask(el, p.key_bits, valid);
      if (el < el_n && __popcll(m & below) == 0) mycnt[el] += __popcll(m);
    }
  }
  __syncthreads();

  // pass 2: totals, split plan, padded offsets, first row of each wavefront
  for (int e = tid; e < E; e += kFusedThreads) {
    int total = 0;
    for (int s = 0; s < p.ep; ++s) {
      const int c = hist[s * E + e];
      if (send_counts) send_counts[s * E + e] = c;
      total += c;
    }
    if (expert_counts) expert_counts[e] = total;
  }
  for (int el = tid; el < el_n; el += kFusedThreads) {
    int total = 0;
    for (int q = 0; q < kFusedWaves; ++q) total += wcnt[q * el_n + el];
    lcnt[el] = total;
  }
  if (recv_counts)
    for (int q = tid; q < p.ep * el_n; q += kFusedThreads)
      recv_counts[q] = hist[(q / el_n) * E + p.first + q % el_n];
  if (output_splits)
    for (int s = tid; s < p.ep; s += kFusedThreads) {
      int sum = 0;
      for (int el = 0; el < el_n; ++el) sum += hist[s * E + p.first + el];
      output_splits[s] = sum;
    }
  if (split_matrix) {
    const int eper = E / p.ep;
    for (int q = tid; q < p.ep * p.ep; q += kFusedThreads) {
      const int s = q / p.ep, d = q % p.ep;
      int sum = 0;
      for (int e = 0; e < eper; ++e) sum += hist[s * E + d * eper + e];
      split_matrix[q] = sum;
    }
  }
  __syncthreads();
  {
    const int padded = tid < el_n ? (lcnt[tid] + p.align - 1) / p.align * p.align : 0;
    const int incl = block_inclusive_scan_1024(padded, wave_tot);
    if (tid == 0) {
      off[0] = 0;
      offsets[0] = 0;
    }
    if (tid < el_n) {
      off[tid + 1] = incl;
      offsets[tid + 1] = incl;
    }
  }
  __syncthreads();
  for (int el = tid; el < el_n; el += kFusedThreads) {
    int run = off[el];
    for (int q = 0; q < kFusedWaves; ++q) {
      const int c = wcnt[q * el_n + el];
      wcnt[q * el_n + el] = run;
      run += c;
    }
  }
  __syncthreads();

  // pass 3: rows in flat-index order (chunks of 64 in order within a batch)
  for (int64_t base = s0; base < s1; base += kWave * kFusedBatch) {
    int ev[kFusedBatch];
#pragma unroll
    for (int v = 0; v < kFusedBatch; ++v) {
      const int64_t i = base + v * kWave + lane;
      ev[v] = i < s1 ? idx[i] : -1;
    }
#pragma unroll
    for (int v = 0; v < kFusedBatch; ++v) {
      const int64_t i = base + v * kWave + lane;
      const bool valid = i < s1;
      const int e = ev[v];
      const int el = (e >= p.first && e < p.first + el_n) ? e - p.first : el_n;
      const uint64_t m = match_mask(el, p.key_bits, valid);
      if (el < el_n) {
        const int old = mycnt[el];
        const int rank = __popcll(m & below);
        const int row = old + rank;
        if (rank == 0) mycnt[el] = old + __popcll(m);
        dst_row[i] = row;
        if (row >= 0 && row < m_cap) src_row[row] = static_cast<int32_t>(i);
      } else if (valid) {
        dst_row[i] = -1;
      }
    }
  }

  // padding rows of each local expert and the tail up to m_cap: -1
  for (int el = w; el < el_n; el += kFusedWaves) {
    const int64_t hi = min(int64_t(off[el + 1]), m_cap);
    for (int64_t r = int64_t(off[el]) + lcnt[el] + lane; r < hi; r += kWave) src_row[r] = -1;
  }
  for (int64_t r = int64_t(off[el_n]) + tid; r < m_cap; r += kFusedThreads) src_row[r] = -1;
}

}  // namespace

LayoutPlan make_layout_plan(int64_t T, int E, int k, int ep, int local_rank, int align) {
  LayoutPlan p{};
  p.T = T;
  p.E = E;
  p.k = k;
  p.ep = ep;
  p.align = align;
  p.first = local_rank < 0 ? 0 : local_rank * (E / ep);
  p.e_loc = local_rank < 0 ? E : E / ep;
  p.chunk = (T / ep) * k;
  const int64_t n = T * k;
  int tile = 1024;
  while (tile < 8192 && int64_t(tile) * 128 < n) tile *= 2;
  p.tile = tile;
  p.tiles_per_rank = static_cast<int>((p.chunk + tile - 1) / tile);
  p.num_tiles = ep * p.tiles_per_rank;
  int bits = 0;
  while ((1 << bits) <= p.e_loc) ++bits;  // keys 0..e_loc
  p.key_bits = bits;
  return p;
}

size_t layout_workspace_bytes(const LayoutPlan& p) {
  return round256(sizeof(int32_t) * size_t(p.num_tiles) * p.E) +
         round256(sizeof(int32_t) * size_t(p.num_tiles) * p.e_loc) +
         round256(sizeof(int32_t) * size_t(p.e_loc));
}

hipError_t launch_layout(const LayoutPlan& p, const int32_t* topk_idx, int32_t* expert_counts,
                         int32_t* send_counts, int32_t* split_matrix, int32_t* recv_counts,
                         int32_t* output_splits, int32_t* offsets, int32_t* dst_row,
                         int32_t* src_row, int64_t m_cap, void* ws_base, hipStream_t s) {
  if (p.T * p.k <= kFusedMaxN && int64_t(p.ep) * p.E <= kFusedMaxHist &&
      p.e_loc <= kFusedMaxLocal) {
    layout_fused_kernel<<<1, kFusedThreads, 0, s>>>(p, topk_idx, expert_counts, send_counts,
                                                    split_matrix, recv_counts, output_splits,
                                                    offsets, dst_row, src_row, m_cap);
    return hipGetLastError();
  }
  const Ws ws = carve(p, ws_base);
  if (p.num_tiles > 0) {
    layout_count_kernel<<<p.num_tiles, kThreads, sizeof(int32_t) * p.E, s>>>(p, topk_idx,
                                                                             ws.tile_hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const size_t scan_lds = sizeof(int32_t) * (size_t(p.ep) * p.E + p.e_loc + 16);
  layout_scan_kernel<<<1, 1024, scan_lds, s>>>(p, ws.tile_hist, ws.tile_base, ws.lcount,
                                               expert_counts, send_counts, split_matrix,
                                               recv_counts, output_splits, offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int grid = std::max(p.num_tiles, 1);
  const size_t lds = sizeof(int32_t) * 8 * size_t(p.e_loc);
  switch (p.tile / 1024) {
    case 1:
      layout_scatter_kernel<4><<<grid, kThreads, lds, s>>>(p, topk_idx, ws.tile_base, ws.lcount,
                                                           offsets, dst_row, src_row, m_cap);
      break;
    case 2:
      layout_scatter_kernel<8><<<grid, kThreads, lds, s>>>(p, topk_idx, ws.tile_base, ws.lcount,
                                                           offsets, dst_row, src_row, m_cap);
      break;
    case 4:
      layout_scatter_kernel<16><<<grid, kThreads, lds, s>>>(p, topk_idx, ws.tile_base, ws.lcount,
                                                            offsets, dst_row, src_row, m_cap);
      break;
    default:
      layout_scatter_kernel<32><<<grid, kThreads, lds, s>>>(p, topk_idx, ws.tile_base, ws.lcount,
                                                            offsets, dst_row, src_row, m_cap);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
