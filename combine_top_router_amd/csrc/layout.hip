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
// layout_fused_kernel): one CU is then as fast as the whole chip. Beyond that,
// two kernels on one stream:
//   count   one workgroup per tile of flat assignments (tiles never cross a
//           source-rank boundary): LDS histogram over all experts, written
//           out.
//   place   one workgroup per tile and one more. Each derives from the tile
//           histograms alone what its tile needs: every local expert's total
//           and padded offset, and the rows the earlier tiles hold; the extra
//           workgroup writes the split plan (per-rank and per-expert totals,
//           split matrix, receive counts). Then ranks inside the tile from
//           wavefront ballots (lanes holding the same local expert find each
//           other with key_bits ballots, then popcount below their lane), in
//           flat-index order, so the permutation is stable and does not
//           depend on scheduling; dst_row and src_row are written, and the
//           padding and tail rows of src_row get -1.
// No workgroup waits for or reads from another inside a launch: placing a row
// needs the totals of every tile, and a grid-wide wait would need a launch
// that guarantees every workgroup is resident, while exchanging data between
// workgroups of one launch costs a device-scope fence, which on this chip
// writes back and invalidates the whole L2 of the XCD. Tiles grow with the
// assignment count (128 to 256 of them), so the histograms each placing
// workgroup reads stay small.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;  // 16 wavefronts, both kernels of the tiled path
constexpr int kWavesPerGroup = kThreads / kWave;

__host__ __device__ inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

__device__ __forceinline__ void tile_range(const LayoutPlan& p, int b, int64_t& start,
                                           int64_t& end) {
  const int s = b / p.tiles_per_rank, j = b % p.tiles_per_rank;
  start = s * p.chunk + int64_t(j) * p.tile;
  end = min(start + p.tile, int64_t(s + 1) * p.chunk);
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

// As batched_run with NB loads in flight per batch: i = i0 .. i1-1, every
// load(i) of a batch issued before the batch's values are used, in order.
template <int NB, class L, class U>
__device__ __forceinline__ void batched_run_n(int i0, int i1, L&& load, U&& use) {
  for (int i = i0; i < i1; i += NB) {
    int v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = i + u < i1 ? load(i + u) : 0;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i + u < i1) use(i + u, v[u]);
  }
}

// One workgroup per tile of flat assignments (tiles never cross a
// source-rank boundary): LDS histogram over all experts, written out. Each
// thread's expert ids are loaded eight at a time before any is counted.
__global__ __launch_bounds__(kThreads) void layout_count_kernel(LayoutPlan p,
                                                                const int32_t* __restrict__ idx,
                                                                int32_t* __restrict__ tile_hist) {
  extern __shared__ int32_t hist[];  // [E]
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < p.E; e += kThreads) hist[e] = 0;
  __syncthreads();
  int64_t start, end;
  tile_range(p, b, start, end);
  for (int64_t i0 = start + threadIdx.x; i0 < end; i0 += 8 * int64_t(kThreads)) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + int64_t(u) * kThreads;
      ev[u] = i < end ? idx[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (static_cast<unsigned>(ev[u]) < static_cast<unsigned>(p.E)) atomicAdd(&hist[ev[u]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += kThreads) tile_hist[size_t(b) * p.E + e] = hist[e];
}

// The split plan (per-rank and per-expert totals, split matrix, receive
// counts, output splits) from the tile histograms, by the one workgroup past
// the tiles of the place kernel. Thread (g, e), g < 1024 / E, sums a run of
// tile rows of expert e, source rank by source rank, into LDS.
__device__ void layout_split_plan(const LayoutPlan& p, const int32_t* __restrict__ tile_hist,
                                  int32_t* __restrict__ expert_counts,
                                  int32_t* __restrict__ send_counts,
                                  int32_t* __restrict__ split_matrix,
                                  int32_t* __restrict__ recv_counts,
                                  int32_t* __restrict__ output_splits, int32_t* send) {
  const int tid = threadIdx.x, E = p.E, el_n = p.e_loc, nt = p.num_tiles;
  for (int q = tid; q < p.ep * E; q += kThreads) send[q] = 0;
  __syncthreads();
  const int G = kThreads / E, e = tid % E, g = tid / E;
  if (g < G) {
    const int per = (nt + G - 1) / G, b0 = min(nt, g * per), b1 = min(nt, b0 + per);
    int rank_sum = 0, cur = b0 < b1 ? b0 / p.tiles_per_rank : 0;
    batched_run_n<32>(b0, b1, [&](int b) { return tile_hist[size_t(b) * E + e]; }, [&](int b, int v) {
      const int s = b / p.tiles_per_rank;
      if (s != cur) {
        atomicAdd(&send[cur * E + e], rank_sum);
        rank_sum = 0;
        cur = s;
      }
      rank_sum += v;
    });
    if (b0 < b1) atomicAdd(&send[cur * E + e], rank_sum);
  }
  __syncthreads();
  if (send_counts)
    for (int q = tid; q < p.ep * E; q += kThreads) send_counts[q] = send[q];
  if (expert_counts)
    for (int e2 = tid; e2 < E; e2 += kThreads) {
      int t = 0;
      for (int s = 0; s < p.ep; ++s) t += send[s * E + e2];
      expert_counts[e2] = t;
    }
  if (recv_counts)
    for (int q = tid; q < p.ep * el_n; q += kThreads)
      recv_counts[q] = send[(q / el_n) * E + p.first + q % el_n];
  if (output_splits)
    for (int s = tid; s < p.ep; s += kThreads) {
      int sum = 0;
      for (int el = 0; el < el_n; ++el) sum += send[s * E + p.first + el];
      output_splits[s] = sum;
    }
  if (split_matrix) {
    const int eper = E / p.ep;
    for (int q = tid; q < p.ep * p.ep; q += kThreads) {
      const int s = q / p.ep, d = q % p.ep;
      int sum = 0;
      for (int e2 = 0; e2 < eper; ++e2) sum += send[s * E + d * eper + e2];
      split_matrix[q] = sum;
    }
  }
}

// One workgroup per tile, plus one for the split plan. Each first derives,
// from the tile histograms alone, every local expert's total and padded
// offset and the rows its tile's predecessors hold (thread (g, el) sums a run
// of tile rows; the tile histograms are small and stay in L2), so no
// workgroup depends on another. Then the tile's rows: ranks inside the tile
// from wavefront ballots (lanes holding the same local expert find each other
// with key_bits ballots, then popcount below their lane), in flat-index
// order, so the permutation is stable and does not depend on scheduling; a
// tile of more than 1024 * R assignments is walked in passes of that many,
// each expert's next row carried from pass to pass. Last, the padding and
// tail rows of src_row get -1.
template <int R>
__global__ __launch_bounds__(kThreads) void layout_place_kernel(
    LayoutPlan p, const int32_t* __restrict__ idx, const int32_t* __restrict__ tile_hist,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ send_counts,
    int32_t* __restrict__ split_matrix, int32_t* __restrict__ recv_counts,
    int32_t* __restrict__ output_splits, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row, int64_t m_cap) {
  extern __shared__ int32_t sm[];
  const int el_n = p.e_loc, nt = p.num_tiles, b = blockIdx.x;
  const int w = threadIdx.x / kWave, lane = lane_id(), tid = threadIdx.x;
  if (b == nt) {  // the split plan, in its own workgroup, and nothing else
    layout_split_plan(p, tile_hist, expert_counts, send_counts, split_matrix, recv_counts,
                      output_splits, sm);
    return;
  }
  const int G = kThreads / el_n;                // runs of tile rows per expert (>= 1)
  // LDS: the run sums [2, G, e_loc] of the offset pass, then the per-wavefront
  // counts [16, e_loc] in the same words; after both, base, offsets, totals
  const int head = max(kWavesPerGroup * el_n, 2 * G * el_n);
  int32_t* part = sm;
  int32_t* cnt = sm;
  int32_t* base = sm + head;                    // [e_loc]: the next row of each local expert
  int32_t* off = base + el_n;                   // [e_loc + 1]: padded offsets
  int32_t* total = off + el_n + 1;              // [e_loc]
  int32_t* wave_tot = total + el_n;             // [16]

  // this wavefront's expert ids of a pass, loaded a pass ahead; the first
  // pass's go out now, so they arrive while the offsets are derived
  int64_t start, end;
  tile_range(p, b, start, end);
  auto load_ids = [&](int64_t pass, int (&ev)[R]) {
    const int64_t sub_start = pass + int64_t(w) * (kWave * R);
    const int64_t sub_end = min(sub_start + kWave * R, end);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = sub_start + kWave * r + lane;
      ev[r] = i < sub_end ? idx[i] : -1;
    }
  };
  int nxt[R];
  load_ids(start, nxt);

  // totals, padded offsets and this tile's first row of each local expert
  {
    const int el = tid % el_n, g = tid / el_n;
    if (g < G) {
      const int per = (nt + G - 1) / G, b0 = min(nt, g * per), b1 = min(nt, b0 + per);
      const int32_t* col = tile_hist + p.first + el;
      int tot = 0, before = 0;
      batched_run_n<32>(b0, b1, [&](int bb) { return col[size_t(bb) * p.E]; }, [&](int bb, int v) {
        tot += v;
        if (bb < b) before += v;
      });
      part[g * el_n + el] = tot;
      part[(G + g) * el_n + el] = before;
    }
    __syncthreads();
    int padded = 0, before = 0;
    if (tid < el_n) {
      int t = 0;
      for (int g2 = 0; g2 < G; ++g2) {
        t += part[g2 * el_n + tid];
        before += part[(G + g2) * el_n + tid];
      }
      total[tid] = t;
      padded = (t + p.align - 1) / p.align * p.align;
    }
    const int incl = block_inclusive_scan_1024(padded, wave_tot);
    if (tid == 0) off[0] = 0;
    if (tid < el_n) {
      off[tid + 1] = incl;
      base[tid] = incl - padded + before;
    }
    if (b == 0) {
      if (tid == 0) offsets[0] = 0;
      if (tid < el_n) offsets[tid + 1] = incl;
    }
    __syncthreads();
  }

  {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    for (int64_t pass = start; pass < end; pass += int64_t(kThreads) * R) {
      int ev[R];
#pragma unroll
      for (int r = 0; r < R; ++r) ev[r] = nxt[r];
      if (pass + int64_t(kThreads) * R < end) load_ids(pass + int64_t(kThreads) * R, nxt);
      for (int q = tid; q < kWavesPerGroup * el_n; q += kThreads) cnt[q] = 0;
      __syncthreads();
      const int64_t sub_start = pass + int64_t(w) * (kWave * R);
      const int64_t sub_end = min(sub_start + kWave * R, end);

      int key[R], pre[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t i = sub_start + kWave * r + lane;
        const bool valid = i < sub_end;
        const int e = ev[r];
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
        if (valid && el < el_n) {
          const int old = cnt[w * el_n + el];
          const int rank = __popcll(m & below);
          pre[r] = old + rank;
          if (rank == 0) cnt[w * el_n + el] = old + __popcll(m);
        }
      }
      __syncthreads();
      // exclusive prefix over the wavefronts, per local expert, from the
      // expert's next row; the total moves that row on for the next pass
      for (int el = tid; el < el_n; el += kThreads) {
        int run = base[el];
        for (int q = 0; q < kWavesPerGroup; ++q) {
          const int c = cnt[q * el_n + el];
          cnt[q * el_n + el] = run;
          run += c;
        }
        base[el] = run;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t i = sub_start + kWave * r + lane;
        if (i >= sub_end) continue;
        const int el = key[r];
        if (el < el_n) {
          const int64_t row = int64_t(cnt[w * el_n + el]) + pre[r];
          dst_row[i] = static_cast<int32_t>(row);
          if (row >= 0 && row < m_cap) src_row[row] = static_cast<int32_t>(i);
        } else {
          dst_row[i] = -1;
        }
      }
      __syncthreads();  // cnt read out before the next pass clears it
    }
  }

  // padding rows of each local expert and the tail up to m_cap: -1
  for (int el = b; el < el_n; el += nt) {
    const int64_t hi = min(int64_t(off[el + 1]), m_cap);
    for (int64_t r = int64_t(off[el]) + total[el] + tid; r < hi; r += kThreads) src_row[r] = -1;
  }
  for (int64_t r = int64_t(off[el_n]) + int64_t(b) * kThreads + tid; r < m_cap;
       r += int64_t(nt) * kThreads)
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
  // about 128 tiles, 256 past 2^21 assignments (each placing workgroup reads
  // every tile's local-expert counts; past that size, passes over its own
  // tile cost more than those reads)
  const int64_t target = n > (int64_t(1) << 21) ? 256 : 128;
  int tile = 1024;
  while (tile < (1 << 20) && int64_t(tile) * target < n) tile *= 2;
  p.tile = tile;
  p.tiles_per_rank = static_cast<int>((p.chunk + tile - 1) / tile);
  p.num_tiles = ep * p.tiles_per_rank;
  int bits = 0;
  while ((1 << bits) <= p.e_loc) ++bits;  // keys 0..e_loc
  p.key_bits = bits;
  return p;
}

size_t layout_workspace_bytes(const LayoutPlan& p) {
  return round256(sizeof(int32_t) * size_t(p.num_tiles) * p.E);
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
  int32_t* tile_hist = static_cast<int32_t*>(ws_base);
  layout_count_kernel<<<p.num_tiles, kThreads, sizeof(int32_t) * p.E, s>>>(p, topk_idx,
                                                                           tile_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // LDS of the place kernel: the per-wavefront counts (also the run sums of
  // the offset pass, 2 x (1024 / e_loc) x e_loc <= 2048), base, offsets,
  // totals, wave totals; the split-plan workgroup reuses it for [ep, E]
  const size_t el = size_t(p.e_loc);
  const size_t head = std::max(kWavesPerGroup * el, size_t(2 * (kThreads / p.e_loc)) * el);
  const size_t words = std::max(head + 3 * el + 1 + 16, size_t(p.ep) * p.E);
  const size_t lds = sizeof(int32_t) * words;
  auto big_lds = [&](const void* f) {
    if (lds > (64u << 10))
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  };
  const int grid = p.num_tiles + 1;
  switch (std::min(p.tile / 1024, 8)) {
#define MOE_PLACE(RR)                                                                      \
  case RR:                                                                                 \
    big_lds(reinterpret_cast<const void*>(layout_place_kernel<RR>));                       \
    layout_place_kernel<RR><<<grid, kThreads, lds, s>>>(                                   \
        p, topk_idx, tile_hist, expert_counts, send_counts, split_matrix, recv_counts,     \
        output_splits, offsets, dst_row, src_row, m_cap);                                  \
    break;
    MOE_PLACE(1)
    MOE_PLACE(2)
    MOE_PLACE(4)
    default:
    MOE_PLACE(8)
#undef MOE_PLACE
  }
  return hipGetLastError();
}

}  // namespace moe
