// Grouped expert GEMMs over ragged expert groups on the gfx950 matrix cores.
//
// The local grouped expert compute of the AutoEP flow (DeepSpeed AutoEP
// commit text, sections "Attribution": GroupedExperts / grouped-GEMM
// execution, and "Design", runtime step 5), in bf16 as the pages' grouped
// GEMM (DeepSpeed PR #8847, section "Tests": torch._grouped_mm, bf16 only).
// It is the only dense contraction of the layer, so it is the only stage on
// MFMA:
//
//   gate_up:  h[r] = silu(x[r] W1[e]) * (x[r] W3[e])   two B operands, SwiGLU fused
//             into the epilogue (fp32), h stored once as bf16
//   down:     y[r] = h[r] W2[e]
//
// for the rows r of local expert e, [offsets[e], offsets[e] + counts[e]).
//
// Design (MI355X / CDNA4):
//  * v_mfma_f32_32x32x16_bf16: a wavefront multiplies a 32x16 A slice by a
//    16x32 B slice into 32x32 fp32 accumulators; each lane feeds 8
//    consecutive K values of one row of A and one row of B^T, so both
//    operands are read K-contiguous (forward weights are repacked once,
//    output-major and cut into K-slices that are each one contiguous run).
//  * 8 wavefronts per workgroup (2 per SIMD), each owning TM 32-row blocks
//    of accumulators. The main tile is 320 rows x 256 staged B rows, waves 2
//    (rows) x 4 (columns), 160 rows x 64 B rows each: 160 accumulator VGPRs,
//    the most two wavefronts per SIMD can hold beside their fragments. 320
//    rows rather than 256 because expert groups a little over 256 rows (the
//    usual case at 256 tokens per expert) then stay one tile instead of two
//    tiles of half height. The gated pair stages 128 gate + 128 up rows for
//    128 output columns, so one epilogue sees both halves of each SwiGLU
//    product.
//  * Operands go memory -> LDS with buffer_load ... lds (16 bytes per lane,
//    no register staging) through a ring of STAGES K-slices: slice kt+STAGES-1
//    is in flight while the matrix cores consume slice kt, one barrier per
//    slice. Each lane picks the global chunk that belongs at its LDS slot,
//    which realises an XOR swizzle of the 16-byte chunks within a row so the
//    fragment reads spread over the LDS banks. A lane's offsets stay fixed
//    for the tile and the K-slice advance rides in the scalar offset. A tile
//    of at most 64 rows (forward kinds) stages 64-row A slices in three
//    stages instead.
//  * With two stages, a slice's loads go out one per MFMA of the step that
//    follows the barrier (weights first, then activations) rather than back
//    to back: all eight wavefronts issuing theirs at once overfill the
//    texture unit's command queue, and a wavefront stalled on a load issue
//    stalls its MFMAs too.
//  * The next 16-wide step's fragment reads are interleaved with the current
//    step's MFMAs (scheduling hints), B fragments first.
//  * Ragged groups: each workgroup derives the per-expert m-tile prefix from
//    the device-side counts (no host sync; grid sized for the chip, not for
//    the routing), then walks tile ids persistently. Ids run expert-major,
//    then over bands of 4 m-tiles, then n-tile, then m-tile within the band,
//    and each of the 8 XCDs gets a contiguous range of ids, so the workgroups
//    sharing a weight tile or an activation tile sit behind the same L2. An expert's c rows form ceil(c/BM) tiles of
//    (nearly) equal height, so no tile is a short tail that would finish
//    early and pull its workgroup out of step with the others sharing its
//    data. Each wavefront runs a K loop specialised for the number of its
//    32-row blocks that hold rows.
//  * Each tile's A range ends at its expert's last row: the rows past it
//    read as zeros through the buffer bound (their results are never stored).
//    gate/up can also gather its rows from the token rows themselves (row r
//    of the grouped layout is token src_row[r] / top_k): each lane's A offset
//    is then that token's row, looked up once per tile, and the expert-major
//    copy of the activations is never written.
//    An expert's rows are clamped to [offsets[e], m_cap), so inconsistent
//    device counts cannot move a read or a write past the buffers.
//  * Epilogue through LDS: fp32 -> bf16 (SwiGLU for the gated pair) into a
//    [BM, OUT_N] tile, then 16-byte row-contiguous stores of the valid rows;
//    a tile larger than the stage buffers goes out in two column passes. The
//    down backward stages its fp32 dh per wavefront column and finishes the
//    SwiGLU backward row-contiguously (16-byte loads of g, u and stores).
#include <algorithm>
#include <type_traits>
#include <utility>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kWaves = 8;
constexpr int kBand = 4;  // row tiles walked together (tile order, below)
constexpr int kThreads = kWaves * kWave;

// What a launch computes. The B operand holds, per local expert, N output
// rows of K: for the forward kinds (kPlain, kGated, kGatedSave) in the packed
// layout of moe_pack_weights, for the backward kinds row-major [E_loc, N, ldb].
//   kPlain      c = a b0^T                                  (down; any plain product)
//   kGated      c = silu(a b0^T) * (a b1^T)                 (gate/up, SwiGLU fused)
//   kGatedSave  as kGated, and aux_out = [a b0^T | a b1^T]  (pre-activations kept for
//                                                            the backward), bf16
//   kSwigluBwd  dh = a b0^T, then with (g, u) = aux:        (down backward)
//               c = [dh u silu'(g) | dh silu(g)]
//   kKSplit     c = a [b0 | b1]^T, b0 for k < k_split and b1 past it
//                                                           (gate/up backward)
//   kGatedGather as kGated, a holding the token rows: grouped row r is
//               a[gather[r] / top_k]                        (gate/up with the permute fused)
enum Kind { kPlain = 0, kGated = 1, kGatedSave = 2, kSwigluBwd = 3, kKSplit = 4,
            kGatedGather = 5 };

struct GemmArgs {
  const uint16_t* a;       // [rows, K] bf16
  const uint16_t* b0;      // [E_loc, N, K] bf16 packed, or [E_loc, N, ldb] row-major
  const uint16_t* b1;      // as b0 (kGated*, kKSplit)
  uint16_t* c;             // [rows, N] bf16 ([rows, 2N] for kSwigluBwd)
  const int32_t* offsets;  // [E_loc + 1]
  const int32_t* counts;   // [E_loc]
  int64_t m_cap;           // rows of a, c (and aux, aux_out): no row at or past it is touched
  int e_loc;
  int n, k;
  int ldb;                 // row-major b0/b1: row length (K, or k_split for kKSplit)
  int k_split;             // kKSplit: K index where b1 takes over
  const uint16_t* aux;     // kSwigluBwd: [rows, 2N] bf16, (g | u) of the forward
  uint16_t* aux_out;       // kGatedSave: [rows, 2N] bf16 (out)
  // kGatedGather: a holds token rows [T, K] and grouped row r reads token
  // gather[r] / top_k (gather = the layout's src_row)
  const int32_t* gather;
  int top_k;
  uint32_t a_bytes;        // gather: bytes of a, T * K * 2 (T * K * 2 + K * 2 < 2^32)
};

__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// XOR key of a row: which 16-byte chunk slot a logical chunk moves to. The
// LDS serves a 16-byte-per-lane read 16 lanes (256 bytes, all 64 four-byte
// banks) at a time, and a fragment read has 16 lanes on 16 consecutive rows
// at one logical chunk. Those rows must land on 16 distinct 16-byte bank
// groups: 128-byte rows (BK 64) split them by row parity (32 banks each), so
// the key takes the next three row bits; 64-byte rows (BK 32) split them by
// row % 4, so the key takes the next two.
template <int BK>
__device__ __forceinline__ int swz_key(int row) {
  return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

template <int BK>
__device__ __forceinline__ int swz(int row, int ch) {
  return row * (BK * 2) + ((ch ^ swz_key<BK>(row)) << 4);
}

// Instruction-scheduling hint for one 16-wide K step with NR fragment reads
// (LDS) and NM matrix products: read slot T is preceded by one or two
// products, so the reads for the next step spread over this step's products
// instead of bunching up in front of them.
template <int T, int NR, int NM>
__device__ __forceinline__ void interleave_slot() {
  constexpr int PRE = NM > NR ? NM - NR : 0;  // slots that take two products
  constexpr int M = T < PRE ? 2 : (T - PRE < NM - 2 * PRE ? 1 : 0);
  if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(0x008, M, 0);  // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                        // LDS read
}
template <int NR, int NM, int... T>
__device__ __forceinline__ void interleave_reads(std::integer_sequence<int, T...>) {
  (interleave_slot<T, NR, NM>(), ...);
}


// Calls f(std::integral_constant<int, nb>) for the run-time nb in 0..NB, so
// each block count gets its own fully unrolled copy of f.
template <int NB, class F>
__device__ __forceinline__ void with_block_count(int nb, F&& f) {
  if constexpr (NB == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (nb >= NB) f(std::integral_constant<int, NB>{});
    else with_block_count<NB - 1>(nb, f);
  }
}

template <int BM, int BN, int BK, int STAGES, int KIND, int TM>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs g) {
  constexpr bool GATED = KIND == kGated || KIND == kGatedSave || KIND == kGatedGather;
  // the forward kinds read packed weights, the backward kinds row-major ones
  constexpr bool BLOCKED = GATED || KIND == kPlain;
  constexpr int WROWS = 32 * TM;               // accumulator rows per wavefront
  constexpr int WAVES_M = BM / WROWS, WAVES_N = kWaves / WAVES_M;
  constexpr int OUT_N = GATED ? BN / 2 : BN;  // output columns per tile
  constexpr int WCOL = OUT_N / WAVES_N;       // output columns per wavefront
  constexpr int TN = (GATED ? 2 : 1) * WCOL / 32;
  constexpr int HALF = GATED ? TN / 2 : TN;   // gated: gate tiles j < HALF, up tiles after
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int A_LOADS = A_BYTES / 1024 / kWaves, B_LOADS = B_BYTES / 1024 / kWaves;
  constexpr int CPR = BK / 8;           // 16-byte chunks per staged row
  constexpr int RB = 64 / CPR;          // rows per 1 KiB wave-load
  static_assert(WAVES_M * WROWS == BM && WAVES_M * WAVES_N == kWaves, "wavefront grid");
  static_assert(A_LOADS * 1024 * kWaves == A_BYTES && B_LOADS * 1024 * kWaves == B_BYTES,
                "whole 1 KiB wave-loads");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && WCOL % 32 == 0 && HALF >= 1, "tile shape");
  // the bf16 output tile goes out through the stage buffers in EP column passes
  constexpr int EP = (BM * OUT_N * 2 > STAGE * STAGES) ? 2 : 1;
  static_assert(BM * OUT_N * 2 <= EP * STAGE * STAGES && WAVES_N % EP == 0, "epilogue passes");
  static_assert(!GATED || (B_LOADS % 2 == 0), "gated B loads split evenly");
  // a tile's B rows lie in one packed row block (OUT_N 256 only where N % 256 == 0)
  static_assert(!BLOCKED || (BK == kPackedSlice && (OUT_N == 128 || OUT_N == 256)),
                "packed B tiles");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
  __shared__ int mt_prefix[kMaxExperts + 1];
  __shared__ int wave_tot[kWaves];
  // each local expert's row count and first row, read once: per-tile reads
  // from memory would wait (vmcnt) for the previous tile's output stores
  __shared__ int cnt_s[kMaxExperts], off_s[kMaxExperts];

  // the wavefront index in a scalar register: LDS destinations are scalar arithmetic
  const int tid = threadIdx.x, lane = lane_id(), wid = uniform(tid / kWave);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int K = g.k, N = g.n;
  const int NT = N / OUT_N, KT = K / BK;

  // m-tiles per local expert, exclusive prefix (each thread: PER experts)
  constexpr int PER = kMaxExperts / kThreads;
  {
    int v[PER], run = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid * PER + q;
      int c = 0;
      if (e < g.e_loc) {
        // an expert's rows stay inside [0, m_cap) whatever the device counts say
        const int o = g.offsets[e];
        const int64_t room = o < 0 ? 0 : max(int64_t(0), g.m_cap - o);
        c = int(min(int64_t(max(g.counts[e], 0)), room));
        cnt_s[e] = c, off_s[e] = o;
      }
      v[q] = (c + BM - 1) / BM;
      run += v[q];
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wave_tot[wid] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wid; ++w) before += wave_tot[w];
    int ex = before + incl - run;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid * PER + q;
      if (e < g.e_loc) mt_prefix[e] = ex;
      ex += v[q];
    }
    if (tid == kThreads - 1) mt_prefix[g.e_loc] = ex;
    __syncthreads();
  }
  const int total = uniform(mt_prefix[g.e_loc]) * NT;

  const int G = gridDim.x;
  int slot = blockIdx.x;
  if ((G & 7) == 0) slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // this lane's 16-byte chunk inside each 1 KiB wave-load: row l / CPR of the
  // RB-row block, physical chunk l % CPR, which holds logical chunk
  // (l % CPR) ^ key(row). The wave-loads of one wavefront start 8*RB rows
  // apart, which leaves the key unchanged, so one chunk index serves them all.
  const int ld_r = lane / CPR;
  const int ld_ch = (lane % CPR) ^ swz_key<BK>(wid * RB + ld_r);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

  for (int tile = slot; tile < total; tile += G) {
    int lo = 0, hi = g.e_loc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mt_prefix[mid] * NT <= tile) lo = mid; else hi = mid - 1;
    }
    // tile coordinates are the same in every lane: keep them in scalar registers
    const int e = uniform(lo);
    const int mtiles = uniform(mt_prefix[e + 1] - mt_prefix[e]);
    // Within the expert, row tiles go in bands of kBand, column tile major
    // inside a band: the workgroups of one XCD (32 consecutive ids) then share
    // the A slices of 4 row tiles and the B slices of 8 column tiles, instead
    // of 32 row tiles and one column tile when an expert has many rows (each
    // A tile would be fetched again for every column tile).
    const int rem = tile - uniform(mt_prefix[e]) * NT;
    const int full = mtiles / kBand * kBand;  // row tiles in whole bands
    int nt, mt;
    if (rem < full * NT) {
      const int band = rem / (kBand * NT), r2 = rem % (kBand * NT);
      nt = r2 / kBand;
      mt = band * kBand + r2 % kBand;
    } else {
      const int tail = mtiles - full, r2 = rem - full * NT;
      nt = r2 / tail;
      mt = full + r2 % tail;
    }
    // The expert's rows split into mtiles tiles of (nearly) equal height, a
    // multiple of 32 and at most BM: no short tail tile, so the workgroups that
    // share weight and activation tiles through L2 take about equally long and
    // stay in step. The gated kinds deal the expert's 32-row blocks out evenly
    // (heights differ by at most one block, nothing is computed past the last
    // block); the others give every tile the same height, the last one
    // holding what is left (measured faster for them).
    const int cnt_e = uniform(cnt_s[e]);
    int hgt, start;
    if constexpr (GATED) {
      const int blks = (cnt_e + 31) / 32, bq = blks / mtiles, br = blks % mtiles;
      hgt = (bq + (mt < br ? 1 : 0)) * 32;
      start = 32 * (mt * bq + min(mt, br));
    } else {
      hgt = ((cnt_e + mtiles - 1) / mtiles + 31) / 32 * 32;
      start = mt * hgt;
    }
    const int64_t row0 = int64_t(uniform(off_s[e])) + start;
    const int rows_valid = min(hgt, cnt_e - start);

    // scalar bases + 32-bit per-lane offsets (elements) within the tile
    const uint16_t* a_base = g.a + row0 * K;
    const int ldb = g.ldb;
    // B: the tile's OUT_N output rows of expert e. Blocked (packed) weights
    // hold each K-slice of those rows in one contiguous run; row-major ones
    // hold each row's K values contiguously, ldb apart.
    int64_t b_off;
    uint32_t b_bytes, b_step, b_row;
    if constexpr (BLOCKED) {
      const int R = packed_row_block(N), n0 = nt * OUT_N;
      b_off = int64_t(e) * N * K + int64_t(n0 / R) * K * R + int64_t(n0 % R) * BK;
      b_bytes = uint32_t(int64_t(K) * R - int64_t(n0 % R) * BK) * 2u;
      b_step = uint32_t(R) * BK;  // elements from one K-slice to the next
      b_row = BK;
    } else {
      b_off = (int64_t(e) * N + int64_t(nt) * OUT_N) * ldb;
      b_bytes = uint32_t(OUT_N) * uint32_t(ldb) * 2u;
      b_step = BK;
      b_row = uint32_t(ldb);
    }
    const uint16_t* b_base0 = g.b0 + b_off;
    const uint16_t* b_base1 = (GATED || KIND == kKSplit) ? g.b1 + b_off : b_base0;
    // A's range ends at the expert's last valid row of the tile: the rows
    // past it read as zeros (their results are never stored). With a row
    // gather the range is all of the token rows, and a row past the tile's
    // valid rows takes the offset a_bytes, past the range, so it reads zeros.
    constexpr bool gathered = KIND == kGatedGather;
    const i32x4 ra = gathered ? make_rsrc(g.a, g.a_bytes)
                              : make_rsrc(a_base, uint32_t(rows_valid) * uint32_t(K) * 2u);
    const i32x4 rb0 = make_rsrc(b_base0, b_bytes);
    const i32x4 rb1 = make_rsrc(b_base1, b_bytes);
    // per-lane byte offsets of the first K-slice (fixed for the tile); each
    // slice adds a wave-uniform advance
    uint32_t oa[A_LOADS], ob[B_LOADS];
    if constexpr (gathered) {
      int src[A_LOADS];
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) {  // the row indices first, all in flight
        const int r = (wid + kWaves * i) * RB + ld_r;
        src[i] = r < rows_valid ? g.gather[row0 + r] : -1;
      }
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i)
        oa[i] = src[i] >= 0
                    ? (uint32_t(src[i] / g.top_k) * uint32_t(K) + ld_ch * 8) * 2u
                    : g.a_bytes;
    } else {
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) {
        const int r = (wid + kWaves * i) * RB + ld_r;
        oa[i] = (uint32_t(r) * uint32_t(K) + ld_ch * 8) * 2u;
      }
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int r = (wid + kWaves * i) * RB + ld_r;  // gated: first half gate rows, then up
      ob[i] = (uint32_t(GATED ? r % (BN / 2) : r) * b_row + ld_ch * 8) * 2u;
    }
    // wave-load i of K-slice kt: A rows into the stage's A part at LDS byte
    // a_lds, B rows into its B part at b_lds
    auto load_a = [&](int i, int kt, uint32_t a_lds) {
      dma16(ra, oa[i], uint32_t(kt) * BK * 2, a_lds + (wid + kWaves * i) * 1024);
    };
    auto load_b = [&](int i, int kt, uint32_t b_lds) {
      if constexpr (KIND == kKSplit) {
        // the same slice of b0 or, past k_split, of b1 (slices never straddle it)
        const uint32_t k0 = uint32_t(kt) * BK;
        const bool second = k0 >= uint32_t(g.k_split);
        dma16(second ? rb1 : rb0, ob[i], (second ? k0 - uint32_t(g.k_split) : k0) * 2,
              b_lds + (wid + kWaves * i) * 1024);
      } else {
        dma16((GATED && i >= B_LOADS / 2) ? rb1 : rb0, ob[i], uint32_t(kt) * b_step * 2,
              b_lds + (wid + kWaves * i) * 1024);
      }
    };
    // all of slice kt into stage st. SM: a tile of at most 64 rows, staged
    // with 64-row A slices so that three stages fit where the full tile has two
    auto issue = [&](int kt, int st, auto sm_tag) {
      constexpr bool SM = decltype(sm_tag)::value;
      constexpr int AB = SM ? 64 * BK * 2 : A_BYTES, ST = AB + B_BYTES, AL = AB / 1024 / kWaves;
      const uint32_t sbase = lds0 + st * ST;
#pragma unroll
      for (int i = 0; i < AL; ++i) load_a(i, kt, sbase);
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) load_b(i, kt, sbase + AB);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // 32-row blocks of this wavefront that hold valid rows (0..TM): a partly
    // filled tile skips the matrix work (and A reads) of its empty blocks
    const int nblk = uniform(min(TM, max(0, (rows_valid - wm * WROWS + 31) / 32)));

    constexpr int KK = BK / 16;
    // The K loop for NB (compile-time) valid 32-row blocks, software-pipelined
    // around its one barrier per slice: the fragments of a slice's last
    // 16-wide step are read before the barrier, so those MFMAs run while the
    // first reads of the next slice are in flight. Every variant executes the
    // same loads and barriers; only the matrix work differs.
    auto kloop = [&](auto nb_tag, auto sm_tag) {
      constexpr int NB = decltype(nb_tag)::value;
      constexpr bool SM = decltype(sm_tag)::value;
      constexpr int AB = SM ? 64 * BK * 2 : A_BYTES, ST = AB + B_BYTES;
      constexpr int NS = SM ? 3 : STAGES, AL = AB / 1024 / kWaves;
      constexpr int WT = (NS - 2) * (AL + B_LOADS);
      static_assert(NS * ST <= STAGES * STAGE, "small-tile stages fit");
      bf16x8 fa[2][TM], fb[2][TN];
      auto read_frags = [&](const char* base, int kk, bf16x8 (&a)[TM], bf16x8 (&b)[TN]) {
        const int ch = 2 * kk + (lane >> 5);
        if (NB == 0) return;
        // B first: a step's first products need both B fragments and A[0]
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int brow = GATED ? (j / HALF) * (BN / 2) + wn * WCOL + (j % HALF) * 32
                                 : wn * WCOL + j * 32;
          b[j] = *reinterpret_cast<const bf16x8*>(base + AB +
                                                  swz<BK>(brow + (lane & 31), ch));
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(
              base + swz<BK>(wm * WROWS + i * 32 + (lane & 31), ch));
      };
      auto mfma = [&](const bf16x8 (&a)[TM], const bf16x8 (&b)[TN]) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      };
      auto steps = [&](const char* base) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
          read_frags(base, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
          mfma(fa[kk & 1], fb[kk & 1]);
          // interleave the next step's fragment reads with this step's products
          if constexpr (NB > 0) interleave_reads<NB + TN, NB * TN>(std::make_integer_sequence<int, NB + TN>{});
        }
      };
      // A step's products with the loads of slice kt2 between them: product q,
      // then load q, the loads left over after the last product. B loads come
      // first (the weights stream from memory, so they get the longest lead),
      // then A. A load issues only once the matrix pipe has taken the product
      // before it, so each wavefront's loads go out spread over its products;
      // issued back to back after the barrier, every wavefront's loads at once
      // fill the texture unit's command queue and stall the issuing
      // wavefronts, products included. ld false: the products alone.
      constexpr int NL = AL + B_LOADS, NP = NB * TN, NQ = NP > NL ? NP : NL;
      auto mfma_loads = [&](const bf16x8 (&a)[TM], const bf16x8 (&b)[TN], int kt2, bool ld) {
        const uint32_t sbase = lds0 + (kt2 % NS) * ST;
        for_each_index([&](auto q_tag) {
          constexpr int q = decltype(q_tag)::value;
          if constexpr (q < NP)
            acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a[q / TN], b[q % TN], acc[q / TN][q % TN], 0, 0, 0);
          if constexpr (q < B_LOADS) {
            if (ld) load_b(q, kt2, sbase + AB);
          } else if constexpr (q < NL) {
            if (ld) load_a(q - B_LOADS, kt2, sbase);
          }
        }, std::make_integer_sequence<int, NQ>{});
      };

#pragma unroll
      for (int s = 0; s < NS - 1; ++s)
        if (s < KT) issue(s, s, sm_tag);
      if (NS - 2 < KT) wait_vmcnt<WT>(); else wait_vmcnt<0>();
      __syncthreads();  // slice 0 visible
      if (NS - 1 < KT) issue(NS - 1, NS - 1, sm_tag);
      read_frags(smem, 0, fa[0], fb[0]);
      if constexpr (!SM && NS == 2) {
        // Two stages: the barrier after slice kt's steps releases slice kt's
        // stage, and slice kt+2's loads into it ride with slice kt's last-step
        // products. The last slice is peeled so that the loop has one path.
        for (int kt = 0; kt + 1 < KT; ++kt) {
          steps(smem + (kt % NS) * ST);
          // slice kt+1 landed (this wavefront's part), and all of slice kt is read
          wait_vmcnt<0>();
          __syncthreads();
          read_frags(smem + ((kt + 1) % NS) * ST, 0, fa[0], fb[0]);
          mfma_loads(fa[(KK - 1) & 1], fb[(KK - 1) & 1], kt + NS, kt + NS < KT);
        }
        steps(smem + ((KT - 1) % NS) * ST);
        mfma(fa[(KK - 1) & 1], fb[(KK - 1) & 1]);
        return;
      }
      for (int kt = 0; kt < KT; ++kt) {
        steps(smem + (kt % NS) * ST);
        if (kt + 1 < KT) {
          // slice kt+1 landed (this wavefront's part), and all of slice kt is read
          if (kt + NS - 1 < KT) wait_vmcnt<WT>(); else wait_vmcnt<0>();
          __syncthreads();
          if (kt + NS < KT) issue(kt + NS, (kt + NS) % NS, sm_tag);
          read_frags(smem + ((kt + 1) % NS) * ST, 0, fa[0], fb[0]);
        }
        mfma(fa[(KK - 1) & 1], fb[(KK - 1) & 1]);
      }
    };
    // one K-loop copy per block count 0..TM: a wavefront multiplies only the
    // blocks that hold rows. A forward tile of at most 64 rows (the few rows
    // of a lightly routed expert) is bound by load latency, not by its matrix
    // work: it gets the three-stage layout
    constexpr bool SMALL_OK = (KIND == kGated || KIND == kGatedGather || KIND == kPlain) && TM >= 2;
    if (SMALL_OK && rows_valid <= 64)
      with_block_count<(TM >= 2 ? 2 : TM)>(nblk, [&](auto nb) { kloop(nb, std::bool_constant<SMALL_OK>{}); });
    else
      with_block_count<TM>(nblk, [&](auto nb) { kloop(nb, std::false_type{}); });
    __syncthreads();  // every wavefront is done reading the last slice

    // accumulators (lane: column lane % 32, rows 8*(q/4) + 4*(lane/32) + q%4)
    // -> bf16 tile in LDS -> 16-byte stores of the valid rows. Each of the
    // NOUT outputs goes out on its own; a tile larger than the stage buffers
    // goes out in EP passes, each over the columns of WAVES_N / EP wavefront
    // columns.
    uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
    if constexpr (KIND == kSwigluBwd) {
      // one pass per wavefront column (PN = WCOL columns): that column's dh
      // (fp32) goes to LDS in the accumulator layout, then every thread takes
      // 8 consecutive columns of a row: the forward's g and u come in with
      // 16-byte loads, dg and du go out with 16-byte stores
      constexpr int PN = WCOL, OCH = PN / 8;
      constexpr int PS = PN + 8;  // fp32 row stride: rows 4 apart land 32 banks apart
      static_assert(BM * PS * 4 <= STAGE * STAGES, "dh tile fits the stages");
      float* dt = reinterpret_cast<float*>(smem);
      for (int pass = 0; pass < WAVES_N; ++pass) {
        if (wn == pass) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int q = 0; q < 16; ++q) {
                const int r = wm * WROWS + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                dt[r * PS + j * 32 + (lane & 31)] = acc[i][j][q];
              }
        }
        __syncthreads();
        const int64_t cb = int64_t(nt) * OUT_N + pass * PN;  // first column of the pass
        for (int c = tid; c < rows_valid * OCH; c += kThreads) {
          const int r = c / OCH, ch = c % OCH;
          const int64_t off = (row0 + r) * 2 * int64_t(N) + cb + ch * 8;
          float gg[8], uu[8];
          unpack8(*reinterpret_cast<const u32x4*>(g.aux + off), gg);
          unpack8(*reinterpret_cast<const u32x4*>(g.aux + off + N), uu);
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(dt + r * PS + ch * 8);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(dt + r * PS + ch * 8 + 4);
          const float dh[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          float dg[8], du[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gg[e]));
            dg[e] = dh[e] * uu[e] * (sg * (1.0f + gg[e] * (1.0f - sg)));
            du[e] = dh[e] * (gg[e] * sg);
          }
          *reinterpret_cast<u32x4*>(g.c + off) = pack8(dg);
          *reinterpret_cast<u32x4*>(g.c + off + N) = pack8(du);
        }
        __syncthreads();  // dt read out before the next pass writes it
      }
    } else {
      constexpr int NOUT = KIND == kGatedSave ? 3 : 1;
      constexpr int PN = OUT_N / EP;  // output columns per pass
      constexpr int OCH = PN / 8;     // 16-byte chunks per output row of a pass
      // output O (compile time): h (or the plain product), then g and u
      auto emit = [&](auto o_tag) __attribute__((always_inline)) {
        constexpr int O = decltype(o_tag)::value;
        uint16_t* dst = O == 0 ? g.c : g.aux_out;
        const int64_t ld = O == 0 ? int64_t(N) : 2 * int64_t(N);
        const int64_t col0 = int64_t(nt) * OUT_N + (O == 2 ? int64_t(N) : 0);
        for (int pass = 0; pass < EP; ++pass) {
          if (wn / (WAVES_N / EP) == pass) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < HALF; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                  const int r = wm * WROWS + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                  const int col = wn * WCOL + j * 32 + (lane & 31);
                  float v = acc[i][j][q];
                  if constexpr (GATED) {
                    if constexpr (O == 0) v = silu(v) * acc[i][j + HALF][q];
                    else if constexpr (O == 2) v = acc[i][j + HALF][q];
                  }
                  ct[r * PN + col - pass * PN] = to_bf16(v);
                }
          }
          __syncthreads();
          uint16_t* C = dst + row0 * ld + col0 + pass * PN;
          for (int c = tid; c < rows_valid * OCH; c += kThreads) {
            const int r = c / OCH, ch = c % OCH;
            *reinterpret_cast<u32x4*>(C + int64_t(r) * ld + ch * 8) =
                *reinterpret_cast<const u32x4*>(ct + r * PN + ch * 8);
          }
          if (pass + 1 < EP || O + 1 < NOUT) __syncthreads();  // read out before the next write
        }
      };
      emit(std::integral_constant<int, 0>{});
      if constexpr (NOUT > 1) {
        emit(std::integral_constant<int, 1>{});
        emit(std::integral_constant<int, 2>{});
      }
    }
    __syncthreads();  // the tile buffer is read out before the next tile's loads
  }
}

template <int BM, int BN, int BK, int STAGES, int KIND, int TM>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  grouped_gemm_kernel<BM, BN, BK, STAGES, KIND, TM><<<device_cu_count(), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const void* x_perm, const int32_t* offsets, const int32_t* counts,
                          int e_loc, int64_t m_cap, int H, int I, const void* w1t,
                          const void* w3t, void* h, hipStream_t s) {
  GemmArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(x_perm);
  a.b0 = static_cast<const uint16_t*>(w1t);
  a.b1 = static_cast<const uint16_t*>(w3t);
  a.c = static_cast<uint16_t*>(h);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc, a.n = I, a.k = H, a.ldb = H;
  return launch<320, 256, 64, 2, kGated, 5>(a, s);  // I % 128 == 0: 128 output columns per tile
}

// gate/up reading its rows straight from the token rows: grouped row r is
// x[src_row[r] / top_k] (the permute fused into the A-operand loads)
hipError_t launch_gate_up_gather(const void* x, int64_t T, int top_k, const int32_t* src_row,
                                 const int32_t* offsets, const int32_t* counts, int e_loc,
                                 int64_t m_cap, int H, int I, const void* w1t, const void* w3t,
                                 void* h, hipStream_t s) {
  GemmArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(x);
  a.gather = src_row;
  a.top_k = top_k;
  a.a_bytes = static_cast<uint32_t>(T * H * 2);
  a.b0 = static_cast<const uint16_t*>(w1t);
  a.b1 = static_cast<const uint16_t*>(w3t);
  a.c = static_cast<uint16_t*>(h);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc, a.n = I, a.k = H, a.ldb = H;
  return launch<320, 256, 64, 2, kGatedGather, 5>(a, s);
}

hipError_t launch_gate_up_save(const void* x_perm, const int32_t* offsets, const int32_t* counts,
                               int e_loc, int64_t m_cap, int H, int I, const void* w1t,
                               const void* w3t, void* h, void* gu, hipStream_t s) {
  GemmArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(x_perm);
  a.b0 = static_cast<const uint16_t*>(w1t);
  a.b1 = static_cast<const uint16_t*>(w3t);
  a.c = static_cast<uint16_t*>(h);
  a.aux_out = static_cast<uint16_t*>(gu);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc, a.n = I, a.k = H, a.ldb = H;
  return launch<320, 256, 64, 2, kGatedSave, 5>(a, s);
}

hipError_t launch_down(const void* h, const int32_t* offsets, const int32_t* counts, int e_loc,
                       int64_t m_cap, int I, int H, const void* w2t, void* y, hipStream_t s) {
  GemmArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(h);
  a.b0 = static_cast<const uint16_t*>(w2t);
  a.c = static_cast<uint16_t*>(y);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc, a.n = H, a.k = I, a.ldb = I;
  if (H % 256 == 0) return launch<320, 256, 64, 2, kPlain, 5>(a, s);
  return launch<256, 128, 64, 2, kPlain, 2>(a, s);
}

// dh = dy W2^T reads W2 in its math orientation [E_loc, I, H]: for this
// product that is already output-major (N = I rows of K = H).
hipError_t launch_down_backward(const void* dy, const void* gu, const int32_t* offsets,
                                const int32_t* counts, int e_loc, int64_t m_cap, int I, int H,
                                const void* w2, void* dgu, hipStream_t s) {
  GemmArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(dy);
  a.b0 = static_cast<const uint16_t*>(w2);
  a.c = static_cast<uint16_t*>(dgu);
  a.aux = static_cast<const uint16_t*>(gu);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc, a.n = I, a.k = H, a.ldb = H;
  if (I % 256 == 0) return launch<320, 256, 64, 2, kSwigluBwd, 5>(a, s);
  return launch<256, 128, 64, 2, kSwigluBwd, 2>(a, s);
}

// dx = [dg | du] [W1 | W3]^T: W1 and W3 in math orientation [E_loc, H, I] are
// output-major for this product (N = H rows of I), one for each half of K = 2I.
hipError_t launch_gate_up_backward(const void* dgu, const int32_t* offsets, const int32_t* counts,
                                   int e_loc, int64_t m_cap, int H, int I, const void* w1,
                                   const void* w3, void* dx, hipStream_t s) {
  GemmArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(dgu);
  a.b0 = static_cast<const uint16_t*>(w1);
  a.b1 = static_cast<const uint16_t*>(w3);
  a.c = static_cast<uint16_t*>(dx);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc, a.n = H, a.k = 2 * I, a.ldb = I;
  a.k_split = I;
  if (H % 256 == 0) return launch<320, 256, 64, 2, kKSplit, 5>(a, s);
  return launch<256, 128, 64, 2, kKSplit, 2>(a, s);
}

}  // namespace moe
