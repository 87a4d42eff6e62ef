// Weight gradients of the grouped SwiGLU experts on the matrix cores.
//
// Training hands the expert weight gradients back in BF16 after the grouped
// GEMM backward (xtuner PR #2056 "Integrate MoonEP dispatcher ...", section
// "Summary"; commit "extend grouped GEMM for dynamic expert gradients"). Per
// local expert e with rows [offsets[e], offsets[e] + counts[e]):
//
//   C[m, n] = sum over the expert's rows r of A[r, m] * B[r, n]
//     dW1 | dW3 = x_perm^T [dg | du]     (M = H, N = 2I, split at column I)
//     dW2       = h^T dy                 (M = I, N = H)
//
// fp32 accumulation, one bf16 rounding. The reduction runs over the rows,
// which are the slow dimension of both operands, so the MFMA fragments (8
// consecutive k per lane) are transposed on the way out of LDS:
//  * tiles land in LDS as they sit in memory, row k of the slice holding BM
//    (or BN) contiguous values, through buffer_load ... lds (16 bytes a lane);
//  * gfx950's ds_read_b64_tr_b16 gives each lane of a 16-lane group four
//    values down a column: the group's lanes point at 4 rows x 4 column
//    quads, and lane i receives column i of the 4 rows. Two such reads make
//    the 8 consecutive k of one A (or B) fragment row;
//  * within a row the 16-byte chunks are XOR-swizzled by 4 * (k % 4): the 32
//    lanes of two groups then cover all 64 LDS banks.
// Rows past the expert's count read as zeros through the buffer range of each
// K slice (padding rows between experts hold stale data). An expert with no
// rows gets a zero gradient. Workgroups are persistent; each XCD takes a
// contiguous range of tile ids (expert-major, then bands of 4 row tiles,
// column tile major inside a band), so the tiles of one expert, which share
// both operands, sit behind the same L2. A slice's loads go out one per
// product of the step after the barrier, not back to back; the next tile's
// first slice is put in flight before a tile's epilogue.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int BK = 64;  // rows of the reduction per slice
constexpr int kMaxExperts = 1024;  // local experts the entry points accept

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

struct WgradArgs {
  const uint16_t* a;       // [rows, M] bf16
  const uint16_t* b;       // [rows, N] bf16
  uint16_t* out0;          // [E_loc, M, n_split] bf16
  uint16_t* out1;          // [E_loc, M, N - n_split] bf16 (unused when n_split == N)
  const int32_t* offsets;  // [E_loc + 1]
  const int32_t* counts;   // [E_loc]
  int64_t m_cap;           // rows of a and b: no row at or past it is read
  int e_loc, m, n, n_split;
  // tile queue of this launch: [0] the next dynamic tile, [1] the workgroups
  // done; zero on entry, zero again when the last workgroup leaves. nullptr:
  // each workgroup walks its tiles statically (tile += gridDim.x).
  uint32_t* queue;
};

// physical 16-byte chunk of logical chunk c in slice row k (an involution)
__device__ __forceinline__ int wg_swz(int c, int k) { return c ^ ((k & 3) << 2); }

__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(WgradArgs g) {
  constexpr int TM = 2;  // 32-row blocks of m per wavefront
  constexpr int WAVES_M = BM / (32 * TM), WAVES_N = kWaves / WAVES_M;
  constexpr int WCOL = BN / WAVES_N, TN = WCOL / 32;
  constexpr int A_BYTES = BK * BM * 2, B_BYTES = BK * BN * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int A_CPR = BM / 8, B_CPR = BN / 8;          // 16-byte chunks per slice row
  constexpr int A_RPL = 64 / A_CPR, B_RPL = 64 / B_CPR;  // slice rows per 1 KiB wave-load
  constexpr int A_LOADS = A_BYTES / 1024 / kWaves, B_LOADS = B_BYTES / 1024 / kWaves;
  static_assert(WAVES_M * WAVES_N == kWaves && TN >= 1 && WCOL % 32 == 0, "wavefront grid");
  static_assert(A_LOADS * 1024 * kWaves == A_BYTES && B_LOADS * 1024 * kWaves == B_BYTES,
                "whole wave-loads");
  // epilogue passes: JP accumulator blocks per wavefront per pass, the most
  // (dividing TN) whose [BM, WAVES_N * JP * 32] bf16 tile fits stage 0
  constexpr int JP = (TN % 2 == 0 && BM * WAVES_N * (TN / 2) * 64 <= STAGE) ? TN / 2 : 1;
  constexpr int NPASS = TN / JP, LW = WAVES_N * JP * 32, LCH = LW / 8;
  constexpr int ST_IT = BM * LCH / kThreads;  // 16-byte chunks per thread per pass
  static_assert(BM * LW * 2 <= STAGE && ST_IT * kThreads == BM * LCH && (LCH & (LCH - 1)) == 0,
                "epilogue tile");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  // each local expert's row count and first row, read once: per-tile reads
  // from memory would wait (vmcnt) for the previous tile's output stores
  __shared__ int cnt_s[kMaxExperts], off_s[kMaxExperts];
  // local experts by descending row count (ties by index): a tile's work
  // grows with its expert's rows while every expert has the same number of
  // tiles, so the tiles of the largest experts go first and the short ones
  // fill in behind them (longest first), instead of a few long tiles ending
  // the launch alone
  __shared__ uint16_t order_s[kMaxExperts];
  __shared__ int next_s;  // the tile after this one (dynamic walk)
  __shared__ long long wave_max[kWaves], wave_sum[kWaves];

  const int tid = threadIdx.x, lane = lane_id(), wid = uniform(tid / kWave);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int M = g.m, N = g.n;
  const int MT = M / BM, NTL = N / BN, per_expert = MT * NTL;
  // Output tiles of an expert in bands of kBand row tiles, column tile major
  // inside a band: one XCD's 32 consecutive tiles then share the slices of 4
  // row tiles and 8 column tiles instead of 1-2 row tiles and 16-28 column
  // tiles. rem: tile index within the expert -> (row tile, column tile).
  constexpr int kBand = 4;
  const int full = MT / kBand * kBand;
  auto coords = [&](int rem, int& mt, int& nt) {
    if (rem < full * NTL) {
      const int r2 = rem % (kBand * NTL);
      nt = r2 / kBand;
      mt = rem / (kBand * NTL) * kBand + r2 % kBand;
    } else {
      const int tail = MT - full, r2 = rem - full * NTL;
      nt = r2 / tail;
      mt = full + r2 % tail;
    }
  };
  // an expert's rows stay inside [0, m_cap) whatever the device counts say
  for (int e = threadIdx.x; e < g.e_loc; e += kThreads) {
    const int o = g.offsets[e];
    const int64_t room = o < 0 ? 0 : max(int64_t(0), g.m_cap - o);
    cnt_s[e] = int(min(int64_t(max(g.counts[e], 0)), room));
    off_s[e] = o;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < g.e_loc; e += kThreads) {
    const int c = cnt_s[e];
    int pos = 0;
    for (int e2 = 0; e2 < g.e_loc; ++e2) {
      const int c2 = cnt_s[e2];
      pos += (c2 > c || (c2 == c && e2 < e)) ? 1 : 0;
    }
    order_s[pos] = static_cast<uint16_t>(e);
  }
  __syncthreads();
  const int total = g.e_loc * per_expert;
  const int G = gridDim.x;
  // Static walk or the queue. The queue evens out skewed experts but gives an
  // expert's tiles to whichever workgroups free up, on any XCD, which costs
  // L2 sharing (a few per cent under even routing), so it is taken only when
  // the static walk's busiest workgroup would have at least 1/16 more work
  // than the average: a tile counts its K slices plus two (its fixed cost).
  // Every workgroup reaches the same decision from the same counts.
  bool dyn = false;
  if (g.queue) {
    long long load = 0;  // the static walk's work of workgroup slot tid
    if (tid < G)
      for (int t = tid; t < total; t += G)
        load += 2 + (cnt_s[order_s[t / per_expert]] + BK - 1) / BK;
    long long mx = load, sum = load;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      mx = max(mx, __shfl_xor(mx, off, kWave));
      sum += __shfl_xor(sum, off, kWave);
    }
    if (lane == 0) wave_max[wid] = mx, wave_sum[wid] = sum;
    __syncthreads();
    mx = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = max(mx, wave_max[w]), sum += wave_sum[w];
    dyn = mx * 16 * G > sum * 17;
  }
  uint32_t* const queue = dyn ? g.queue : nullptr;
  int slot = blockIdx.x;
  if ((G & 7) == 0) slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

  // fragment-read coordinates of this lane: group of 16, row quad r, column quad q
  const int grp = lane >> 4, fr = (lane >> 2) & 3, fq = lane & 3;

  // A tile whose first K slice the previous tile put in flight (into stage 1,
  // before its epilogue, which stages through stage 0 only): its slices then
  // live in stage (kt + 1) & 1.
  bool pf = false;
  // Tiles go out longest first (the experts in order_s). With the queue, after
  // its first one a workgroup takes the next unclaimed tile whenever it
  // finishes one: the largest experts' tiles then spread over the workgroups
  // that free up first, instead of ending on the few workgroups a static
  // stride gives them to (under Zipf-skewed routing the static walk left the
  // busiest workgroups 1.2-1.6x the mean work).
  for (int tile = slot; tile < total;) {
    // claim the next tile now: the atomic's latency hides under the K loop,
    // whose barriers publish next_s before anyone reads it
    if (queue && tid == 0)
      next_s = G + int(__hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const int pos = tile / per_expert;
    const int e = uniform(int(order_s[pos]));
    int mt, nt;
    coords(tile - pos * per_expert, mt, nt);
    const int cnt = uniform(cnt_s[e]);
    const int64_t base = int64_t(uniform(off_s[e]));
    const int KT = (cnt + BK - 1) / BK;
    const int m0 = mt * BM, n0 = nt * BN;

    // per-lane source offsets (bytes) of each wave-load inside a slice
    uint32_t oa[A_LOADS], ob[B_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int kr = (wid + kWaves * i) * A_RPL + lane / A_CPR;
      const int lc = wg_swz(lane % A_CPR, kr);
      oa[i] = (uint32_t(kr) * uint32_t(M) + uint32_t(m0 + 8 * lc)) * 2u;
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int kr = (wid + kWaves * i) * B_RPL + lane / B_CPR;
      const int lc = wg_swz(lane % B_CPR, kr);
      ob[i] = (uint32_t(kr) * uint32_t(N) + uint32_t(n0 + 8 * lc)) * 2u;
    }
    // the buffer ranges of slice kt end at the expert's last row (none past it)
    auto slice_rsrc = [&](int kt, i32x4& ra, i32x4& rb) {
      const int rows = max(0, min(BK, cnt - kt * BK));
      ra = make_rsrc(g.a + (base + int64_t(kt) * BK) * M, uint32_t(rows) * uint32_t(M) * 2u);
      rb = make_rsrc(g.b + (base + int64_t(kt) * BK) * N, uint32_t(rows) * uint32_t(N) * 2u);
    };
    // wave-load q of a slice (A loads first, then B) into the stage at sbase
    auto load = [&](int q, const i32x4& ra, const i32x4& rb, uint32_t sbase) {
      if (q < A_LOADS) dma16(ra, oa[q], sbase + (wid + kWaves * q) * 1024);
      else dma16(rb, ob[q - A_LOADS], sbase + A_BYTES + (wid + kWaves * (q - A_LOADS)) * 1024);
    };
    auto issue = [&](int kt, int st) {
      i32x4 ra, rb;
      slice_rsrc(kt, ra, rb);
#pragma unroll
      for (int q = 0; q < A_LOADS + B_LOADS; ++q) load(q, ra, rb, lds0 + st * STAGE);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // fragments of the 16-wide step kk of a slice: row k = 16 kk + 8 (grp / 2) + fr
    // (+4 for the second read), column 16 (grp % 2) + 4 fq within the 32-block
    auto read_frags = [&](const char* sb, int kk, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
      const int k = kk * 16 + 8 * (grp >> 1) + fr;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int c = (wm * 64 + i * 32 + 16 * (grp & 1) + 4 * fq);
        const int off = 16 * wg_swz(c >> 3, k) + 8 * (fq & 1);
        fa[i] = tr_pair(sb + k * (BM * 2) + off, sb + (k + 4) * (BM * 2) + off);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = (wn * WCOL + j * 32 + 16 * (grp & 1) + 4 * fq);
        const int off = 16 * wg_swz(c >> 3, k) + 8 * (fq & 1);
        fb[j] = tr_pair(sb + A_BYTES + k * (BN * 2) + off, sb + A_BYTES + (k + 4) * (BN * 2) + off);
      }
    };
    // the products with B as the first operand: each 32x32 block of acc
    // holds the transposed output block, so a lane's four consecutive
    // accumulators are four consecutive output columns of one row (one
    // packed 8-byte LDS write in the epilogue)
    auto mfma = [&](const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN]) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    };
    // A step's products with slice kt2's loads between them (product q, then
    // load q): issued back to back after the barrier, every wavefront's loads
    // at once overfill the texture unit's command queue and stall the
    // wavefronts, their products with them. ld false: the products alone.
    constexpr int NL = A_LOADS + B_LOADS, NP = TM * TN, NQ = NP > NL ? NP : NL;
    auto mfma_loads = [&](const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN], int kt2, int st2,
                          bool ld) {
      i32x4 ra, rb;
      slice_rsrc(kt2, ra, rb);
      const uint32_t sbase = lds0 + st2 * STAGE;
      for_each_index([&](auto q_tag) {
        constexpr int q = decltype(q_tag)::value;
        if constexpr (q < NP)
          acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              fb[q % TN], fa[q / TN], acc[q / TN][q % TN], 0, 0, 0);
        if constexpr (q < NL) {
          if (ld) load(q, ra, rb, sbase);
        }
      }, std::make_integer_sequence<int, NQ>{});
    };

    const int sp = pf ? 1 : 0;  // stage of slice 0
    if (KT > 0) {
      bf16x8 fa[2][TM], fb[2][TN];
      if (!pf) issue(0, 0);
      wait_vmcnt<0>();
      __syncthreads();  // slice 0 visible
      if (KT > 1) issue(1, (1 + sp) & 1);
      read_frags(smem + sp * STAGE, 0, fa[0], fb[0]);
      auto steps = [&](const char* sb) {
#pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
          read_frags(sb, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
          mfma(fa[kk & 1], fb[kk & 1]);
        }
      };
      // every slice but the last: its first three steps, the barrier, then its
      // last step's products paced with slice kt+2's loads into the stage the
      // barrier released; the last slice peeled so that the loop has one path
      for (int kt = 0; kt + 1 < KT; ++kt) {
        steps(smem + ((kt + sp) & 1) * STAGE);
        wait_vmcnt<0>();  // slice kt+1 landed (this wavefront's part)
        __syncthreads();  // ... everyone's, and slice kt is read
        read_frags(smem + ((kt + 1 + sp) & 1) * STAGE, 0, fa[0], fb[0]);
        mfma_loads(fa[1], fb[1], kt + 2, (kt + sp) & 1, kt + 2 < KT);
      }
      steps(smem + ((KT - 1 + sp) & 1) * STAGE);
      mfma(fa[1], fb[1]);
    }
    __syncthreads();  // the stages are free for the epilogue

    // the next tile's first slice goes into stage 1 now, so its latency hides
    // under this tile's epilogue
    pf = false;
    const int t2 = queue ? uniform(next_s) : tile + G;
    {
      if (t2 < total) {
        const int pos2 = t2 / per_expert;
        const int e2 = uniform(int(order_s[pos2]));
        int mt2, nt2;
        coords(t2 - pos2 * per_expert, mt2, nt2);
        const int cnt2 = uniform(cnt_s[e2]);
        if (cnt2 > 0) {
          const int64_t base2 = int64_t(uniform(off_s[e2]));
          const int rows = min(BK, cnt2);
          const i32x4 ra2 = make_rsrc(g.a + base2 * M, uint32_t(rows) * uint32_t(M) * 2u);
          const i32x4 rb2 = make_rsrc(g.b + base2 * N, uint32_t(rows) * uint32_t(N) * 2u);
          const uint32_t sbase = lds0 + STAGE;
#pragma unroll
          for (int i = 0; i < A_LOADS; ++i) {
            const int kr = (wid + kWaves * i) * A_RPL + lane / A_CPR;
            const int lc = wg_swz(lane % A_CPR, kr);
            dma16(ra2, (uint32_t(kr) * uint32_t(M) + uint32_t(mt2 * BM + 8 * lc)) * 2u,
                  sbase + (wid + kWaves * i) * 1024);
          }
#pragma unroll
          for (int i = 0; i < B_LOADS; ++i) {
            const int kr = (wid + kWaves * i) * B_RPL + lane / B_CPR;
            const int lc = wg_swz(lane % B_CPR, kr);
            dma16(rb2, (uint32_t(kr) * uint32_t(N) + uint32_t(nt2 * BN + 8 * lc)) * 2u,
                  sbase + A_BYTES + (wid + kWaves * i) * 1024);
          }
          pf = true;
        }
      }
    }

    // Epilogue through a bf16 tile in stage 0, in NPASS passes. In pass p
    // every wavefront writes its accumulator blocks j = p*JP .. p*JP + JP - 1
    // (all eight write at once), then all threads store the tile's rows with
    // 16-byte stores. Block (i, j) holds output row wm*64 + 32i + lane % 32
    // and, in q, column 32j + 8(q / 4) + 4(lane / 32) + q % 4 of the
    // wavefront's columns: four accumulators make one packed 8-byte LDS
    // write. LDS tile column (wn*JP + jj)*32 + c holds wavefront column wn's
    // block p*JP + jj; the 16-byte chunks of LDS row r sit XOR-swizzled by
    // r % LCH, so the 32 rows one write touches spread over the banks.
    uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
        for (int jj = 0; jj < JP; ++jj)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x16& a = acc[i][pass * JP + jj];
            const int ch = (wn * JP + jj) * 4 + qq;
            *reinterpret_cast<uint2*>(ct + r * LW + (ch ^ (r & (LCH - 1))) * 8 + 4 * (lane >> 5)) =
                make_uint2(pack_bf16x2(a[4 * qq], a[4 * qq + 1]),
                           pack_bf16x2(a[4 * qq + 2], a[4 * qq + 3]));
          }
      }
      __syncthreads();
      // all of the pass's LDS reads first, then the stores
      u32x4 v[ST_IT];
#pragma unroll
      for (int it = 0; it < ST_IT; ++it) {
        const int c = tid + it * kThreads, r = c / LCH, ch = c % LCH;
        v[it] = *reinterpret_cast<const u32x4*>(ct + r * LW + (ch ^ (r & (LCH - 1))) * 8);
      }
#pragma unroll
      for (int it = 0; it < ST_IT; ++it) {
        const int c = tid + it * kThreads, r = c / LCH, ch = c % LCH;
        // the chunk's output column; a 32-column block never straddles n_split
        // (a multiple of 128)
        const int col = n0 + (ch / (4 * JP)) * WCOL + (pass * JP + (ch / 4) % JP) * 32 + (ch % 4) * 8;
        const bool second = col >= g.n_split;
        const int ld = second ? N - g.n_split : g.n_split;
        uint16_t* dst = (second ? g.out1 : g.out0) + (int64_t(e) * M + m0 + r) * ld +
                        (second ? col - g.n_split : col);
        *reinterpret_cast<u32x4*>(dst) = v[it];
      }
      __syncthreads();  // the pass is read out before the next one (or the next tile's loads)
    }
    tile = t2;
  }
  // Every workgroup, its last claim made (or none, when its first tile was
  // already past the end), counts itself out; the last one sets the queue
  // back to zero for the next launch on the stream. No claim can follow: each
  // workgroup's claims returned before it counted itself out.
  if (queue && tid == 0) {
    if (__hip_atomic_fetch_add(queue + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        uint32_t(G) - 1) {
      __hip_atomic_store(queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(queue + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Tile queues: per GPU, kQueueSlots pairs of counters in a static device
// array (zero when the library loads; each launch leaves its pair at zero).
// A pair belongs to the first stream that uses it, so launches that may run
// at the same time (different streams) never share one; launches on one
// stream run one after another. Past kQueueSlots streams a launch walks its
// tiles statically. In host code `tile_queues` is a host-side stand-in: the
// device address of each GPU's copy comes from hipGetSymbolAddress.
constexpr int kQueueSlots = 64;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint32_t tile_queues[2 * kQueueSlots];
std::mutex queue_mu;
uint32_t* queue_base[kMaxDevices];
hipStream_t queue_owner[kMaxDevices][kQueueSlots];
int queue_count[kMaxDevices];

uint32_t* queue_for(hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(queue_mu);
  if (!queue_base[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(tile_queues)) != hipSuccess || !p) {
      (void)hipGetLastError();  // the static walk needs no queue
      return nullptr;
    }
    queue_base[dev] = static_cast<uint32_t*>(p);
  }
  for (int i = 0; i < queue_count[dev]; ++i)
    if (queue_owner[dev][i] == s) return queue_base[dev] + 2 * i;
  if (queue_count[dev] == kQueueSlots) return nullptr;
  queue_owner[dev][queue_count[dev]] = s;
  return queue_base[dev] + 2 * queue_count[dev]++;
}

template <int BM, int BN>
hipError_t launch(const WgradArgs& a, hipStream_t s) {
  wgrad_kernel<BM, BN><<<device_cu_count(), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_any(WgradArgs a, hipStream_t s) {
  a.queue = queue_for(s);
  if (a.m % 256 == 0 && a.n % 256 == 0) return launch<256, 256>(a, s);
  if (a.m % 256 == 0) return launch<256, 128>(a, s);
  if (a.n % 256 == 0) return launch<128, 256>(a, s);
  return launch<128, 128>(a, s);
}

}  // namespace

hipError_t launch_gate_up_wgrad(const void* x_perm, const void* dgu, const int32_t* offsets,
                                const int32_t* counts, int e_loc, int64_t m_cap, int H, int I,
                                void* dw1, void* dw3, hipStream_t s) {
  WgradArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(x_perm);
  a.b = static_cast<const uint16_t*>(dgu);
  a.out0 = static_cast<uint16_t*>(dw1);
  a.out1 = static_cast<uint16_t*>(dw3);
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc;
  a.m = H, a.n = 2 * I, a.n_split = I;
  return launch_any(a, s);
}

hipError_t launch_down_wgrad(const void* h, const void* dy, const int32_t* offsets,
                             const int32_t* counts, int e_loc, int64_t m_cap, int I, int H,
                             void* dw2, hipStream_t s) {
  WgradArgs a{};
  a.m_cap = m_cap;
  a.a = static_cast<const uint16_t*>(h);
  a.b = static_cast<const uint16_t*>(dy);
  a.out0 = static_cast<uint16_t*>(dw2);
  a.out1 = nullptr;
  a.offsets = offsets, a.counts = counts, a.e_loc = e_loc;
  a.m = I, a.n = H, a.n_split = H;
  return launch_any(a, s);
}

}  // namespace moe
