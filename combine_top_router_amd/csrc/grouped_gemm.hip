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
//    operands are read K-contiguous (weights are stored output-major,
//    [E, N, K], by the one-time repack).
//  * Workgroup tile BM x BN (x2 for the gated pair), K staged through LDS in
//    64-element slices (128-byte rows, 16-byte chunks XOR-swizzled by row so
//    the MFMA fragment reads spread over the banks), two LDS stages: the
//    next slice is fetched into registers while the matrix cores work on the
//    current one.
//  * Ragged groups: each workgroup derives the per-expert m-tile prefix from
//    the device-side counts (no host sync, grid sized for the chip, not for
//    the routing), then walks tile ids persistently. Ids run expert-major,
//    then n-tile, then m-tile, and each of the 8 XCDs gets a contiguous range
//    of ids, so the workgroups sharing a weight tile or an activation tile
//    sit behind the same L2.
//  * Rows past an expert's count are zero-filled in LDS and never stored.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;           // K per LDS stage: 64 bf16 = 128 B per row
constexpr int kThreads = 256;     // 4 wavefronts, 2 (M) x 2 (N)
constexpr int kMaxExperts = 1024;

struct GemmArgs {
  const uint16_t* a;       // [rows, K] bf16
  const uint16_t* b0;      // [E_loc, N, K] bf16
  const uint16_t* b1;      // [E_loc, N, K] bf16 (gated only)
  uint16_t* c;             // [rows, N] bf16
  const int32_t* offsets;  // [E_loc + 1]
  const int32_t* counts;   // [E_loc]
  int e_loc;
  int n, k;
};

// byte offset of 16-byte chunk `ch` of row `row` in a [rows][64] bf16 stage
__device__ __forceinline__ int swz(int row, int ch) { return row * 128 + ((ch ^ (row & 7)) << 4); }

__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

template <int BM, int BN, bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;    // wavefront tile
  constexpr int TM = WM / 32, TN = WN / 32;  // MFMA tiles per wavefront
  constexpr int NB = GATED ? 2 : 1;          // B operands
  constexpr int A_LD = BM * kBK / 8 / kThreads;  // 16-byte chunks per thread per stage
  constexpr int B_LD = BN * kBK / 8 / kThreads;
  constexpr int A_BYTES = BM * kBK * 2, B_BYTES = BN * kBK * 2;
  constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ int mt_prefix[kMaxExperts + 1];
  __shared__ int wave_tot[kThreads / kWave];

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const int wm = wid / 2, wn = wid % 2;
  const int K = g.k, N = g.n;
  const int NT = N / BN, KT = K / kBK;

  // ---- m-tiles per local expert, exclusive prefix (each thread: 4 experts)
  {
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      v[q] = e < g.e_loc ? (g.counts[e] + BM - 1) / BM : 0;
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
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e < g.e_loc) mt_prefix[e] = ex;
      ex += v[q];
    }
    if (tid == kThreads - 1) mt_prefix[g.e_loc] = ex;  // grand total
    __syncthreads();
  }
  const int total = mt_prefix[g.e_loc] * NT;

  const int G = gridDim.x;
  int slot = blockIdx.x;
  if ((G & 7) == 0) slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // global->LDS assignment: chunk (tid % 8) of rows tid/8 + 32*i
  const int ld_ch = tid & 7, ld_row = tid >> 3;

  for (int tile = slot; tile < total; tile += G) {
    // ---- decode tile -> (expert, n-tile, m-tile)
    int lo = 0, hi = g.e_loc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mt_prefix[mid] * NT <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int mtiles = mt_prefix[e + 1] - mt_prefix[e];
    const int rem = tile - mt_prefix[e] * NT;
    const int nt = rem / mtiles, mt = rem % mtiles;
    const int64_t row0 = int64_t(g.offsets[e]) + int64_t(mt) * BM;
    const int rows_valid = min(BM, g.counts[e] - mt * BM);

    const uint16_t* A = g.a + row0 * K;
    const uint16_t* B0 = g.b0 + (int64_t(e) * N + int64_t(nt) * BN) * K;
    const uint16_t* B1 = GATED ? g.b1 + (int64_t(e) * N + int64_t(nt) * BN) * K : nullptr;

    u32x4 ra[A_LD], rb0[B_LD], rb1[GATED ? B_LD : 1];
    auto fetch = [&](int kt) {
      const int k0 = kt * kBK + ld_ch * 8;
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int r = ld_row + 32 * i;
        ra[i] = r < rows_valid ? *reinterpret_cast<const u32x4*>(A + int64_t(r) * K + k0)
                               : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int r = ld_row + 32 * i;
        rb0[i] = *reinterpret_cast<const u32x4*>(B0 + int64_t(r) * K + k0);
        if constexpr (GATED) rb1[i] = *reinterpret_cast<const u32x4*>(B1 + int64_t(r) * K + k0);
      }
    };
    auto stash = [&](int st) {
      char* base = smem + st * STAGE;
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        *reinterpret_cast<u32x4*>(base + swz(ld_row + 32 * i, ld_ch)) = ra[i];
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        *reinterpret_cast<u32x4*>(base + A_BYTES + swz(ld_row + 32 * i, ld_ch)) = rb0[i];
        if constexpr (GATED)
          *reinterpret_cast<u32x4*>(base + A_BYTES + B_BYTES + swz(ld_row + 32 * i, ld_ch)) =
              rb1[i];
      }
    };

    f32x16 acc[NB][TM][TN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[b][i][j][q] = 0.f;

    fetch(0);
    stash(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) fetch(kt + 1);
      const char* base = smem + cur * STAGE;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ch = 2 * kk + (lane >> 5);
        bf16x8 af[TM], bf[NB][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(base + swz(wm * WM + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            bf[b][j] = *reinterpret_cast<const bf16x8*>(
                base + A_BYTES + b * B_BYTES + swz(wn * WN + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[b][i][j] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[b][j], acc[b][i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) stash(cur ^ 1);
      __syncthreads();
    }

    // ---- epilogue: lane holds column (lane % 32), rows 8*(q/4) + 4*(lane/32) + q%4
    uint16_t* C = g.c + row0 * N + int64_t(nt) * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * WM + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
          const int col = wn * WN + j * 32 + (lane & 31);
          if (r < rows_valid) {
            float v = acc[0][i][j][q];
            if constexpr (GATED) v = silu(v) * acc[NB - 1][i][j][q];
            C[int64_t(r) * N + col] = to_bf16(v);
          }
        }
  }
}

template <int BM, int BN, bool GATED>
hipError_t launch_grouped(const GemmArgs& a, hipStream_t s) {
  // workgroups per CU that fit in LDS (160 KiB per CU on gfx950)
  constexpr int lds = 2 * (BM * kBK * 2 + (GATED ? 2 : 1) * BN * kBK * 2) + 4 * (kMaxExperts + 5);
  const int per_cu = std::max(1, std::min(2, (160 * 1024) / lds));
  const int grid = device_cu_count() * per_cu;
  grouped_gemm_kernel<BM, BN, GATED><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const void* x_perm, const int32_t* offsets, const int32_t* counts,
                          int e_loc, int64_t m_cap, int H, int I, const void* w1t,
                          const void* w3t, void* h, hipStream_t s) {
  (void)m_cap;
  GemmArgs a{static_cast<const uint16_t*>(x_perm), static_cast<const uint16_t*>(w1t),
             static_cast<const uint16_t*>(w3t), static_cast<uint16_t*>(h), offsets, counts,
             e_loc, I, H};
  return launch_grouped<128, 128, true>(a, s);
}

hipError_t launch_down(const void* h, const int32_t* offsets, const int32_t* counts, int e_loc,
                       int64_t m_cap, int I, int H, const void* w2t, void* y, hipStream_t s) {
  (void)m_cap;
  GemmArgs a{static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w2t), nullptr,
             static_cast<uint16_t*>(y), offsets, counts, e_loc, H, I};
  return launch_grouped<128, 128, false>(a, s);
}

}  // namespace moe
