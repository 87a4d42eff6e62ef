// Row movers of the layer: the expert-major permute (gather) and the fused
// weighted-sum combine (restore). Both are HBM-bound row copies: one
// wavefront per token, 16-byte bf16 vectors, lanes striding along the row so
// a wavefront moves 1 KiB of contiguous row per instruction.
//
// permute: the reorder-by-expert step of the AutoEP flow (DeepSpeed AutoEP
//   commit text, section "Design", runtime step 3), the local half of
//   DeepEP's dispatch (DeepEP issue #272). Token-major: each token row is read
//   once and written to each of its local rows, so HBM traffic is the
//   algorithmic minimum (T_local*H*2 read + N_local*H*2 written).
//
// combine: the fused weighted restore of DeepSpeed PR #8847 (sections
//   "Problem", "Change", "Benchmark"): per token, sum over slots in slot order
//   of fp32 weight x bf16 row, products and sums in fp32, one rounding to
//   bf16; rows addressed through dst_row (flat index token*top_k + slot).
//   Without a weight array every weight is 1: the sum of a token's local row
//   gradients, which is the permute's backward (a combine, DeepEP issue #272).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;  // one wavefront each

// Each lane buffers up to kBuf vectors of its token's row before storing.
constexpr int kBuf = 16;  // 16 x 64 lanes x 8 bf16 = 8192 elements per pass

// Padding rows of the expert groups: every row r below offsets[E_loc] whose
// src_row[r] is negative becomes zeros. The padding of a group is a run of up
// to align - 1 rows at its end, so rows are dealt out round-robin over the
// wavefronts doing this (row r to wavefront r mod W): each tests 64 of its
// rows per src_row load (one ballot), then zeroes its padding rows, 1 KiB per
// store instruction, and every run of padding spreads over as many
// wavefronts as it has rows. Run by the permute's last `nblocks` workgroups.
__device__ void pad_zero_rows(const int32_t* __restrict__ src_row,
                              const int32_t* __restrict__ offsets, int e_loc, int64_t m_cap,
                              int hv, u32x4* __restrict__ x_perm, int64_t block, int64_t nblocks) {
  const int64_t lim = min(m_cap, static_cast<int64_t>(max(offsets[e_loc], 0)));
  const int lane = lane_id();
  const int64_t W = nblocks * kTokensPerBlock;
  const int64_t w = block * kTokensPerBlock + threadIdx.x / kWave;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int64_t j0 = 0; w + j0 * W < lim; j0 += kWave) {
    const int64_t r = w + (j0 + lane) * W;
    uint64_t m = __ballot(r < lim && src_row[r] < 0);
    while (m) {
      const int i = __builtin_ctzll(m);
      m &= m - 1;
      u32x4* dst = x_perm + (w + (j0 + i) * W) * hv;
      for (int v = lane; v < hv; v += kWave) dst[v] = zero;
    }
  }
}

// With weights (the score applied before the experts) each copy is
// bf16(w[t, s] * x[t]), an fp32 product rounded once. Workgroups from
// tok_blocks on zero the padding rows instead (src_row given).
template <int K, bool WEIGHTED>
__global__ __launch_bounds__(256) void permute_kernel(const u32x4* __restrict__ x, int64_t T,
                                                      int hv, int k_rt,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ topk_w,
                                                      int64_t m_cap, u32x4* __restrict__ x_perm,
                                                      const int32_t* __restrict__ src_row,
                                                      const int32_t* __restrict__ offsets,
                                                      int e_loc, int64_t tok_blocks) {
#pragma clang fp contract(off)
  if (static_cast<int64_t>(blockIdx.x) >= tok_blocks) {
    pad_zero_rows(src_row, offsets, e_loc, m_cap, hv, x_perm, blockIdx.x - tok_blocks,
                  gridDim.x - tok_blocks);
    return;
  }
  const int k = K > 0 ? K : k_rt;
  const int64_t t = uniform(static_cast<int64_t>(blockIdx.x) * kTokensPerBlock +
                            threadIdx.x / kWave);
  if (t >= T) return;
  const int lane = lane_id();

  int64_t rows[16];
  float wts[16];  // read with the rows, ahead of the row loads
  int nvalid = 0;
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : 16); ++j) {
    if (j < k) {
      const int r = dst_row[t * k + j];
      rows[j] = (r >= 0 && r < m_cap) ? int64_t(r) : -1;
      wts[j] = WEIGHTED ? topk_w[t * k + j] : 1.0f;
      nvalid += rows[j] >= 0;
    } else {
      rows[j] = -1;
      wts[j] = 0.f;
    }
  }
  if (nvalid == 0) return;  // no local slot: this token's row is not read at all

  // vectors per lane per pass: the weighted copy's conversions need registers,
  // so it buffers fewer and keeps more wavefronts resident
  constexpr int NB = WEIGHTED ? kBuf / 2 : kBuf;
  const u32x4* src = x + t * hv;
  for (int base = 0; base < hv; base += NB * kWave) {
    u32x4 buf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int v = base + i * kWave + lane;
      if (v < hv) buf[i] = __builtin_nontemporal_load(src + v);
    }
#pragma unroll
    for (int j = 0; j < (K > 0 ? K : 16); ++j) {
      if (j >= k || rows[j] < 0) continue;
      u32x4* dst = x_perm + rows[j] * hv;
      if constexpr (WEIGHTED) {
        const float w = wts[j];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int v = base + i * kWave + lane;
          if (v < hv) {
            float f[8];
            unpack8(buf[i], f);
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] = w * f[q];
            dst[v] = pack8(f);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int v = base + i * kWave + lane;
          if (v < hv) dst[v] = buf[i];
        }
      }
    }
  }
}

// Row element types of the combine: bf16 (8 per 16-byte vector), fp16 (8),
// fp32 (4).
enum RowType { kRowBf16 = 0, kRowF16 = 1, kRowF32 = 2 };

template <int RT>
struct Rows {
  static constexpr int NV = RT == kRowF32 ? 4 : 8;  // elements per 16-byte vector
  __device__ static void load(const u32x4& v, float (&f)[NV]) {
    if constexpr (RT == kRowBf16) {
      unpack8(v, f);
    } else if constexpr (RT == kRowF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = v[i];
        f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(word & 0xffffu)));
        f[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(word >> 16)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
  }
  __device__ static u32x4 store(const float (&f)[NV]) {
    if constexpr (RT == kRowBf16) {
      return pack8(f);
    } else if constexpr (RT == kRowF16) {
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(f[2 * i]));  // nearest even
        const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(f[2 * i + 1]));
        v[i] = lo | (hi << 16);
      }
      return v;
    } else {
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
      return v;
    }
  }
};

// out[t] = round( sum over local slots, in slot order, of w[t, s] * y[r]
//                 (+ shared[t]) ), fp32 products and sums, one rounding to the
// row type. No weight array: every weight is 1. No shared rows: nothing added.
template <int K, int RT>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y, int64_t y_rows,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ topk_w,
                                                      const u32x4* __restrict__ shared,
                                                      int64_t T, int hv, int k_rt,
                                                      u32x4* __restrict__ out) {
  // fp32 product, then fp32 sum: two IEEE roundings per slot, never contracted
  // to an FMA, so the result is the plain fp32 slot-order sum
#pragma clang fp contract(off)
  using R = Rows<RT>;
  constexpr int NV = R::NV;
  const int k = K > 0 ? K : k_rt;
  constexpr int KM = K > 0 ? K : 16;
  const int64_t t = uniform(static_cast<int64_t>(blockIdx.x) * kTokensPerBlock +
                            threadIdx.x / kWave);
  if (t >= T) return;
  const int lane = lane_id();

  // the token's local slots, in slot order (wave-uniform: scalar registers)
  int64_t rows[KM];
  float w[KM];
  int nv = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      const int r = dst_row[t * k + j];
      if (r >= 0 && r < y_rows) {
        rows[nv] = int64_t(r);
        w[nv] = topk_w ? topk_w[t * k + j] : 1.0f;  // no weights: a plain sum
        ++nv;
      }
    }
  }

  // kU vectors per lane per round. The local slots go in groups of GS (the
  // whole token at top-k <= 2, pairs above): a group's loads are all issued
  // before its first product, so a wavefront keeps GS * kU KiB in flight, and
  // the products still run in slot order.
  constexpr int kU = 4;
  constexpr int GS = (K > 0 && K <= 2) ? K : 2;
  u32x4* dst = out + t * hv;
  for (int v0 = lane; v0 < hv; v0 += kU * kWave) {
    float acc[kU][NV];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int q = 0; q < NV; ++q) acc[u][q] = 0.f;
    // at top-k <= 2 one group (a compile-time trip count, so constant indices)
    for (int j0 = 0; (K > 0 && K <= 2) ? j0 < GS : j0 < nv; j0 += GS) {
      u32x4 in[GS][kU];
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        if (j0 + g < nv) {
          const u32x4* src = y + rows[j0 + g] * hv;
#pragma unroll
          for (int u = 0; u < kU; ++u)
            if (v0 + u * kWave < hv) in[g][u] = __builtin_nontemporal_load(src + v0 + u * kWave);
        }
      }
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        if (j0 + g < nv) {
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            if (v0 + u * kWave < hv) {
              float f[NV];
              R::load(in[g][u], f);
#pragma unroll
              for (int q = 0; q < NV; ++q) acc[u][q] = acc[u][q] + w[j0 + g] * f[q];
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * kWave;
      if (v < hv) {
        if (shared) {  // the shared expert's row joins before the one rounding
          float f[NV];
          R::load(__builtin_nontemporal_load(shared + t * hv + v), f);
#pragma unroll
          for (int q = 0; q < NV; ++q) acc[u][q] = acc[u][q] + f[q];
        }
        __builtin_nontemporal_store(R::store(acc[u]), dst + v);
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(const void* x, int64_t T, int H, int k, const int32_t* dst_row,
                          const float* topk_w, int64_t m_cap, void* x_perm,
                          const int32_t* src_row, const int32_t* offsets, int e_loc,
                          hipStream_t s) {
  // one workgroup per kTokensPerBlock tokens, then (with src_row) four per CU
  // for the padding rows
  const int64_t tok_blocks = (T + kTokensPerBlock - 1) / kTokensPerBlock;
  const int64_t pad_blocks = (src_row && m_cap > 0) ? 4 * device_cu_count() : 0;
  if (tok_blocks + pad_blocks == 0) return hipSuccess;
  const int hv = H / 8;
  const dim3 grid(static_cast<unsigned>(tok_blocks + pad_blocks));
  const u32x4* xs = static_cast<const u32x4*>(x);
  u32x4* xp = static_cast<u32x4*>(x_perm);
#define MOE_PERMUTE(KK)                                                                          \
  (topk_w ? permute_kernel<KK, true><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, topk_w, m_cap,  \
                                                          xp, src_row, offsets, e_loc, tok_blocks) \
          : permute_kernel<KK, false><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, topk_w, m_cap, \
                                                           xp, src_row, offsets, e_loc, tok_blocks))
  switch (k) {
    case 1: MOE_PERMUTE(1); break;
    case 2: MOE_PERMUTE(2); break;
    case 4: MOE_PERMUTE(4); break;
    case 6: MOE_PERMUTE(6); break;
    case 8: MOE_PERMUTE(8); break;
    default: MOE_PERMUTE(0); break;
  }
#undef MOE_PERMUTE
  return hipGetLastError();
}

template <int RT>
static void combine_for(const void* y, int64_t y_rows, const int32_t* dst_row, const float* w,
                        const void* shared, int64_t T, int H, int k, void* out, hipStream_t s) {
  const int hv = H / Rows<RT>::NV;
  const dim3 grid(static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock));
  const u32x4* ys = static_cast<const u32x4*>(y);
  const u32x4* sh = static_cast<const u32x4*>(shared);
  u32x4* o = static_cast<u32x4*>(out);
#define MOE_COMBINE(KK) combine_kernel<KK, RT><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, sh, T, hv, k, o)
  switch (k) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 6: MOE_COMBINE(6); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
}

hipError_t launch_combine(const void* y, int64_t y_rows, const int32_t* dst_row, const float* w,
                          int64_t T, int H, int k, void* out, hipStream_t s) {
  return launch_combine_rows(y, 0, y_rows, dst_row, w, nullptr, T, H, k, out, s);
}

hipError_t launch_combine_rows(const void* y, int row_type, int64_t y_rows,
                               const int32_t* dst_row, const float* w, const void* shared,
                               int64_t T, int H, int k, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (row_type) {
    case kRowBf16: combine_for<kRowBf16>(y, y_rows, dst_row, w, shared, T, H, k, out, s); break;
    case kRowF16: combine_for<kRowF16>(y, y_rows, dst_row, w, shared, T, H, k, out, s); break;
    default: combine_for<kRowF32>(y, y_rows, dst_row, w, shared, T, H, k, out, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
