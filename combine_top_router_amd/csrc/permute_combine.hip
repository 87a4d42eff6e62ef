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

template <int K>
__global__ __launch_bounds__(256) void permute_kernel(const u32x4* __restrict__ x, int64_t T,
                                                      int hv, int k_rt,
                                                      const int32_t* __restrict__ dst_row,
                                                      int64_t m_cap, u32x4* __restrict__ x_perm) {
  const int k = K > 0 ? K : k_rt;
  const int64_t t = uniform(static_cast<int64_t>(blockIdx.x) * kTokensPerBlock +
                            threadIdx.x / kWave);
  if (t >= T) return;
  const int lane = lane_id();

  int64_t rows[16];
  int nvalid = 0;
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : 16); ++j) {
    if (j < k) {
      const int r = dst_row[t * k + j];
      rows[j] = (r >= 0 && r < m_cap) ? int64_t(r) : -1;
      nvalid += rows[j] >= 0;
    } else {
      rows[j] = -1;
    }
  }
  if (nvalid == 0) return;  // no local slot: this token's row is not read at all

  const u32x4* src = x + t * hv;
  for (int base = 0; base < hv; base += kBuf * kWave) {
    u32x4 buf[kBuf];
#pragma unroll
    for (int i = 0; i < kBuf; ++i) {
      const int v = base + i * kWave + lane;
      if (v < hv) buf[i] = __builtin_nontemporal_load(src + v);
    }
#pragma unroll
    for (int j = 0; j < (K > 0 ? K : 16); ++j) {
      if (j >= k || rows[j] < 0) continue;
      u32x4* dst = x_perm + rows[j] * hv;
#pragma unroll
      for (int i = 0; i < kBuf; ++i) {
        const int v = base + i * kWave + lane;
        if (v < hv) dst[v] = buf[i];
      }
    }
  }
}

template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y, int64_t y_rows,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ topk_w,
                                                      int64_t T, int hv, int k_rt,
                                                      u32x4* __restrict__ out) {
  // fp32 product, then fp32 sum: two IEEE roundings per slot, never contracted
  // to an FMA, so the result is the plain fp32 slot-order sum
#pragma clang fp contract(off)
  const int k = K > 0 ? K : k_rt;
  constexpr int KM = K > 0 ? K : 16;
  const int64_t t = uniform(static_cast<int64_t>(blockIdx.x) * kTokensPerBlock +
                            threadIdx.x / kWave);
  if (t >= T) return;
  const int lane = lane_id();

  int64_t rows[KM];
  float w[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      const int r = dst_row[t * k + j];
      rows[j] = (r >= 0 && r < y_rows) ? int64_t(r) : -1;
      w[j] = topk_w ? topk_w[t * k + j] : 1.0f;  // no weights: the permute's backward
    } else {
      rows[j] = -1;
      w[j] = 0.f;
    }
  }

  u32x4* dst = out + t * hv;
  for (int v = lane; v < hv; v += kWave) {
    u32x4 in[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (rows[j] >= 0) in[j] = __builtin_nontemporal_load(y + rows[j] * hv + v);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (rows[j] < 0) continue;
      float f[8];
      unpack8(in[j], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = acc[q] + w[j] * f[q];
    }
    __builtin_nontemporal_store(pack8(acc), dst + v);
  }
}

}  // namespace

hipError_t launch_permute(const void* x, int64_t T, int H, int k, const int32_t* dst_row,
                          int64_t m_cap, void* x_perm, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int hv = H / 8;
  const dim3 grid(static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock));
  const u32x4* xs = static_cast<const u32x4*>(x);
  u32x4* xp = static_cast<u32x4*>(x_perm);
  switch (k) {
    case 1: permute_kernel<1><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, m_cap, xp); break;
    case 2: permute_kernel<2><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, m_cap, xp); break;
    case 4: permute_kernel<4><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, m_cap, xp); break;
    case 6: permute_kernel<6><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, m_cap, xp); break;
    case 8: permute_kernel<8><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, m_cap, xp); break;
    default: permute_kernel<0><<<grid, 256, 0, s>>>(xs, T, hv, k, dst_row, m_cap, xp); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, int64_t y_rows, const int32_t* dst_row, const float* w,
                          int64_t T, int H, int k, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int hv = H / 8;
  const dim3 grid(static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock));
  const u32x4* ys = static_cast<const u32x4*>(y);
  u32x4* o = static_cast<u32x4*>(out);
  switch (k) {
    case 1: combine_kernel<1><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, T, hv, k, o); break;
    case 2: combine_kernel<2><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, T, hv, k, o); break;
    case 4: combine_kernel<4><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, T, hv, k, o); break;
    case 6: combine_kernel<6><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, T, hv, k, o); break;
    case 8: combine_kernel<8><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, T, hv, k, o); break;
    default: combine_kernel<0><<<grid, 256, 0, s>>>(ys, y_rows, dst_row, w, T, hv, k, o); break;
  }
  return hipGetLastError();
}

}  // namespace moe
