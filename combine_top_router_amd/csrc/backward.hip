// Backward of the routing softmax and of the fused combine.
//
// The fused restore of DeepSpeed PR #8847 back-propagates a row gradient and
// a score gradient (section "Tests"), the score gradient in FP32 (section
// "Benchmark"). The backward of a combine is a dispatch of the output
// gradient (DeepEP issue #272, the maintainer's answer), here to the local
// rows the forward read:
//
//   grad_y[r]    = bf16(w[t, s] * G[t])          r = dst_row[t, s] >= 0, fp32 product
//   grad_w[t, s] = <G[t], y[r]> in fp32          0 where the slot is not local
//
// The routing weights are the softmax of the k selected logits, so their
// gradient reaches the logits as
//
//   grad_logits[t, e_j] = w_j * (g_j - sum_i w_i g_i),  0 for unselected experts.
//
// The permute's backward is a combine with unit weights (launch_combine with
// no weight array).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;  // one wavefront each

// One wavefront per token: the output-gradient row is read once; each local
// slot's y row is read once and its gradient row written once. The score
// dot product keeps one fp32 partial per (slot, element of the 16-byte
// vector) in each lane, then sums the eight by halves and the 64 lanes by a
// butterfly: a tree-shaped fp32 reduction. bf16 x bf16 products are exact in
// fp32, so only the additions round.
template <int K>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const u32x4* __restrict__ grad_out, const u32x4* __restrict__ y, int64_t y_rows,
    const int32_t* __restrict__ dst_row, const float* __restrict__ topk_w, int64_t T, int hv,
    int k_rt, u32x4* __restrict__ grad_y, float* __restrict__ grad_w) {
#pragma clang fp contract(off)
  const int k = K > 0 ? K : k_rt;
  constexpr int KM = K > 0 ? K : 16;
  const int64_t t = uniform(static_cast<int64_t>(blockIdx.x) * kTokensPerBlock +
                            threadIdx.x / kWave);
  if (t >= T) return;
  const int lane = lane_id();

  int64_t rows[KM];
  float w[KM];
  int nvalid = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      const int r = dst_row[t * k + j];
      rows[j] = (r >= 0 && r < y_rows) ? int64_t(r) : -1;
      w[j] = topk_w[t * k + j];
      nvalid += rows[j] >= 0;
    } else {
      rows[j] = -1;
      w[j] = 0.f;
    }
  }
  if (nvalid == 0) {  // nothing of this token is on this share
    if (lane < k) grad_w[t * k + lane] = 0.f;
    return;
  }

  float dot[KM][8];
#pragma unroll
  for (int j = 0; j < KM; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) dot[j][q] = 0.f;

  // kU vectors per lane per round (ascending, so each lane's partial sums
  // take the row in the same order as one vector at a time), each slot's
  // loads issued together before its products
  constexpr int kU = 4;
  const u32x4* g_row = grad_out + t * hv;
  for (int v0 = lane; v0 < hv; v0 += kU * kWave) {
    u32x4 graw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (v0 + u * kWave < hv) graw[u] = __builtin_nontemporal_load(g_row + v0 + u * kWave);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (rows[j] < 0) continue;
      u32x4 yraw[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (v0 + u * kWave < hv) yraw[u] = __builtin_nontemporal_load(y + rows[j] * hv + v0 + u * kWave);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int v = v0 + u * kWave;
        if (v < hv) {
          float g[8], yv[8], gy[8];
          unpack8(graw[u], g);
          unpack8(yraw[u], yv);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            dot[j][q] = dot[j][q] + g[q] * yv[q];
            gy[q] = w[j] * g[q];
          }
          __builtin_nontemporal_store(pack8(gy), grad_y + rows[j] * hv + v);
        }
      }
    }
  }

#pragma unroll
  for (int j = 0; j < KM; ++j) {
    float s = ((dot[j][0] + dot[j][1]) + (dot[j][2] + dot[j][3])) +
              ((dot[j][4] + dot[j][5]) + (dot[j][6] + dot[j][7]));
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) s = s + __shfl_xor(s, off, kWave);
    if (lane == 0 && j < k) grad_w[t * k + j] = rows[j] >= 0 ? s : 0.f;
  }
}

// One thread per (token, expert) entry of grad_logits: the selected entries
// get the softmax gradient, the rest zero. sum_i w_i g_i is formed in fp32 in
// slot order.
__global__ __launch_bounds__(256) void route_backward_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ grad_w, uint32_t total, int E, int k,
    float* __restrict__ grad_logits) {
#pragma clang fp contract(off)
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= total) return;
  const uint32_t t = i / static_cast<uint32_t>(E);
  const int e = static_cast<int>(i - t * static_cast<uint32_t>(E));
  const size_t base = size_t(t) * k;
  float s = 0.f;
  int sel = -1;
  for (int j = 0; j < k; ++j) {
    s = s + topk_w[base + j] * grad_w[base + j];
    if (topk_idx[base + j] == e) sel = j;
  }
  grad_logits[i] = sel < 0 ? 0.f : topk_w[base + sel] * (grad_w[base + sel] - s);
}

}  // namespace

hipError_t launch_combine_backward(const void* grad_out, const void* y, int64_t y_rows,
                                   const int32_t* dst_row, const float* w, int64_t T, int H,
                                   int k, void* grad_y, float* grad_w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int hv = H / 8;
  const dim3 grid(static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock));
  const u32x4* g = static_cast<const u32x4*>(grad_out);
  const u32x4* ys = static_cast<const u32x4*>(y);
  u32x4* gy = static_cast<u32x4*>(grad_y);
#define MOE_CB(KK)                                                                              \
  combine_backward_kernel<KK><<<grid, 256, 0, s>>>(g, ys, y_rows, dst_row, w, T, hv, k, gy, \
                                                   grad_w)
  switch (k) {
    case 1: MOE_CB(1); break;
    case 2: MOE_CB(2); break;
    case 4: MOE_CB(4); break;
    case 6: MOE_CB(6); break;
    case 8: MOE_CB(8); break;
    default: MOE_CB(0); break;
  }
#undef MOE_CB
  return hipGetLastError();
}

hipError_t launch_route_backward(const int32_t* topk_idx, const float* topk_w,
                                 const float* grad_w, int64_t T, int E, int k,
                                 float* grad_logits, hipStream_t s) {
  const int64_t total = T * E;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  route_backward_kernel<<<grid, 256, 0, s>>>(topk_idx, topk_w, grad_w,
                                             static_cast<uint32_t>(total), E, k, grad_logits);
  return hipGetLastError();
}

}  // namespace moe
