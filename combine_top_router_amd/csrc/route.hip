// Token-choice top-k routing: one wavefront per token.
//
// Selection follows the token-choice top-k router of the AutoEP runtime
// (DeepSpeed AutoEP commit text, section "Attribution": ep_router.py after
// TorchTitan's TokenChoiceTopKRouter): per token the k largest logits,
// distinct experts, descending, ties to the lower expert id. Weights are the
// softmax over all experts renormalised over the selected ones, which is the
// softmax of the k selected logits; kept in fp32, the router dtype
// (DeepSpeed PR #8847, section "Change").
//
// Each lane holds up to VPL logits (expert ids lane, lane+64, ...) as 64-bit
// keys whose order is (logit descending, id ascending); k rounds of a wave
// max pick the winners. HBM-bound: T*E*4 bytes in, T*k*8 out.
#include "moe_internal.h"

namespace moe {
namespace {

// Order-preserving map of a finite fp32 to uint32 (-0.0 folded onto +0.0).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// Key: ordered logit in the high word, ~expert in the low word, so the max
// key is the largest logit and, among equal logits, the lowest expert id.
// 0 never occurs for a real expert (low word ~e != 0), so it marks "taken".
__device__ __forceinline__ uint64_t make_key(float f, int e) {
  return (static_cast<uint64_t>(ordered_bits(f)) << 32) | static_cast<uint32_t>(~e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out) {
  const int64_t t = uniform(static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave);
  if (t >= T) return;
  const int lane = lane_id();
  const float* row = logits + t * E;

  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? make_key(__builtin_nontemporal_load(row + e), e) : 0ull;
  }

  int my_e = 0;
  float my_l = 0.f, l_max = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = key[i] == best ? 0ull : key[i];
    const int e = static_cast<int>(~static_cast<uint32_t>(best));
    const float l = from_ordered(static_cast<uint32_t>(best >> 32));
    if (j == 0) l_max = l;
    if (lane == j) {
      my_e = e;
      my_l = l;
    }
  }

  // softmax over the selected logits, fp32
  float ex = lane < k ? expf(my_l - l_max) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off, kWave);
  // lanes 0..15 now all hold the sum over lanes 0..15 (k <= 16)
  if (lane < k) {
    idx_out[t * k + lane] = my_e;
    w_out[t * k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 block(256), grid(static_cast<unsigned>((T + 3) / 4));
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 512)
    route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
