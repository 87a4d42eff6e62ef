// Token-choice top-k routing.
//
// Selection follows the token-choice top-k router of the AutoEP runtime
// (DeepSpeed AutoEP commit text, section "Attribution": ep_router.py after
// TorchTitan's TokenChoiceTopKRouter): per token the k largest logits,
// distinct experts, descending, ties to the lower expert id. Weights are the
// softmax over all experts renormalised over the selected ones, which is the
// softmax of the k selected logits; kept in fp32, the router dtype
// (DeepSpeed PR #8847, section "Change").
//
// A group of G lanes (8, 16 or 32) owns one token, so a wavefront routes 64/G
// tokens at once; lane j of the group holds the VPL consecutive logits of
// experts j*VPL .. j*VPL+VPL-1 (one contiguous load per lane) as 64-bit keys
// whose order is (logit descending, id ascending). Each of the k rounds takes
// the lane's best key, a max inside the group (DPP exchanges within the
// group's 16-lane row), and retires the winner; lane j keeps the j-th winner.
// T*E*4 bytes in, T*k*8 out.
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
// The low word is unique per expert and never 0, so 0 marks a slot with no
// expert; a selected expert is retired by clearing its high word, which puts
// it below every finite logit (whose ordered bits are at least 0x00800000).
__device__ __forceinline__ uint64_t make_key(float f, int e) {
  return (static_cast<uint64_t>(ordered_bits(f)) << 32) | static_cast<uint32_t>(~e);
}

// 64-bit value of another lane of the same 16-lane DPP row (CTRL: a DPP
// row pattern), as two 32-bit DPP moves.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v >> 32), CTRL, 0xF, 0xF, false);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Max over the G lanes of a group, in every lane of the group. Inside a
// 16-lane row the exchanges are DPP moves (rotate by 8 and 4 for 16-lane
// groups, the half-row mirror for 8-lane groups, then two quad swaps); a
// 32-lane group first combines its two rows through a shuffle. Any pairing
// gives the same maximum.
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  if constexpr (G == 32) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), 16, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), 16, kWave);
    v = mx(v, (static_cast<uint64_t>(hi) << 32) | lo);
  }
  if constexpr (G >= 16) {
    v = mx(v, dpp64<0x128>(v));  // row_ror:8
    v = mx(v, dpp64<0x124>(v));  // row_ror:4
  } else {
    static_assert(G == 8, "groups of 8, 16 or 32 lanes");
    v = mx(v, dpp64<0x141>(v));  // row_half_mirror
  }
  v = mx(v, dpp64<0x4E>(v));  // quad_perm [2,3,0,1]
  v = mx(v, dpp64<0xB1>(v));  // quad_perm [1,0,3,2]
  return v;
}

template <int G, int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out) {
  const int64_t t = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / G;
  const int j = threadIdx.x % G;  // lane within the token's group
  // every lane of a group shares t; groups past T still run the shuffles
  // (they are all in the same wavefront) but load and store nothing
  const bool live = t < T;
  const float* row = logits + (live ? t : 0) * E;

  uint64_t key[VPL];
  const int e0 = j * VPL;
  const bool vec = E == G * VPL && (VPL % 4) == 0 &&
                   (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  if (live && vec) {
#pragma unroll
    for (int v = 0; v < VPL; v += 4) {
      const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0 + v));
#pragma unroll
      for (int u = 0; u < 4; ++u) key[v + u] = make_key(q[u], e0 + v + u);
    }
  } else {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = e0 + v;
      key[v] = (live && e < E) ? make_key(__builtin_nontemporal_load(row + e), e) : 0ull;
    }
  }

  int my_e = 0;
  float my_l = 0.f, l_max = 0.f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) best = key[v] > best ? key[v] : best;
    best = group_max_u64<G>(best);
    // retire the winner: the one key whose low word (its ~expert) matches
    const uint32_t won = static_cast<uint32_t>(best);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      key[v] = static_cast<uint32_t>(key[v]) == won ? (key[v] & 0xffffffffull) : key[v];
    const float l = from_ordered(static_cast<uint32_t>(best >> 32));
    if (r == 0) l_max = l;
    if (j == r) {
      my_e = static_cast<int>(~static_cast<uint32_t>(best));
      my_l = l;
    }
  }

  // softmax over the selected logits, fp32
  const float ex = j < k ? expf(my_l - l_max) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if (live && j < k) {
    idx_out[t * k + j] = my_e;
    w_out[t * k + j] = ex / sum;
  }
}

template <int G, int VPL>
void launch(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const int64_t per_block = 256 / G;
  const dim3 grid(static_cast<unsigned>((T + per_block - 1) / per_block));
  route_kernel<G, VPL><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 8)
    launch<8, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 16 && k <= 8)
    launch<8, 2>(logits, T, E, k, idx, w, s);
  else if (E <= 32 && k <= 8)
    launch<8, 4>(logits, T, E, k, idx, w, s);
  else if (E <= 64 && k <= 8)
    launch<8, 8>(logits, T, E, k, idx, w, s);
  else if (E <= 64)
    launch<16, 4>(logits, T, E, k, idx, w, s);
  else if (E <= 128)
    launch<16, 8>(logits, T, E, k, idx, w, s);
  else if (E <= 256)
    launch<16, 16>(logits, T, E, k, idx, w, s);
  else
    launch<32, 32>(logits, T, E, k, idx, w, s);
  return hipGetLastError();
}

}  // namespace moe
