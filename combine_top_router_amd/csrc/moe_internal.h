// Internal helpers shared by the HIP kernels of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes = 8 bf16
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed lo|hi.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float from_bf16(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Eight bf16 in a 16-byte vector -> fp32.
__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// ---- buffer loads straight into LDS (shared by the matrix-core kernels)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for a raw byte range [base, base + bytes): loads past the
// end return zeros instead of touching memory.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));               // num_records
  r[3] = 0x00020000;  // raw 32-bit data format, no swizzle
  return r;
}

// 16 bytes per lane, memory -> LDS through the buffer path, no register
// staging: lane l's chunk lands at LDS byte lds_addr + 16*l. Issued through
// inline assembly so that the compiler does not wait for these transfers
// before unrelated LDS reads; the kernel waits for them itself (s_waitcnt
// vmcnt + barrier) before reading the stage they fill. The instruction has
// no register result.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t byte_off, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(byte_off), "s"(rsrc),
               "{m0}"(lds_addr)
               : "memory");
}

// As dma16, at byte offset voff + soff: a per-lane part that a loop can keep
// in one register and a wave-uniform part (a K-slice advance) in a scalar
// register. A loop that recomputes the per-lane register between transfers
// makes the compiler wait for the transfer that read it (it cannot see that
// the hardware read the address at issue), so the per-lane parts stay fixed.
// The buffer range check covers the per-lane part; callers keep soff within
// the same range (rows past the range are decided by voff alone).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                      uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
               "{m0}"(lds_addr)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A value every lane of the wave agrees on, moved to a scalar register.
__device__ __forceinline__ int64_t uniform(int64_t v) {
  uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Walks i = i0 .. i1-1 in batches of 8: load(i) for a whole batch is issued
// before any value is used (the loads of a run are independent), then
// use(i, value) in order. Returns nothing; use carries the state.
template <class L, class U>
__device__ __forceinline__ void batched_run(int i0, int i1, L&& load, U&& use) {
  for (int i = i0; i < i1; i += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i + u < i1 ? load(i + u) : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i + u < i1) use(i + u, v[u]);
  }
}

// f(std::integral_constant<int, q>) for q = 0, 1, ..., in order: a fully
// unrolled sequence whose steps can differ at compile time.
template <class F, int... Q>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, Q...>) {
  (f(std::integral_constant<int, Q>{}), ...);
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Host-side launchers, one per kernel family (defined in the .hip files).
// They assume arguments were checked by the C ABI layer.
namespace moe {

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s);

struct LayoutPlan {
  int64_t T;
  int E, k, ep, first, e_loc, align;
  int64_t chunk;      // assignments per source rank, (T/ep)*k
  int tile;           // assignments per tile (multiple of 256)
  int tiles_per_rank;
  int num_tiles;
  int key_bits;       // ballot rounds to tell local experts (and "not local") apart
};
LayoutPlan make_layout_plan(int64_t T, int E, int k, int ep, int local_rank, int align);
size_t layout_workspace_bytes(const LayoutPlan& p);
hipError_t launch_layout(const LayoutPlan& p, const int32_t* topk_idx, int32_t* expert_counts,
                         int32_t* send_counts, int32_t* split_matrix, int32_t* recv_counts,
                         int32_t* output_splits, int32_t* offsets, int32_t* dst_row,
                         int32_t* src_row, int64_t m_cap, void* ws, hipStream_t s);

// src_row, offsets and e_loc (or nullptr, nullptr, 0): also zero the padding
// rows of the expert groups below offsets[e_loc]
hipError_t launch_permute(const void* x, int64_t T, int H, int k, const int32_t* dst_row,
                          const float* topk_w, int64_t m_cap, void* x_perm,
                          const int32_t* src_row, const int32_t* offsets, int e_loc,
                          hipStream_t s);
hipError_t launch_combine(const void* y, int64_t y_rows, const int32_t* dst_row, const float* w,
                          int64_t T, int H, int k, void* out, hipStream_t s);
// row_type: 0 bf16, 1 fp16, 2 fp32; w and shared may be null
hipError_t launch_combine_rows(const void* y, int row_type, int64_t y_rows,
                               const int32_t* dst_row, const float* w, const void* shared,
                               int64_t T, int H, int k, void* out, hipStream_t s);
hipError_t launch_combine_backward(const void* grad_out, const void* y, int64_t y_rows,
                                   const int32_t* dst_row, const float* w, int64_t T, int H,
                                   int k, void* grad_y, float* grad_w, hipStream_t s);
hipError_t launch_route_backward(const int32_t* topk_idx, const float* topk_w,
                                 const float* grad_w, int64_t T, int E, int k,
                                 float* grad_logits, hipStream_t s);
// Packed expert-weight layout (written by launch_pack, read by the forward
// grouped GEMMs): for each matrix, its N output rows form blocks of
// R = packed_row_block(N) rows, and each block is stored as K / kPackedSlice
// consecutive [R][kPackedSlice] slices, so one K-slice of up to R rows of a
// block is a single contiguous run. Element (n, k) of matrix m sits at
//   m*N*K + (n / R) * K * R + (k / kPackedSlice) * R * kPackedSlice
//         + (n % R) * kPackedSlice + k % kPackedSlice.
constexpr int kPackedSlice = 64;
__host__ __device__ constexpr int packed_row_block(int n) { return n % 256 == 0 ? 256 : 128; }

hipError_t launch_pack(const void* w, int64_t mats, int rows, int cols, void* wt, hipStream_t s);

hipError_t launch_gate_up(const void* x_perm, const int32_t* offsets, const int32_t* counts,
                          int e_loc, int64_t m_cap, int H, int I, const void* w1t,
                          const void* w3t, void* h, hipStream_t s);
hipError_t launch_gate_up_gather(const void* x, int64_t T, int top_k, const int32_t* src_row,
                                 const int32_t* offsets, const int32_t* counts, int e_loc,
                                 int64_t m_cap, int H, int I, const void* w1t, const void* w3t,
                                 void* h, hipStream_t s);
hipError_t launch_down(const void* h, const int32_t* offsets, const int32_t* counts, int e_loc,
                       int64_t m_cap, int I, int H, const void* w2t, void* y, hipStream_t s);
hipError_t launch_gate_up_save(const void* x_perm, const int32_t* offsets, const int32_t* counts,
                               int e_loc, int64_t m_cap, int H, int I, const void* w1t,
                               const void* w3t, void* h, void* gu, hipStream_t s);
hipError_t launch_down_backward(const void* dy, const void* gu, const int32_t* offsets,
                                const int32_t* counts, int e_loc, int64_t m_cap, int I, int H,
                                const void* w2, void* dgu, hipStream_t s);
hipError_t launch_gate_up_backward(const void* dgu, const int32_t* offsets, const int32_t* counts,
                                   int e_loc, int64_t m_cap, int H, int I, const void* w1,
                                   const void* w3, void* dx, hipStream_t s);
hipError_t launch_gate_up_wgrad(const void* x_perm, const void* dgu, const int32_t* offsets,
                                const int32_t* counts, int e_loc, int64_t m_cap, int H, int I,
                                void* dw1, void* dw3, hipStream_t s);
hipError_t launch_down_wgrad(const void* h, const void* dy, const int32_t* offsets,
                             const int32_t* counts, int e_loc, int64_t m_cap, int I, int H,
                             void* dw2, hipStream_t s);
size_t dispatch_layout_workspace_bytes(int64_t T, int E, int ep);
hipError_t launch_dispatch_layout(const int32_t* idx, int64_t T, int E, int k, int ep,
                                  int32_t* per_rank, int32_t* per_expert, uint8_t* in_rank,
                                  int32_t* pos, void* ws, hipStream_t s);

int device_cu_count();

}  // namespace moe
