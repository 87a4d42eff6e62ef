// One-time weight repack: wt[m, c, r] = w[m, r, c] (bf16 bit copy), turning
// math-orientation expert matrices into the output-major, reduction-
// contiguous layout the grouped GEMM streams (the load-time conversion into
// the grouped expert layout, DeepSpeed AutoEP commit text, section "Design":
// ep_repack.py). 64x64 tiles through LDS so both the read and the write are
// row-contiguous.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kT = 64;

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w, int rows,
                                                   int cols, uint16_t* __restrict__ wt) {
  __shared__ uint16_t tile[kT][kT + 2];
  const int64_t m = blockIdx.z;
  const int r0 = blockIdx.y * kT, c0 = blockIdx.x * kT;
  const uint16_t* src = w + m * int64_t(rows) * cols;
  uint16_t* dst = wt + m * int64_t(rows) * cols;
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;  // 64 x 4
  for (int i = ty; i < kT; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[int64_t(r) * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < kT; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[int64_t(c) * rows + r] = tile[tx][i];
  }
}

}  // namespace

hipError_t launch_pack(const void* w, int64_t mats, int rows, int cols, void* wt, hipStream_t s) {
  if (mats == 0 || rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((cols + kT - 1) / kT, (rows + kT - 1) / kT, static_cast<unsigned>(mats));
  pack_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(w), rows, cols,
                                   static_cast<uint16_t*>(wt));
  return hipGetLastError();
}

}  // namespace moe
