// One-time weight repack: math-orientation expert matrices w[m, r, c]
// (r < rows = K, the reduction dimension; c < cols = N, the output dimension)
// become the packed layout the forward grouped GEMMs stream (the load-time
// conversion into the grouped expert layout, DeepSpeed AutoEP commit text,
// section "Design": ep_repack.py): output-major with K contiguous, and the N
// rows cut into blocks of packed_row_block(N) rows whose K-slices of
// kPackedSlice values are each one contiguous run, so a GEMM tile's B slice
// is a single sequential read. A bf16 bit copy: 64x64 tiles through LDS, so
// the reads are row-contiguous and the writes 128-byte runs.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kT = 64;

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w, int rows,
                                                   int cols, uint16_t* __restrict__ wt) {
  static_assert(kT == kPackedSlice, "one tile column is one packed K-slice");
  __shared__ uint16_t tile[kT][kT + 2];
  const int64_t m = blockIdx.z;
  const int r0 = blockIdx.y * kT, c0 = blockIdx.x * kT;
  const int R = packed_row_block(cols);
  const uint16_t* src = w + m * int64_t(rows) * cols;
  // this tile's K-slice r0 / kT of the row blocks
  uint16_t* dst = wt + m * int64_t(rows) * cols + int64_t(r0 / kT) * R * kT;
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;  // 64 x 4
  for (int i = ty; i < kT; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[int64_t(r) * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < kT; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols)
      dst[int64_t(c / R) * rows * R + (c % R) * kT + tx] = tile[tx][i];
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
