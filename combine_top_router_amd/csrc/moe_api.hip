// C ABI of libmoe: host-side argument checks, then kernel launches on the
// caller's stream. See include/moe.h for the contract of every call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moe

namespace {

constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxHidden = 16384;

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int32_t status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool desc_ok(const moe_layout_desc* d) {
  if (!d) return false;
  if (d->num_tokens < 0 || d->num_experts < 1 || d->num_experts > kMaxExperts) return false;
  if (d->top_k < 1 || d->top_k > std::min(d->num_experts, kMaxTopK)) return false;
  if (d->ep_size < 1 || d->ep_size > 64) return false;
  if (d->num_tokens % d->ep_size || d->num_experts % d->ep_size) return false;
  if (d->local_rank < -1 || d->local_rank >= d->ep_size) return false;
  if (d->align < 1 || d->align > 1024 || (d->align & (d->align - 1))) return false;
  if (int64_t(d->ep_size) * d->num_experts > 16384) return false;  // LDS of the scan
  if (d->num_tokens * d->top_k > (int64_t(1) << 31) - 1) return false;  // int32 flat index
  return true;
}

moe::LayoutPlan plan_of(const moe_layout_desc* d) {
  return moe::make_layout_plan(d->num_tokens, d->num_experts, d->top_k, d->ep_size,
                               d->local_rank, d->align);
}

int64_t m_cap_of(const moe_layout_desc* d) {
  const int64_t el = d->local_rank < 0 ? d->num_experts : d->num_experts / d->ep_size;
  return d->num_tokens * std::min<int64_t>(d->top_k, el) + el * (d->align - 1);
}

void put_detail(char* detail, size_t len, const char* fmt, long long a, long long b) {
  if (detail && len) std::snprintf(detail, len, fmt, a, b);
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_COVERAGE: return "MOE_ERR_COVERAGE";
    case MOE_ERR_EXPERT_ID: return "MOE_ERR_EXPERT_ID";
    case MOE_ERR_LAYOUT: return "MOE_ERR_LAYOUT";
    case MOE_ERR_TOO_LARGE: return "MOE_ERR_TOO_LARGE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int32_t moe_abi_version(void) { return 2; }

int32_t moe_route(const float* logits_d, int64_t num_tokens, int32_t num_experts, int32_t top_k,
                  int32_t* topk_idx_d, float* topk_w_d, void* stream) {
  if (num_tokens < 0 || num_experts < 1 || num_experts > kMaxExperts || top_k < 1 ||
      top_k > std::min(num_experts, kMaxTopK))
    return MOE_ERR_ARG;
  if (num_tokens > (int64_t(1) << 31) / top_k) return MOE_ERR_ARG;
  if (num_tokens == 0) return MOE_OK;
  if (!logits_d || !topk_idx_d || !topk_w_d) return MOE_ERR_ARG;
  return status_of(moe::launch_route(logits_d, num_tokens, num_experts, top_k, topk_idx_d,
                                     topk_w_d, as_stream(stream)));
}

int64_t moe_layout_m_cap(const moe_layout_desc* desc) {
  return desc_ok(desc) ? m_cap_of(desc) : -1;
}

size_t moe_layout_workspace_bytes(const moe_layout_desc* desc) {
  return desc_ok(desc) ? moe::layout_workspace_bytes(plan_of(desc)) : 0;
}

}  // extern "C"

namespace {

// moe_layout's checks of everything but the workspace
int32_t layout_args(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                    const int32_t* offsets_d, const int32_t* dst_row_d, const int32_t* src_row_d,
                    int64_t m_cap) {
  if (!desc_ok(desc)) return MOE_ERR_ARG;
  if (!offsets_d || !src_row_d) return MOE_ERR_ARG;
  if (desc->num_tokens > 0 && (!topk_idx_d || !dst_row_d)) return MOE_ERR_ARG;
  if (m_cap < m_cap_of(desc) || m_cap > (int64_t(1) << 31) - 1) return MOE_ERR_ARG;
  return MOE_OK;
}

// The layout's workspace for callers that cannot allocate: a static device
// array of MOE_LAYOUT_SCRATCH_BYTES. Each GPU the library runs on holds its
// own copy, at its own address, until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address of each GPU's copy comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address reaches a
// kernel. Nothing in the layout's workspace needs to start at zero: every
// word is written before it is read in the same call.
static __device__ __align__(256) char scratch[MOE_LAYOUT_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];  // device address of each GPU's copy, once looked up

int32_t scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_layout(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                   int32_t* expert_counts_d, int32_t* send_counts_d, int32_t* split_matrix_d,
                   int32_t* recv_counts_d, int32_t* output_splits_d, int32_t* offsets_d,
                   int32_t* dst_row_d, int32_t* src_row_d, int64_t m_cap, void* workspace_d,
                   size_t workspace_bytes, void* stream) {
  const int32_t st = layout_args(desc, topk_idx_d, offsets_d, dst_row_d, src_row_d, m_cap);
  if (st != MOE_OK) return st;
  if (!workspace_d || !aligned16(workspace_d)) return MOE_ERR_ARG;
  const moe::LayoutPlan p = plan_of(desc);
  if (workspace_bytes < moe::layout_workspace_bytes(p)) return MOE_ERR_ARG;
  return status_of(moe::launch_layout(p, topk_idx_d, expert_counts_d, send_counts_d,
                                      split_matrix_d, recv_counts_d, output_splits_d, offsets_d,
                                      dst_row_d, src_row_d, m_cap, workspace_d,
                                      as_stream(stream)));
}

int32_t moe_layout_noalloc(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                           int32_t* expert_counts_d, int32_t* send_counts_d,
                           int32_t* split_matrix_d, int32_t* recv_counts_d,
                           int32_t* output_splits_d, int32_t* offsets_d, int32_t* dst_row_d,
                           int32_t* src_row_d, int64_t m_cap, void* stream) {
  int32_t st = layout_args(desc, topk_idx_d, offsets_d, dst_row_d, src_row_d, m_cap);
  if (st != MOE_OK) return st;
  const moe::LayoutPlan p = plan_of(desc);
  if (moe::layout_workspace_bytes(p) > MOE_LAYOUT_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  return status_of(moe::launch_layout(p, topk_idx_d, expert_counts_d, send_counts_d,
                                      split_matrix_d, recv_counts_d, output_splits_d, offsets_d,
                                      dst_row_d, src_row_d, m_cap, ws, as_stream(stream)));
}

static bool dl_args_ok(int64_t T, int32_t E, int32_t k, int32_t ep) {
  return T >= 0 && T < (int64_t(1) << 31) / 64 && E >= 1 && E <= kMaxExperts && k >= 1 &&
         k <= std::min(E, kMaxTopK) && ep >= 1 && ep <= 64 && E % ep == 0;
}

size_t moe_dispatch_layout_workspace_bytes(int64_t num_tokens, int32_t num_experts,
                                           int32_t top_k, int32_t ep_size) {
  if (!dl_args_ok(num_tokens, num_experts, top_k, ep_size)) return 0;
  return moe::dispatch_layout_workspace_bytes(num_tokens, num_experts, ep_size);
}

int32_t moe_dispatch_layout(const int32_t* topk_idx_d, int64_t num_tokens, int32_t num_experts,
                            int32_t top_k, int32_t ep_size, int32_t* num_tokens_per_rank_d,
                            int32_t* num_tokens_per_expert_d, uint8_t* is_token_in_rank_d,
                            int32_t* token_rank_pos_d, void* workspace_d, size_t workspace_bytes,
                            void* stream) {
  if (!dl_args_ok(num_tokens, num_experts, top_k, ep_size)) return MOE_ERR_ARG;
  if (!num_tokens_per_rank_d || !num_tokens_per_expert_d) return MOE_ERR_ARG;
  const size_t need = moe::dispatch_layout_workspace_bytes(num_tokens, num_experts, ep_size);
  if (num_tokens > 0 && (!topk_idx_d || !is_token_in_rank_d || !token_rank_pos_d ||
                         !workspace_d || workspace_bytes < need))
    return MOE_ERR_ARG;
  return status_of(moe::launch_dispatch_layout(topk_idx_d, num_tokens, num_experts, top_k, ep_size,
                                               num_tokens_per_rank_d, num_tokens_per_expert_d,
                                               is_token_in_rank_d, token_rank_pos_d, workspace_d,
                                               as_stream(stream)));
}

int32_t moe_permute(const void* x_d, int64_t num_tokens, int32_t hidden, int32_t top_k,
                    const int32_t* dst_row_d, const int32_t* src_row_d, const int32_t* offsets_d,
                    int32_t num_local_experts, int64_t m_cap, void* x_perm_d, void* stream) {
  if (num_tokens < 0 || hidden < 8 || hidden > kMaxHidden || hidden % 8 || top_k < 1 ||
      top_k > kMaxTopK || m_cap < 0 || num_local_experts < 1 || num_local_experts > kMaxExperts)
    return MOE_ERR_ARG;
  if (m_cap == 0) return MOE_OK;
  if (!x_perm_d || !aligned16(x_perm_d) || !src_row_d || !offsets_d) return MOE_ERR_ARG;
  if (num_tokens > 0 && (!x_d || !dst_row_d || !aligned16(x_d))) return MOE_ERR_ARG;
  return status_of(moe::launch_permute(x_d, num_tokens, hidden, top_k, dst_row_d, nullptr, m_cap,
                                       x_perm_d, src_row_d, offsets_d, num_local_experts,
                                       as_stream(stream)));
}

int32_t moe_permute_weighted(const void* x_d, int64_t num_tokens, int32_t hidden, int32_t top_k,
                             const int32_t* dst_row_d, const float* topk_w_d, int64_t m_cap,
                             void* x_perm_d, void* stream) {
  if (num_tokens < 0 || hidden < 8 || hidden > kMaxHidden || hidden % 8 || top_k < 1 ||
      top_k > kMaxTopK || m_cap < 0)
    return MOE_ERR_ARG;
  if (num_tokens == 0) return MOE_OK;
  if (!x_d || !dst_row_d || !topk_w_d || !x_perm_d || !aligned16(x_d) || !aligned16(x_perm_d))
    return MOE_ERR_ARG;
  return status_of(moe::launch_permute(x_d, num_tokens, hidden, top_k, dst_row_d, topk_w_d, m_cap,
                                       x_perm_d, nullptr, nullptr, 0, as_stream(stream)));
}

int32_t moe_pack_weights(const void* w_d, int64_t num_mats, int32_t rows, int32_t cols,
                         void* wt_d, void* stream) {
  if (num_mats < 0 || num_mats > 65535 || rows < 0 || cols < 0) return MOE_ERR_ARG;
  if (num_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!w_d || !wt_d || w_d == wt_d) return MOE_ERR_ARG;
  if (rows % 128 || cols % 128) return MOE_ERR_UNSUPPORTED;
  return status_of(moe::launch_pack(w_d, num_mats, rows, cols, wt_d, as_stream(stream)));
}

static int32_t check_gemm(const void* a, const int32_t* offsets, const int32_t* counts, int32_t e_loc,
                          int64_t m_cap, int32_t k_dim, int32_t n_dim, const void* b0,
                          const void* b1, const void* c) {
  if (e_loc < 1 || e_loc > kMaxExperts || m_cap < 0 || k_dim < 1 || n_dim < 1) return MOE_ERR_ARG;
  if (!a || !offsets || !counts || !b0 || !b1 || !c) return MOE_ERR_ARG;
  if (!aligned16(a) || !aligned16(b0) || !aligned16(b1) || !aligned16(c)) return MOE_ERR_ARG;
  if (k_dim % 128 || n_dim % 128) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int32_t moe_grouped_gate_up(const void* x_perm_d, const int32_t* offsets_d,
                            const int32_t* counts_d, int32_t num_local_experts, int64_t m_cap,
                            int32_t hidden, int32_t inter, const void* w1t_d, const void* w3t_d,
                            void* h_d, void* stream) {
  const int32_t st = check_gemm(x_perm_d, offsets_d, counts_d, num_local_experts, m_cap, hidden,
                                inter, w1t_d, w3t_d, h_d);
  if (st != MOE_OK) return st;
  return status_of(moe::launch_gate_up(x_perm_d, offsets_d, counts_d, num_local_experts, m_cap,
                                       hidden, inter, w1t_d, w3t_d, h_d, as_stream(stream)));
}

int32_t moe_grouped_gate_up_gather(const void* x_d, int64_t num_tokens, int32_t top_k,
                                   const int32_t* src_row_d, const int32_t* offsets_d,
                                   const int32_t* counts_d, int32_t num_local_experts,
                                   int64_t m_cap, int32_t hidden, int32_t inter,
                                   const void* w1t_d, const void* w3t_d, void* h_d,
                                   void* stream) {
  const int32_t st = check_gemm(x_d, offsets_d, counts_d, num_local_experts, m_cap, hidden,
                                inter, w1t_d, w3t_d, h_d);
  if (st != MOE_OK) return st;
  if (num_tokens < 0 || top_k < 1 || top_k > kMaxTopK || (m_cap > 0 && !src_row_d))
    return MOE_ERR_ARG;
  // the token rows are addressed with 32-bit byte offsets
  if ((num_tokens + 1) * int64_t(hidden) * 2 >= (int64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  return status_of(moe::launch_gate_up_gather(x_d, num_tokens, top_k, src_row_d, offsets_d,
                                              counts_d, num_local_experts, m_cap, hidden, inter,
                                              w1t_d, w3t_d, h_d, as_stream(stream)));
}

int32_t moe_grouped_down(const void* h_d, const int32_t* offsets_d, const int32_t* counts_d,
                         int32_t num_local_experts, int64_t m_cap, int32_t inter, int32_t hidden,
                         const void* w2t_d, void* y_d, void* stream) {
  const int32_t st = check_gemm(h_d, offsets_d, counts_d, num_local_experts, m_cap, inter, hidden,
                                w2t_d, w2t_d, y_d);
  if (st != MOE_OK) return st;
  return status_of(moe::launch_down(h_d, offsets_d, counts_d, num_local_experts, m_cap, inter,
                                    hidden, w2t_d, y_d, as_stream(stream)));
}

int32_t moe_grouped_swiglu(const void* x_perm_d, const int32_t* offsets_d,
                           const int32_t* counts_d, int32_t num_local_experts, int64_t m_cap,
                           int32_t hidden, int32_t inter, const void* w1t_d, const void* w3t_d,
                           const void* w2t_d, void* h_d, void* y_d, void* stream) {
  int32_t st = check_gemm(x_perm_d, offsets_d, counts_d, num_local_experts, m_cap, hidden, inter,
                          w1t_d, w3t_d, h_d);
  if (st == MOE_OK)
    st = check_gemm(h_d, offsets_d, counts_d, num_local_experts, m_cap, inter, hidden, w2t_d,
                    w2t_d, y_d);
  if (st != MOE_OK) return st;
  st = moe_grouped_gate_up(x_perm_d, offsets_d, counts_d, num_local_experts, m_cap, hidden, inter,
                           w1t_d, w3t_d, h_d, stream);
  if (st != MOE_OK) return st;
  return moe_grouped_down(h_d, offsets_d, counts_d, num_local_experts, m_cap, inter, hidden,
                          w2t_d, y_d, stream);
}

int32_t moe_grouped_gate_up_save(const void* x_perm_d, const int32_t* offsets_d,
                                 const int32_t* counts_d, int32_t num_local_experts,
                                 int64_t m_cap, int32_t hidden, int32_t inter, const void* w1t_d,
                                 const void* w3t_d, void* h_d, void* gu_d, void* stream) {
  int32_t st = check_gemm(x_perm_d, offsets_d, counts_d, num_local_experts, m_cap, hidden, inter,
                          w1t_d, w3t_d, h_d);
  if (st == MOE_OK && (!gu_d || !aligned16(gu_d))) st = MOE_ERR_ARG;
  if (st != MOE_OK) return st;
  return status_of(moe::launch_gate_up_save(x_perm_d, offsets_d, counts_d, num_local_experts,
                                            m_cap, hidden, inter, w1t_d, w3t_d, h_d, gu_d,
                                            as_stream(stream)));
}

int32_t moe_grouped_down_backward(const void* dy_d, const void* gu_d, const int32_t* offsets_d,
                                  const int32_t* counts_d, int32_t num_local_experts,
                                  int64_t m_cap, int32_t inter, int32_t hidden, const void* w2_d,
                                  void* dgu_d, void* stream) {
  int32_t st = check_gemm(dy_d, offsets_d, counts_d, num_local_experts, m_cap, hidden, inter,
                          w2_d, w2_d, dgu_d);
  if (st == MOE_OK && (!gu_d || !aligned16(gu_d))) st = MOE_ERR_ARG;
  if (st != MOE_OK) return st;
  return status_of(moe::launch_down_backward(dy_d, gu_d, offsets_d, counts_d, num_local_experts,
                                             m_cap, inter, hidden, w2_d, dgu_d, as_stream(stream)));
}

int32_t moe_grouped_gate_up_backward(const void* dgu_d, const int32_t* offsets_d,
                                     const int32_t* counts_d, int32_t num_local_experts,
                                     int64_t m_cap, int32_t hidden, int32_t inter,
                                     const void* w1_d, const void* w3_d, void* dx_perm_d,
                                     void* stream) {
  const int32_t st = check_gemm(dgu_d, offsets_d, counts_d, num_local_experts, m_cap, inter,
                                hidden, w1_d, w3_d, dx_perm_d);
  if (st != MOE_OK) return st;
  return status_of(moe::launch_gate_up_backward(dgu_d, offsets_d, counts_d, num_local_experts,
                                                m_cap, hidden, inter, w1_d, w3_d, dx_perm_d,
                                                as_stream(stream)));
}

int32_t moe_grouped_gate_up_wgrad(const void* x_perm_d, const void* dgu_d,
                                  const int32_t* offsets_d, const int32_t* counts_d,
                                  int32_t num_local_experts, int64_t m_cap, int32_t hidden,
                                  int32_t inter, void* dw1_d, void* dw3_d, void* stream) {
  const int32_t st = check_gemm(x_perm_d, offsets_d, counts_d, num_local_experts, m_cap, hidden,
                                inter, dgu_d, dw1_d, dw3_d);
  if (st != MOE_OK) return st;
  return status_of(moe::launch_gate_up_wgrad(x_perm_d, dgu_d, offsets_d, counts_d,
                                             num_local_experts, m_cap, hidden, inter, dw1_d, dw3_d,
                                             as_stream(stream)));
}

int32_t moe_grouped_down_wgrad(const void* h_d, const void* dy_d, const int32_t* offsets_d,
                               const int32_t* counts_d, int32_t num_local_experts,
                               int64_t m_cap, int32_t inter, int32_t hidden, void* dw2_d,
                               void* stream) {
  const int32_t st = check_gemm(h_d, offsets_d, counts_d, num_local_experts, m_cap, inter, hidden,
                                dy_d, dy_d, dw2_d);
  if (st != MOE_OK) return st;
  return status_of(moe::launch_down_wgrad(h_d, dy_d, offsets_d, counts_d, num_local_experts,
                                          m_cap, inter, hidden, dw2_d, as_stream(stream)));
}

int32_t moe_combine(const void* y_d, int64_t y_rows, const int32_t* dst_row_d,
                    const float* topk_w_d, int64_t num_tokens, int32_t hidden, int32_t top_k,
                    void* out_d, void* stream) {
  if (num_tokens < 0 || y_rows < 0 || hidden < 8 || hidden > kMaxHidden || hidden % 8 ||
      top_k < 1 || top_k > kMaxTopK)
    return MOE_ERR_ARG;
  if (num_tokens == 0) return MOE_OK;
  if (!dst_row_d || !topk_w_d || !out_d || !aligned16(out_d)) return MOE_ERR_ARG;
  if (y_rows > 0 && (!y_d || !aligned16(y_d))) return MOE_ERR_ARG;
  return status_of(moe::launch_combine(y_d, y_rows, dst_row_d, topk_w_d, num_tokens, hidden,
                                       top_k, out_d, as_stream(stream)));
}

int32_t moe_combine_backward(const void* grad_out_d, const void* y_d, int64_t y_rows,
                             const int32_t* dst_row_d, const float* topk_w_d, int64_t num_tokens,
                             int32_t hidden, int32_t top_k, void* grad_y_d, float* grad_w_d,
                             void* stream) {
  if (num_tokens < 0 || y_rows < 0 || hidden < 8 || hidden > kMaxHidden || hidden % 8 ||
      top_k < 1 || top_k > kMaxTopK)
    return MOE_ERR_ARG;
  if (num_tokens == 0) return MOE_OK;
  if (!grad_out_d || !dst_row_d || !topk_w_d || !grad_w_d || !aligned16(grad_out_d))
    return MOE_ERR_ARG;
  if (y_rows > 0 && (!y_d || !grad_y_d || !aligned16(y_d) || !aligned16(grad_y_d)))
    return MOE_ERR_ARG;
  return status_of(moe::launch_combine_backward(grad_out_d, y_d, y_rows, dst_row_d, topk_w_d,
                                                num_tokens, hidden, top_k, grad_y_d, grad_w_d,
                                                as_stream(stream)));
}

int32_t moe_permute_backward(const void* grad_x_perm_d, int64_t x_perm_rows,
                             const int32_t* dst_row_d, int64_t num_tokens, int32_t hidden,
                             int32_t top_k, void* grad_x_d, void* stream) {
  if (num_tokens < 0 || x_perm_rows < 0 || hidden < 8 || hidden > kMaxHidden || hidden % 8 ||
      top_k < 1 || top_k > kMaxTopK)
    return MOE_ERR_ARG;
  if (num_tokens == 0) return MOE_OK;
  if (!dst_row_d || !grad_x_d || !aligned16(grad_x_d)) return MOE_ERR_ARG;
  if (x_perm_rows > 0 && (!grad_x_perm_d || !aligned16(grad_x_perm_d))) return MOE_ERR_ARG;
  return status_of(moe::launch_combine(grad_x_perm_d, x_perm_rows, dst_row_d, nullptr,
                                       num_tokens, hidden, top_k, grad_x_d, as_stream(stream)));
}

int32_t moe_route_backward(const int32_t* topk_idx_d, const float* topk_w_d,
                           const float* grad_w_d, int64_t num_tokens, int32_t num_experts,
                           int32_t top_k, float* grad_logits_d, void* stream) {
  if (num_tokens < 0 || num_experts < 1 || num_experts > kMaxExperts || top_k < 1 ||
      top_k > std::min(num_experts, kMaxTopK))
    return MOE_ERR_ARG;
  if (num_tokens > int64_t(UINT32_MAX) / num_experts) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  if (!topk_idx_d || !topk_w_d || !grad_w_d || !grad_logits_d) return MOE_ERR_ARG;
  return status_of(moe::launch_route_backward(topk_idx_d, topk_w_d, grad_w_d, num_tokens,
                                              num_experts, top_k, grad_logits_d,
                                              as_stream(stream)));
}

int32_t moe_combine_rows(const void* y_d, int32_t row_dtype, int64_t y_rows,
                         const int32_t* dst_row_d, const float* topk_w_d, const void* shared_d,
                         int64_t num_tokens, int32_t hidden, int32_t top_k, void* out_d,
                         void* stream) {
  if (num_tokens < 0 || y_rows < 0 || hidden < 8 || hidden > kMaxHidden || hidden % 8 ||
      top_k < 1 || top_k > kMaxTopK)
    return MOE_ERR_ARG;
  if (row_dtype != MOE_ROWS_BF16 && row_dtype != MOE_ROWS_F16 && row_dtype != MOE_ROWS_F32)
    return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  if (!dst_row_d || !out_d || !aligned16(out_d)) return MOE_ERR_ARG;
  if (y_rows > 0 && (!y_d || !aligned16(y_d))) return MOE_ERR_ARG;
  if (shared_d && !aligned16(shared_d)) return MOE_ERR_ARG;
  return status_of(moe::launch_combine_rows(y_d, row_dtype, y_rows, dst_row_d, topk_w_d, shared_d,
                                            num_tokens, hidden, top_k, out_d, as_stream(stream)));
}

int32_t moe_validate_layout(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                            const int32_t* offsets_d, const int32_t* dst_row_d,
                            const int32_t* src_row_d, int64_t m_cap, void* stream, char* detail,
                            size_t detail_len) {
  if (detail && detail_len) detail[0] = 0;
  if (!desc_ok(desc) || m_cap < 0 || !offsets_d || (m_cap > 0 && !src_row_d)) return MOE_ERR_ARG;
  const int64_t T = desc->num_tokens;
  const int k = desc->top_k, E = desc->num_experts;
  if (T > 0 && (!topk_idx_d || !dst_row_d)) return MOE_ERR_ARG;
  const int first = desc->local_rank < 0 ? 0 : desc->local_rank * (E / desc->ep_size);
  const int el = desc->local_rank < 0 ? E : E / desc->ep_size;
  const int64_t n = T * k;
  std::vector<int32_t> idx(n), dst(n), src(m_cap), off(el + 1);
  hipStream_t s = as_stream(stream);
  hipError_t err = hipSuccess;
  if (n) err = hipMemcpyAsync(idx.data(), topk_idx_d, n * 4, hipMemcpyDeviceToHost, s);
  if (n && err == hipSuccess) err = hipMemcpyAsync(dst.data(), dst_row_d, n * 4, hipMemcpyDeviceToHost, s);
  if (m_cap && err == hipSuccess)
    err = hipMemcpyAsync(src.data(), src_row_d, m_cap * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipMemcpyAsync(off.data(), offsets_d, (el + 1) * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return MOE_ERR_HIP;

  // expert ids in range and distinct per token
  for (int64_t t = 0; t < T; ++t)
    for (int a = 0; a < k; ++a) {
      const int e = idx[t * k + a];
      if (e < 0 || e >= E) {
        put_detail(detail, detail_len, "expert id out of range at token %lld slot %lld", t, a);
        return MOE_ERR_EXPERT_ID;
      }
      for (int b = 0; b < a; ++b)
        if (idx[t * k + b] == e) {
          put_detail(detail, detail_len, "token %lld repeats an expert at slot %lld", t, a);
          return MOE_ERR_EXPERT_ID;
        }
    }
  // offsets aligned, monotone, within m_cap
  if (off[0] != 0 || off[el] > m_cap) {
    put_detail(detail, detail_len, "offsets[0]=%lld offsets[E_loc]=%lld", off[0], off[el]);
    return MOE_ERR_LAYOUT;
  }
  for (int e = 0; e < el; ++e)
    if (off[e + 1] < off[e] || off[e + 1] % desc->align) {
      put_detail(detail, detail_len, "offsets not aligned/monotone at expert %lld (%lld)", e, off[e + 1]);
      return MOE_ERR_LAYOUT;
    }
  // every local (t, slot) has exactly one row in its expert's group, and back
  std::vector<int> claimed(m_cap, 0);
  for (int64_t f = 0; f < n; ++f) {
    const int e = idx[f] - first;
    const bool local = e >= 0 && e < el;
    const int r = dst[f];
    if (!local) {
      if (r != -1) {
        put_detail(detail, detail_len, "non-local flat index %lld has row %lld", f, r);
        return MOE_ERR_LAYOUT;
      }
      continue;
    }
    if (r < off[e] || r >= off[e + 1]) {
      put_detail(detail, detail_len, "flat index %lld has no row in its expert group (row %lld)", f, r);
      return MOE_ERR_COVERAGE;
    }
    if (claimed[r]++) {
      put_detail(detail, detail_len, "row %lld claimed twice (flat index %lld)", r, f);
      return MOE_ERR_COVERAGE;
    }
    if (src[r] != f) {
      put_detail(detail, detail_len, "src_row[%lld] != flat index %lld", r, f);
      return MOE_ERR_LAYOUT;
    }
  }
  // padding and tail rows are -1; groups hold ascending flat indices first
  for (int e = 0; e < el; ++e) {
    int64_t prev = -1;
    bool pad = false;
    for (int64_t r = off[e]; r < off[e + 1]; ++r) {
      if (src[r] < 0) {
        pad = true;
        continue;
      }
      if (pad || src[r] <= prev || !claimed[r]) {
        put_detail(detail, detail_len, "group of expert %lld out of order at row %lld", e, r);
        return MOE_ERR_LAYOUT;
      }
      prev = src[r];
    }
  }
  for (int64_t r = off[el]; r < m_cap; ++r)
    if (src[r] != -1) {
      put_detail(detail, detail_len, "tail row %lld is %lld, not -1", r, src[r]);
      return MOE_ERR_LAYOUT;
    }
  return MOE_OK;
}

}  // extern "C"
