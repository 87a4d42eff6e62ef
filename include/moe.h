/*
 * moe.h -- C ABI of libmoe.so, the single-GPU MoE-layer hot path for AMD
 * Instinct MI355X (gfx950):
 *
 *   moe_route -> moe_layout -> moe_permute -> moe_grouped_swiglu -> moe_combine
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument named *_d is DEVICE memory on the current HIP
 *   device; descriptors (moe_layout_desc) are HOST memory. The caller owns
 *   and allocates every buffer; the library allocates nothing, keeps no state
 *   between calls and never blocks the host (moe_validate_layout excepted).
 *   The one exception to the ownership rule is moe_layout_noalloc, whose
 *   workspace is a static device array of the library (one per GPU). The
 *   weight-gradient calls also use small library-held device counters, one
 *   pair per stream, which each call leaves at zero.
 * - `stream` is a hipStream_t (NULL = the default stream). Each call only
 *   enqueues kernels on it and returns; results are ready when the stream
 *   reaches that point. Calls on different streams may run concurrently as
 *   long as they do not share output buffers.
 * - bf16 buffers hold IEEE bfloat16 bit patterns (uint16); float is fp32;
 *   indices are int32. Matrices are row-major and densely packed.
 * - Return value: a moe_status. Argument checks run on the host before any
 *   launch: a call that returns anything but MOE_OK has enqueued nothing.
 *   MOE_ERR_HIP reports a failed launch (hipGetLastError after the launch).
 * - Data errors (an expert id out of [0, E), a row index past the end of a
 *   buffer) are not diagnosed on the fast path; the kernels skip such
 *   entries so every access stays in bounds. moe_validate_layout reports them.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null pointer, size out of range, misaligned buffer,
                               workspace or m_cap too small */
  MOE_ERR_UNSUPPORTED = 2,  /* a shape the kernels do not implement (see each call) */
  MOE_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed */
  MOE_ERR_COVERAGE = 4,     /* validator: a (token, slot) is missing or covered twice */
  MOE_ERR_EXPERT_ID = 5,    /* validator: expert id out of range or repeated in a token */
  MOE_ERR_LAYOUT = 6,       /* validator: offsets / src_row / dst_row inconsistent */
  MOE_ERR_TOO_LARGE = 7     /* moe_layout_noalloc: the layout needs more scratch than the
                               library's static array holds */
} moe_status;

/* Static name of a status code ("MOE_OK", ...); never NULL. */
const char* moe_status_string(int32_t status);

/* ABI version of this header; bumped on any incompatible change. */
int32_t moe_abi_version(void);

/*
 * moe_route -- token-choice top-k routing.
 *
 * Follows the token-choice top-k router of the AutoEP runtime (DeepSpeed
 * AutoEP commit text, section "Attribution": ep_router.py after TorchTitan's
 * TokenChoiceTopKRouter; section "Design", runtime step 2), with distinct
 * experts per token (DeepSpeed PR #8847, section "Benchmark") and FP32
 * routing weights kept in the router dtype (same page, section "Change").
 * Per token t: the k experts with the largest logits[t, :], in descending
 * order, ties to the lower expert id (-0.0 equals +0.0); weights are the
 * softmax over all E experts renormalised over the k selected, computed as
 * exp(l_j - l_max) / sum_selected exp(l_i - l_max) in fp32.
 *
 *   logits_d    [T, E] float, finite values
 *   topk_idx_d  [T, k] int32 (out)
 *   topk_w_d    [T, k] float (out)
 * Limits: T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 16). T = 0 is a no-op.
 */
int32_t moe_route(const float* logits_d, int64_t num_tokens, int32_t num_experts,
                  int32_t top_k, int32_t* topk_idx_d, float* topk_w_d, void* stream);

/*
 * Layout of one GPU's share when `ep_size` virtual ranks split the work:
 * source rank s owns tokens [s*T/ep, (s+1)*T/ep); destination rank d owns
 * experts [d*E/ep, (d+1)*E/ep); this GPU is destination `local_rank`
 * (-1: every expert is local, E_loc = E; otherwise E_loc = E/ep).
 */
typedef struct moe_layout_desc {
  int64_t num_tokens;  /* T, a multiple of ep_size */
  int32_t num_experts; /* E, a multiple of ep_size, <= 1024 */
  int32_t top_k;       /* k, 1..min(E, 16) */
  int32_t ep_size;     /* >= 1, <= 64 */
  int32_t local_rank;  /* -1 or 0..ep_size-1 */
  int32_t align;       /* row alignment of each local expert's group, power of two <= 1024 */
} moe_layout_desc;

/* Worst-case local rows: T*min(k, E_loc) + E_loc*(align-1). Returns -1 for
 * an invalid descriptor. Size src_row_d, x_perm, h and y with it. */
int64_t moe_layout_m_cap(const moe_layout_desc* desc);

/* Bytes of device workspace moe_layout needs (0 for an invalid descriptor). */
size_t moe_layout_workspace_bytes(const moe_layout_desc* desc);

/*
 * moe_layout -- dispatch layout from topk_idx, with no host sync.
 *
 * The layout is computed from topk_idx and the expert count before any data
 * moves (DeepEP issue #272, the maintainer's dispatch example:
 * get_dispatch_layout, then dispatch), its histogram must not force a host
 * sync (xtuner PR #2056, review comments: histc kept over bincount), and the
 * split plan comes from the per-expert count matrix alone, its row sums being
 * the splits (DeepSpeed PR #8190 "Derive AutoEP rank splits from the
 * per-expert count exchange", sections "Redundancy" and "Fix"). Rows are
 * grouped by local expert and each group is padded to `align` for the
 * grouped GEMM (DeepSpeed AutoEP commit text, section "Attribution": token
 * group alignment / padding helpers). Rows are named by the flat index
 * token*top_k + slot (DeepSpeed PR #8847, section "Change").
 *
 * Outputs (all int32, device):
 *   expert_counts_d [E]            assignments per expert (all E)
 *   send_counts_d   [ep, E]        [s, e]: assignments of source s to expert e
 *   split_matrix_d  [ep, ep]       [s, d]: assignments of source s to destination d
 *                                  (row sums: input splits; column local_rank: output splits)
 *   recv_counts_d   [ep, E_loc]    [s, e]: assignments of source s to local expert e
 *   output_splits_d [ep]           recv_counts row sums
 *   offsets_d       [E_loc + 1]    offsets[0] = 0, offsets[e+1] = offsets[e] + ceil(c_e/align)*align
 *   dst_row_d       [T, k]         local row of (t, slot), or -1 if its expert is not local
 *   src_row_d       [m_cap]        flat index t*k+slot held by a row; -1 for padding and
 *                                  for every row from offsets[E_loc] to m_cap
 * Within an expert's group, rows follow ascending flat index (a stable
 * order, independent of thread scheduling).
 *   topk_idx_d      [T, k] int32 expert ids; ids outside [0, E) are skipped.
 *   m_cap           >= moe_layout_m_cap(desc)
 *   workspace_d     >= moe_layout_workspace_bytes(desc) bytes, 16-byte aligned;
 *                   contents on entry do not matter.
 * Any output pointer except offsets_d, dst_row_d and src_row_d may be NULL
 * to skip it.
 */
int32_t moe_layout(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                   int32_t* expert_counts_d, int32_t* send_counts_d,
                   int32_t* split_matrix_d, int32_t* recv_counts_d,
                   int32_t* output_splits_d, int32_t* offsets_d, int32_t* dst_row_d,
                   int32_t* src_row_d, int64_t m_cap, void* workspace_d,
                   size_t workspace_bytes, void* stream);

/*
 * moe_layout_noalloc -- moe_layout for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument, and the call allocates nothing.
 * The workspace lives in a static device array of MOE_LAYOUT_SCRATCH_BYTES
 * (4 MiB) that each GPU the library runs on holds until the process ends;
 * its device address is looked up once per device, on the first call with
 * that device current. Outputs, arguments and results are those of
 * moe_layout (the same kernels), on the current device's stream `stream`.
 * Limit: moe_layout_workspace_bytes(desc) <= MOE_LAYOUT_SCRATCH_BYTES, else
 * MOE_ERR_TOO_LARGE and nothing is launched (the layout's tiles grow with the
 * assignment count, so every layout of up to 2^30 assignments T * top_k fits,
 * and every valid one with at most 512 experts). Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on two streams, or from two host threads
 * without ordering) race and must not be made. Nothing in the array needs to
 * start at zero; a call leaves its contents behind.
 */
#define MOE_LAYOUT_SCRATCH_BYTES (4u << 20)

int32_t moe_layout_noalloc(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                           int32_t* expert_counts_d, int32_t* send_counts_d,
                           int32_t* split_matrix_d, int32_t* recv_counts_d,
                           int32_t* output_splits_d, int32_t* offsets_d, int32_t* dst_row_d,
                           int32_t* src_row_d, int64_t m_cap, void* stream);

/*
 * moe_dispatch_layout -- per-rank deduplicated dispatch layout.
 *
 * The counts and table DeepEP's dispatch consumes, computed from topk_idx
 * and the expert count before any data moves (DeepEP issue #272, the
 * maintainer's example: get_dispatch_layout returns num_tokens_per_rank,
 * num_tokens_per_expert and is_token_in_rank). A token is sent once to each
 * rank that holds at least one of its experts (rank r holds experts
 * [r*E/ep, (r+1)*E/ep)), however many of its slots land there:
 *   is_token_in_rank_d      [T, ep] uint8: 1 if some slot of t maps to rank r
 *   num_tokens_per_rank_d   [ep] int32: column sums of is_token_in_rank
 *   num_tokens_per_expert_d [E] int32: assignments per expert
 *   token_rank_pos_d        [T, ep] int32: position of t among the tokens rank r
 *                           receives, in token order; -1 where t is not sent to r
 * Expert ids outside [0, E) are skipped. No host sync; the result does not
 * depend on scheduling.
 *   workspace_d >= moe_dispatch_layout_workspace_bytes(...) bytes.
 * Limits: 1 <= ep <= 64, E a multiple of ep, E <= 1024, 1 <= k <= min(E, 16),
 * T < 2^25.
 */
size_t moe_dispatch_layout_workspace_bytes(int64_t num_tokens, int32_t num_experts,
                                           int32_t top_k, int32_t ep_size);

int32_t moe_dispatch_layout(const int32_t* topk_idx_d, int64_t num_tokens, int32_t num_experts,
                            int32_t top_k, int32_t ep_size, int32_t* num_tokens_per_rank_d,
                            int32_t* num_tokens_per_expert_d, uint8_t* is_token_in_rank_d,
                            int32_t* token_rank_pos_d, void* workspace_d,
                            size_t workspace_bytes, void* stream);

/*
 * moe_permute -- expert-major token gather (the local part of dispatch).
 *
 * The reorder-by-expert step of the AutoEP flow (DeepSpeed AutoEP commit
 * text, section "Design", runtime step 3) and the local half of DeepEP's
 * dispatch (DeepEP issue #272: x, topk_idx, topk_weights in; rows grouped per
 * expert out). For every (t, slot) with dst_row[t, slot] = r >= 0:
 * x_perm[r, :] = x[t, :], a bit copy (each token row read once); every row r
 * below offsets[E_loc] with src_row[r] < 0 (the alignment padding of the
 * expert groups) is set to zero. Rows from offsets[E_loc] to m_cap are not
 * written.
 *   x_d         [T, H] bf16, 16-byte aligned
 *   dst_row_d   [T, k] int32 (from moe_layout); rows >= m_cap are skipped
 *   src_row_d   [m_cap] int32 (from moe_layout)
 *   offsets_d   [E_loc + 1] int32 (from moe_layout)
 *   x_perm_d    [m_cap, H] bf16 (out), 16-byte aligned
 * Limits: H a multiple of 8, 8 <= H <= 16384; 1 <= k <= 16;
 * 1 <= E_loc <= 1024. T = 0 writes only the padding rows.
 */
int32_t moe_permute(const void* x_d, int64_t num_tokens, int32_t hidden, int32_t top_k,
                    const int32_t* dst_row_d, const int32_t* src_row_d,
                    const int32_t* offsets_d, int32_t num_local_experts, int64_t m_cap,
                    void* x_perm_d, void* stream);

/*
 * moe_permute_weighted -- the permute with the routing score applied before
 * the experts (AutoEP's score_apply="pre", DeepSpeed PR #8847, section
 * "Change", which the fused restore refuses): x_perm[dst_row[t, s], :] =
 * bf16(topk_w[t, s] * x[t, :]), an fp32 product rounded once. The experts
 * then see scaled rows and the restore is a plain sum (moe_combine_rows with
 * no weights). x_d, dst_row_d, x_perm_d and the limits as moe_permute, plus
 * topk_w_d [T, k]; padding rows are not written.
 */
int32_t moe_permute_weighted(const void* x_d, int64_t num_tokens, int32_t hidden, int32_t top_k,
                             const int32_t* dst_row_d, const float* topk_w_d, int64_t m_cap,
                             void* x_perm_d, void* stream);

/*
 * moe_pack_weights -- one-time repack of expert matrices into the packed
 * layout the forward grouped GEMMs read (moe_grouped_gate_up, _gate_up_save,
 * _down, _swiglu). This is the load-time conversion into the grouped expert
 * layout the runtime expects (DeepSpeed AutoEP commit text, section "Design":
 * ep_repack.py), done once per weight set, outside the per-step path; the
 * layout itself is this library's. Expert weights arrive in math orientation
 * w[m, k, n] (gate/up [E, H, I], down [E, I, H]; k the reduction index, n the
 * output index, K = rows, N = cols). The packed matrix is output-major with
 * the N rows cut into blocks of R = 256 rows if N % 256 == 0, else 128, and
 * each block stored as K/64 consecutive [R][64] slices:
 *   wt[m*N*K + (n/R)*K*R + (k/64)*R*64 + (n%R)*64 + k%64] = w[m, k, n]
 * (a bf16 bit copy; wt has the element count of w).
 *   w_d  [num_mats, rows, cols] bf16;  wt_d (out), num_mats * rows * cols bf16
 * rows and cols multiples of 128, else MOE_ERR_UNSUPPORTED; w_d and wt_d
 * distinct (MOE_ERR_ARG otherwise).
 */
int32_t moe_pack_weights(const void* w_d, int64_t num_mats, int32_t rows, int32_t cols,
                         void* wt_d, void* stream);

/*
 * Grouped SwiGLU expert MLPs over ragged expert groups (local grouped expert
 * compute of the AutoEP flow, DeepSpeed AutoEP commit text, sections
 * "Attribution" (ep_experts.py, grouped-GEMM execution) and "Design",
 * runtime step 5; bf16 grouped GEMM as in DeepSpeed PR #8847, section
 * "Tests"). For local expert e the rows [offsets[e], offsets[e] + counts[e])
 * of the input go through expert e:
 *
 *   moe_grouped_gate_up:  h = silu(x_perm W1[e]) * (x_perm W3[e])   (fp32 math, bf16 out)
 *   moe_grouped_down:     y = h W2[e]                               (fp32 accumulate, bf16 out)
 *   moe_grouped_swiglu:   both, in that order, through the caller's h buffer
 *
 * silu(a) = a / (1 + e^-a). Products are bf16 x bf16 on the matrix cores,
 * accumulated in fp32, rounded to bf16 (nearest even) once at the end.
 * Rows outside every [offsets[e], offsets[e] + counts[e]) are neither read
 * nor written.
 *   x_perm_d   [m_cap, H] bf16          h_d [m_cap, I] bf16        y_d [m_cap, H] bf16
 *   offsets_d  [E_loc + 1] int32        counts_d [E_loc] int32 (local expert counts,
 *                                       = expert_counts_d + first local expert)
 *   w1t_d, w3t_d: W1, W3 packed by moe_pack_weights (rows H, cols I), E_loc * I * H bf16
 *   w2t_d: W2 packed by moe_pack_weights (rows I, cols H), E_loc * H * I bf16
 * Limits: H and I multiples of 128; E_loc <= 1024; offsets[E_loc] <= m_cap.
 * All bf16 pointers 16-byte aligned. Unsupported shapes: MOE_ERR_UNSUPPORTED.
 */
int32_t moe_grouped_gate_up(const void* x_perm_d, const int32_t* offsets_d,
                            const int32_t* counts_d, int32_t num_local_experts,
                            int64_t m_cap, int32_t hidden, int32_t inter,
                            const void* w1t_d, const void* w3t_d, void* h_d, void* stream);

/*
 * moe_grouped_gate_up_gather -- moe_grouped_gate_up with the permute fused
 * into its operand loads: the rows of local expert e are read straight from
 * the token rows, row r of the grouped layout being x[src_row[r] / top_k]
 * (the expert-major gather of the dispatch, DeepEP issue #272: rows grouped
 * per expert; DeepSpeed AutoEP commit text, section "Design", runtime steps
 * 3 and 5, reorder then grouped expert compute). h is then bit-identical to
 * moe_permute followed by moe_grouped_gate_up, and the expert-major copy of x
 * is never written.
 *   x_d        [T, H] bf16 token rows, 16-byte aligned
 *   src_row_d  [m_cap] int32, moe_layout's src_row
 *   h_d        [m_cap, I] bf16 (out); other arguments as moe_grouped_gate_up
 * Limits as moe_grouped_gate_up, 1 <= top_k <= 16, and (T + 1) * H * 2 < 2^32
 * (MOE_ERR_UNSUPPORTED otherwise).
 */
int32_t moe_grouped_gate_up_gather(const void* x_d, int64_t num_tokens, int32_t top_k,
                                   const int32_t* src_row_d, const int32_t* offsets_d,
                                   const int32_t* counts_d, int32_t num_local_experts,
                                   int64_t m_cap, int32_t hidden, int32_t inter,
                                   const void* w1t_d, const void* w3t_d, void* h_d,
                                   void* stream);

int32_t moe_grouped_down(const void* h_d, const int32_t* offsets_d, const int32_t* counts_d,
                         int32_t num_local_experts, int64_t m_cap, int32_t inter,
                         int32_t hidden, const void* w2t_d, void* y_d, void* stream);

int32_t moe_grouped_swiglu(const void* x_perm_d, const int32_t* offsets_d,
                           const int32_t* counts_d, int32_t num_local_experts,
                           int64_t m_cap, int32_t hidden, int32_t inter,
                           const void* w1t_d, const void* w3t_d, const void* w2t_d,
                           void* h_d, void* y_d, void* stream);

/*
 * Training: the forward keeps the pre-activations, and the backward of the
 * grouped SwiGLU experts produces the data gradient of x_perm. Training runs
 * the grouped-GEMM path forward and backward and hands the expert gradients
 * back in BF16 (xtuner PR #2056 "Integrate MoonEP dispatcher ...", section
 * "Summary"). With g = x W1[e], u = x W3[e] (fp32 accumulators), for the rows
 * [offsets[e], offsets[e] + counts[e]) of local expert e:
 *
 *   moe_grouped_gate_up_save:     h as moe_grouped_gate_up, and gu = [g | u] rounded to
 *                                 bf16 (the two halves of each gu row)
 *   moe_grouped_down_backward:    dh = dy W2[e]^T (fp32), then with g, u read from gu
 *                                 dgu = [dh u silu'(g) | dh silu(g)] rounded to bf16,
 *                                 silu'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g)
 *   moe_grouped_gate_up_backward: dx_perm = dg W1[e]^T + du W3[e]^T (one fp32 sum over
 *                                 the 2I products), rounded to bf16
 *
 *   x_perm_d, dy_d, dx_perm_d [m_cap, H] bf16;  h_d [m_cap, I];  gu_d, dgu_d [m_cap, 2I]
 *   w1t_d, w3t_d: W1, W3 packed by moe_pack_weights (forward only)
 *   w1_d, w3_d [E_loc, H, I], w2_d [E_loc, I, H]: the math-orientation weights, which
 *   are already output-major for the backward products
 * Rows outside the expert groups are neither read nor written. Limits as the
 * forward calls (H and I multiples of 128).
 */
int32_t moe_grouped_gate_up_save(const void* x_perm_d, const int32_t* offsets_d,
                                 const int32_t* counts_d, int32_t num_local_experts,
                                 int64_t m_cap, int32_t hidden, int32_t inter,
                                 const void* w1t_d, const void* w3t_d, void* h_d, void* gu_d,
                                 void* stream);

int32_t moe_grouped_down_backward(const void* dy_d, const void* gu_d, const int32_t* offsets_d,
                                  const int32_t* counts_d, int32_t num_local_experts,
                                  int64_t m_cap, int32_t inter, int32_t hidden,
                                  const void* w2_d, void* dgu_d, void* stream);

int32_t moe_grouped_gate_up_backward(const void* dgu_d, const int32_t* offsets_d,
                                     const int32_t* counts_d, int32_t num_local_experts,
                                     int64_t m_cap, int32_t hidden, int32_t inter,
                                     const void* w1_d, const void* w3_d, void* dx_perm_d,
                                     void* stream);

/*
 * Weight gradients of the grouped experts (BF16 out, fp32 accumulation over
 * the expert's rows; xtuner PR #2056, section "Summary", and its commit
 * "extend grouped GEMM for dynamic expert gradients"):
 *
 *   moe_grouped_gate_up_wgrad:  dW1[e] = x_perm_e^T dg_e,  dW3[e] = x_perm_e^T du_e
 *   moe_grouped_down_wgrad:     dW2[e] = h_e^T dy_e
 *
 * where _e is the expert's rows [offsets[e], offsets[e] + counts[e]) and
 * dgu = [dg | du] is moe_grouped_down_backward's output. An expert without
 * rows gets a zero gradient.
 *   dw1_d, dw3_d [E_loc, H, I] bf16 (out);  dw2_d [E_loc, I, H] bf16 (out)
 *   (the math orientation of the weights)
 * Limits as the forward calls.
 * When the experts' row counts are skewed (a fixed tile order would give some
 * workgroup 1/16 more work than the mean), tiles are handed out at run time
 * from a small counter pair in library-held device memory, one pair per
 * stream (the first 64 streams a GPU sees; later streams keep the fixed
 * order). Each tile is one workgroup's fixed-order sum either way, so the
 * result does not depend on the order. A launch leaves its pair at zero.
 * Calls on different streams may overlap. A captured graph holding one of
 * these calls uses the pair of the stream it was captured on: do not replay
 * it while other calls run on that stream.
 */
int32_t moe_grouped_gate_up_wgrad(const void* x_perm_d, const void* dgu_d,
                                  const int32_t* offsets_d, const int32_t* counts_d,
                                  int32_t num_local_experts, int64_t m_cap, int32_t hidden,
                                  int32_t inter, void* dw1_d, void* dw3_d, void* stream);

int32_t moe_grouped_down_wgrad(const void* h_d, const void* dy_d, const int32_t* offsets_d,
                               const int32_t* counts_d, int32_t num_local_experts,
                               int64_t m_cap, int32_t inter, int32_t hidden, void* dw2_d,
                               void* stream);

/*
 * moe_combine -- fused weighted-sum restore.
 *
 * The fused restore of DeepSpeed PR #8847 ("AutoEP: support
 * combine_impl=fused_weighted_sum ...", sections "Problem" and "Change"):
 * each row is addressed by the flat index token*top_k + slot, the routing
 * weights stay FP32 in a [tokens, top_k] layout, and weight x row products
 * are accumulated in FP32 (section "Benchmark": the error left is the bf16
 * output rounding). Per token t:
 *
 *   out[t, :] = bf16( sum over slots s = 0..k-1 with 0 <= dst_row[t, s] < y_rows
 *                     of topk_w[t, s] * y[dst_row[t, s], :] )
 *
 * summed in fp32 in slot order (each product rounded to fp32, then added:
 * no fused multiply-add), rounded once to bf16 (nearest even). A token with no local slot gets a zero row. The result
 * does not depend on where the rows sit in y.
 *   y_d       [y_rows, H] bf16, 16-byte aligned
 *   dst_row_d [T, k] int32;  topk_w_d [T, k] float
 *   out_d     [T, H] bf16 (out), 16-byte aligned
 * Limits: H a multiple of 8, 8 <= H <= 16384; 1 <= k <= 16.
 */
int32_t moe_combine(const void* y_d, int64_t y_rows, const int32_t* dst_row_d,
                    const float* topk_w_d, int64_t num_tokens, int32_t hidden,
                    int32_t top_k, void* out_d, void* stream);

/*
 * Backward of the combine, the permute and the routing weights.
 *
 * The fused restore back-propagates a row gradient and a score gradient, the
 * score (router) gradient in FP32 (DeepSpeed PR #8847, sections "Tests" and
 * "Benchmark"); the backward of a combine is a dispatch of the output
 * gradient and the backward of a dispatch is a combine (DeepEP issue #272,
 * the maintainer's answer). G is the gradient of the combine's output.
 *
 * moe_combine_backward: for every (t, s) with 0 <= r = dst_row[t, s] < y_rows
 *   grad_y[r, :]  = bf16(topk_w[t, s] * G[t, :])    (fp32 product, one rounding)
 *   grad_w[t, s]  = sum_h G[t, h] * y[r, h]          (fp32, tree-shaped sum)
 * and grad_w[t, s] = 0 for every other slot. Rows of grad_y that no slot
 * points at are not written.
 *   grad_out_d [T, H] bf16;  y_d [y_rows, H] bf16 (the forward's expert output)
 *   dst_row_d, topk_w_d [T, k] as in moe_combine
 *   grad_y_d   [y_rows, H] bf16 (out);  grad_w_d [T, k] float (out)
 * Limits as moe_combine; bf16 pointers 16-byte aligned.
 */
int32_t moe_combine_backward(const void* grad_out_d, const void* y_d, int64_t y_rows,
                             const int32_t* dst_row_d, const float* topk_w_d,
                             int64_t num_tokens, int32_t hidden, int32_t top_k,
                             void* grad_y_d, float* grad_w_d, void* stream);

/*
 * moe_permute_backward: grad_x[t, :] = bf16( sum over slots s with
 *   0 <= dst_row[t, s] < x_perm_rows of grad_x_perm[dst_row[t, s], :] ),
 * an fp32 sum in slot order rounded once (moe_combine with unit weights); a
 * token with no local slot gets a zero row.
 *   grad_x_perm_d [x_perm_rows, H] bf16;  grad_x_d [T, H] bf16 (out)
 * Limits as moe_combine.
 */
int32_t moe_permute_backward(const void* grad_x_perm_d, int64_t x_perm_rows,
                             const int32_t* dst_row_d, int64_t num_tokens, int32_t hidden,
                             int32_t top_k, void* grad_x_d, void* stream);

/*
 * moe_route_backward: the routing weights are the softmax of the k selected
 * logits (moe_route), so with g = grad_w[t, :] (the score gradient)
 *   grad_logits[t, topk_idx[t, j]] = topk_w[t, j] * (g_j - sum_i topk_w[t, i] * g_i)
 * (the sum in fp32, slot order) and 0 for every unselected expert.
 *   topk_idx_d, topk_w_d, grad_w_d [T, k];  grad_logits_d [T, E] float (out)
 * Limits as moe_route; T * E < 2^32 (else MOE_ERR_UNSUPPORTED).
 */
int32_t moe_route_backward(const int32_t* topk_idx_d, const float* topk_w_d,
                           const float* grad_w_d, int64_t num_tokens, int32_t num_experts,
                           int32_t top_k, float* grad_logits_d, void* stream);

/*
 * moe_combine_rows -- the fused restore on other row dtypes and variants.
 *
 * The fused restore runs on bf16 and on fp32 rows (DeepSpeed PR #8847,
 * section "Tests"); fp16 rows are the third activation dtype the page
 * discusses. Per token t:
 *
 *   out[t, :] = round( sum over local slots s, in slot order, of w[t, s] * y[dst_row[t, s], :]
 *                      + shared[t, :] )
 *
 * in fp32 (products, then sums, no fused multiply-add) and rounded once to the
 * row dtype (nearest even; fp32 rows are not rounded again). topk_w_d = NULL
 * gives w = 1, the plain sum used when the score was applied before the
 * experts (moe_permute_weighted). shared_d = NULL adds nothing; otherwise it
 * holds the output rows [T, H] of a shared expert, merged as the last step of
 * the AutoEP runtime (DeepSpeed AutoEP commit text, section "Design": merge
 * shared experts if the model has them). y_d, shared_d and out_d are all of
 * the row dtype; MOE_ROWS_BF16 with weights and no shared rows is moe_combine.
 * Limits as moe_combine.
 */
enum { MOE_ROWS_BF16 = 0, MOE_ROWS_F16 = 1, MOE_ROWS_F32 = 2 };

int32_t moe_combine_rows(const void* y_d, int32_t row_dtype, int64_t y_rows,
                         const int32_t* dst_row_d, const float* topk_w_d, const void* shared_d,
                         int64_t num_tokens, int32_t hidden, int32_t top_k, void* out_d,
                         void* stream);

/*
 * moe_validate_layout -- debug check of a layout (SYNCHRONISES the stream,
 * copies the buffers to the host and checks there). Mirrors the fused
 * restore's coverage check (DeepSpeed PR #8847, section "Change": a missing
 * (token, slot) raises instead of reading an unset row).
 * Returns MOE_OK, MOE_ERR_EXPERT_ID (id out of range or repeated in a token),
 * MOE_ERR_COVERAGE (a local (t, slot) without a row, or a row claimed twice) or
 * MOE_ERR_LAYOUT (offsets not aligned/monotone, src_row and dst_row not
 * inverse, padding or order wrong). `detail` (may be NULL) receives a
 * NUL-terminated message of at most detail_len bytes.
 */
int32_t moe_validate_layout(const moe_layout_desc* desc, const int32_t* topk_idx_d,
                            const int32_t* offsets_d, const int32_t* dst_row_d,
                            const int32_t* src_row_d, int64_t m_cap, void* stream,
                            char* detail, size_t detail_len);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
