"""Dispatch layout (oracle): per-expert histogram, split plan, alignment-padded
offsets and the stable expert-major permutation.

Passages followed:

* The layout is computed from ``topk_idx`` and the expert count before any
  data moves, and yields tokens per expert (DeepEP issue #272 "Does DeepEP's
  Dispatch/Combine Support Autograd ...", the maintainer's dispatch example:
  get_dispatch_layout before dispatch).
* The per-expert histogram must not need a host sync (xtuner PR #2056
  "Integrate MoonEP dispatcher ...", review comments: histc kept over
  bincount, which forces a host-device sync).
* Split plan (DeepSpeed PR #8190 "Derive AutoEP rank splits from the
  per-expert count exchange", sections "Redundancy" and "Fix"): a count
  matrix ``[ep_size, E_local]`` per destination rank and local expert; the
  matrix a rank receives, ``received_counts[s, e]`` = tokens source rank s
  sends to local expert e; ``input_splits`` = row sums of what a rank sends,
  ``output_splits = received_counts.sum(1)``.
* Rows are reordered by expert assignment and each expert's group is padded
  to the grouped-GEMM alignment (DeepSpeed AutoEP commit text, section
  "Attribution": TokenReorderer, generate_permute_indices, token-group
  alignment / padding helpers; section "Design", runtime step 3).
* A row is addressed by the flat index ``token * top_k + slot`` (DeepSpeed PR
  #8847 "AutoEP: support combine_impl=fused_weighted_sum ...", section
  "Change").

Readings where the pages are silent (one GPU stands for ``ep_size`` virtual
ranks): source rank s owns the contiguous tokens ``[s*T/ep, (s+1)*T/ep)``;
destination rank d owns the contiguous experts ``[d*E_loc, (d+1)*E_loc)``;
``local_rank = -1`` means all E experts are local. Local rows are ordered by
(local expert, flat index); an expert with c rows occupies ``ceil(c/A)*A``
rows (0 when c = 0); padding rows and the tail up to ``m_cap`` carry
``src_row = -1``; an assignment to a non-local expert has ``dst_row = -1``.
"""
from __future__ import annotations

import numpy as np


def local_range(num_experts: int, ep_size: int, local_rank: int):
    if local_rank < 0:
        return 0, num_experts
    el = num_experts // ep_size
    return local_rank * el, el


def m_cap_bound(num_tokens: int, num_experts: int, top_k: int, ep_size: int,
                local_rank: int, align: int) -> int:
    """Worst-case local rows: every token sends min(k, E_loc) distinct local
    assignments and every local expert pads by at most align - 1 rows."""
    _, el = local_range(num_experts, ep_size, local_rank)
    return num_tokens * min(top_k, el) + el * (align - 1)


def layout(topk_idx, num_experts: int, ep_size: int = 1, local_rank: int = -1,
           align: int = 128, m_cap: int | None = None) -> dict:
    """All layout outputs for one GPU share, as int32 numpy arrays.

    send_counts   [ep, E]      rows source rank s sends to expert e
    expert_counts [E]          column sums of send_counts
    split_matrix  [ep, ep]     [s, d]: rows source s sends to destination d
    recv_counts   [ep, E_loc]  [s, e]: rows source s sends to local expert e
    input_splits  [ep]         row sums of split_matrix (what each source sends)
    output_splits [ep]         recv_counts.sum(1) (what this share receives)
    offsets       [E_loc + 1]  padded exclusive prefix of local expert counts
    dst_row       [T, k]       local row of (t, slot), -1 if not local
    src_row       [m_cap]      flat index t*k+slot of a local row, -1 if padding
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    E = int(num_experts)
    if T % ep_size or E % ep_size:
        raise ValueError("T and E must be multiples of ep_size")
    first, el = local_range(E, ep_size, local_rank)
    if m_cap is None:
        m_cap = m_cap_bound(T, E, k, ep_size, local_rank, align)

    # histogram per (source rank, expert): bincount of a combined key
    src_rank = np.repeat(np.arange(T) // (T // ep_size), k)
    flat = idx.reshape(-1)
    send_counts = np.bincount(src_rank * E + flat, minlength=ep_size * E).reshape(ep_size, E)
    expert_counts = send_counts.sum(axis=0)

    # split plan: destination d holds experts [d*E/ep, (d+1)*E/ep)
    split_matrix = send_counts.reshape(ep_size, ep_size, E // ep_size).sum(axis=2)
    recv_counts = send_counts[:, first:first + el]
    input_splits = split_matrix.sum(axis=1)
    output_splits = recv_counts.sum(axis=1)

    # padded offsets over local experts
    counts = recv_counts.sum(axis=0)
    padded = (counts + align - 1) // align * align
    offsets = np.concatenate([[0], np.cumsum(padded)])
    if offsets[-1] > m_cap:
        raise ValueError(f"m_cap {m_cap} below the {offsets[-1]} rows this routing needs")

    # stable permutation: sort local assignments by (local expert, flat index)
    is_local = (flat >= first) & (flat < first + el)
    key = np.where(is_local, flat - first, el)
    order = np.argsort(key, kind="stable")
    src_row = np.full(m_cap, -1, dtype=np.int64)
    pos = 0
    for e in range(el):
        c = int(counts[e])
        src_row[offsets[e]:offsets[e] + c] = order[pos:pos + c]
        pos += c
    dst_row = np.full(T * k, -1, dtype=np.int64)
    rows = np.nonzero(src_row >= 0)[0]
    dst_row[src_row[rows]] = rows

    i32 = lambda a: np.ascontiguousarray(a).astype(np.int32)  # noqa: E731
    return {
        "send_counts": i32(send_counts),
        "expert_counts": i32(expert_counts),
        "split_matrix": i32(split_matrix),
        "recv_counts": i32(recv_counts),
        "input_splits": i32(input_splits),
        "output_splits": i32(output_splits),
        "local_counts": i32(counts),
        "offsets": i32(offsets),
        "dst_row": i32(dst_row.reshape(T, k)),
        "src_row": i32(src_row),
        "first_local": first,
        "num_local": el,
        "m_cap": int(m_cap),
    }


def dispatch_layout(topk_idx, num_experts: int, ep_size: int) -> dict:
    """Per-token, per-destination-rank layout of a deduplicated dispatch, as
    int32 / uint8 numpy arrays.

    DeepEP computes, before dispatching, the tokens per rank, tokens per
    expert and a token-in-rank table from ``topk_idx`` and the expert count
    (DeepEP issue #272, the maintainer's example: get_dispatch_layout returns
    num_tokens_per_rank, num_tokens_per_expert and is_token_in_rank, which
    the dispatch then consumes). The pages print only the names; the reading
    taken is the plain one: a token is sent once to each rank that holds at
    least one of its experts, whatever the number of its slots there.

    is_token_in_rank     [T, ep] uint8   1 if some slot of t maps to an expert of rank r
    num_tokens_per_rank  [ep]            column sums of is_token_in_rank
    num_tokens_per_expert[E]             assignments per expert (ids outside [0, E) skipped)
    token_rank_pos       [T, ep]         position of t among the tokens rank r receives,
                                         in token order; -1 where t is not sent to r

    Rank r holds the experts [r*E/ep, (r+1)*E/ep) (one GPU standing for ep
    virtual ranks, as in ``layout``)."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    el = num_experts // ep_size
    valid = (idx >= 0) & (idx < num_experts)
    in_rank = np.zeros((T, ep_size), dtype=bool)
    for s in range(k):
        m = valid[:, s]
        in_rank[np.nonzero(m)[0], idx[m, s] // el] = True
    per_rank = in_rank.sum(axis=0)
    per_expert = np.bincount(idx[valid], minlength=num_experts)
    pos = np.where(in_rank, np.cumsum(in_rank, axis=0) - 1, -1)
    return {
        "is_token_in_rank": in_rank.astype(np.uint8),
        "num_tokens_per_rank": per_rank.astype(np.int32),
        "num_tokens_per_expert": per_expert.astype(np.int32),
        "token_rank_pos": pos.astype(np.int32),
    }
