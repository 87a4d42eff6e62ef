"""Invariant checks on routing and layout results (oracle side).

Each function raises AssertionError (or RuntimeError for coverage, as the
fused restore does) naming the first violation. They state what the pages
fix about the layout, independently of how it was computed:

* split projection: ``received_counts.sum(dim=1)[s] == output_splits[s]``
  exactly (DeepSpeed PR #8190 "Derive AutoEP rank splits ...", section
  "Redundancy");
* every (token, slot) is covered exactly once (DeepSpeed PR #8847 "AutoEP:
  support combine_impl=fused_weighted_sum ...", section "Change");
* distinct experts per token (same page, section "Benchmark").
"""
from __future__ import annotations

import numpy as np


def check_route(logits, topk_idx, topk_w, atol=1e-6):
    logits = np.asarray(logits, dtype=np.float32)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, E = logits.shape
    k = idx.shape[1]
    assert ((idx >= 0) & (idx < E)).all(), "expert id out of range"
    srt = np.sort(idx, axis=1)
    assert (np.diff(srt, axis=1) > 0).all(), "a token repeats an expert"
    sel = np.take_along_axis(logits, idx, axis=1)
    mask = np.ones((T, E), dtype=bool)
    np.put_along_axis(mask, idx, False, axis=1)
    rest = np.where(mask, logits, -np.inf).max(axis=1) if k < E else np.full(T, -np.inf)
    assert (sel.min(axis=1) >= rest).all(), "an unselected logit beats a selected one"
    assert (np.diff(sel, axis=1) <= 0).all(), "slots not in descending logit order"
    assert np.allclose(w.sum(axis=1), 1.0, atol=atol, rtol=0), "weights do not sum to one"
    assert (np.diff(w, axis=1) <= atol).all(), "weights increase along k"


def check_layout(topk_idx, L: dict, num_experts: int, ep_size: int, local_rank: int,
                 align: int):
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    first, el = L["first_local"], L["num_local"]
    sc, ec = L["send_counts"].astype(np.int64), L["expert_counts"].astype(np.int64)
    assert ec.sum() == T * k, "expert counts do not sum to T*k"
    assert (sc.sum(axis=0) == ec).all()
    assert (L["split_matrix"].sum(axis=1) == L["input_splits"]).all()
    assert (L["recv_counts"].sum(axis=1) == L["output_splits"]).all(), "split projection broken"
    if local_rank >= 0:
        assert (L["split_matrix"][:, local_rank] == L["output_splits"]).all()
    else:
        assert (L["output_splits"] == L["input_splits"]).all()
    for s in range(ep_size):
        assert sc[s].sum() == (T // ep_size) * k, "a source rank does not send all its rows"
    off = L["offsets"].astype(np.int64)
    assert off[0] == 0 and (off % align == 0).all() and (np.diff(off) >= 0).all()
    assert off[-1] <= L["m_cap"]
    cnt = L["local_counts"].astype(np.int64)
    assert (np.diff(off) == (cnt + align - 1) // align * align).all()
    src, dst = L["src_row"].astype(np.int64), L["dst_row"].astype(np.int64)
    flat = idx.reshape(-1)
    local = (flat >= first) & (flat < first + el)
    d = dst.reshape(-1)
    assert ((d >= 0) == local).all(), "dst_row sign disagrees with locality"
    assert (src[d[local]] == np.nonzero(local)[0]).all(), "src_row is not dst_row's inverse"
    rows = np.nonzero(src >= 0)[0]
    assert (d[src[rows]] == rows).all(), "dst_row is not src_row's inverse"
    for e in range(el):
        seg = src[off[e]:off[e + 1]]
        c = int(cnt[e])
        assert (seg[:c] >= 0).all() and (seg[c:] == -1).all(), "padding misplaced"
        assert (np.diff(seg[:c]) > 0).all(), "segment not in flat-index order (unstable)"
        assert (flat[seg[:c]] == first + e).all(), "row in the wrong expert segment"
    assert (src[off[-1]:] == -1).all(), "tail rows not marked -1"


def check_coverage(dst_rows, num_tokens: int, top_k: int):
    """Every (token, slot) is covered by exactly one share's dst_row."""
    hits = np.zeros((num_tokens, top_k), dtype=np.int64)
    for d in dst_rows:
        hits += np.asarray(d) >= 0
    if (hits != 1).any():
        t, s = np.argwhere(hits != 1)[0]
        raise RuntimeError(f"(token {t}, slot {s}) covered {hits[t, s]} times")
