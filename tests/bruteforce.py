"""Sort-based brute force for tiny inputs (pure Python; T*K up to a few hundred).

A different method from the oracle's cursor pass: every valid (expert, token,
k) triple is listed, the list is sorted by that key, and rows are handed out
group by group. Used only as a pin of the oracle.
"""
from __future__ import annotations

import numpy as np


def layout(idx, E: int, R: int, A: int):
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    L = E // R
    triples = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K)
                     if 0 <= idx[t, k] < E)
    groups = {e: [] for e in range(E)}
    for e, t, k in triples:
        groups[e].append((t, k))
    count = [len(groups[e]) for e in range(E)]
    offset = [0]
    for e in range(E):
        offset.append(offset[-1] + -(-count[e] // A) * A)
    slot = [[-1] * K for _ in range(T)]
    row_src = [-1] * offset[E]
    for e in range(E):
        for j, (t, k) in enumerate(groups[e]):
            slot[t][k] = offset[e] + j
            row_src[offset[e] + j] = t * K + k
    hits = {(t, e // L) for e, t, k in triples}
    in_rank = [[1 if (t, r) in hits else 0 for r in range(R)] for t in range(T)]
    rtc = [sum(in_rank[t][r] for t in range(T)) for r in range(R)]
    bad = any(not (-1 <= idx[t, k] < E) for t in range(T) for k in range(K))
    return dict(count=count, offset=offset, slot=slot, row_src=row_src,
                is_token_in_rank=in_rank, rank_token_count=rtc, bad=bad)


def ll_layout(idx, E: int, R: int, M: int, s: int):
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    triples = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K)
                     if 0 <= idx[t, k] < E)
    groups = {e: [] for e in range(E)}
    for e, t, k in triples:
        groups[e].append((t, k))
    slot = [[-1] * K for _ in range(T)]
    row_src = [-1] * (E * M)
    overflow = False
    for e in range(E):
        for j, (t, k) in enumerate(groups[e]):
            if j >= M:
                overflow = True
                continue
            slot[t][k] = e * R * M + s * M + j
            row_src[e * M + j] = t * K + k
    recv_count = [min(len(groups[e]), M) for e in range(E)]
    return dict(slot=slot, row_src=row_src, recv_count=recv_count, overflow=overflow)


def dense_combine(y_f32: np.ndarray, slot: np.ndarray, w) -> np.ndarray:
    """Combine written as one matrix product: out = W @ Y with W[t, row] the
    summed weight of token t's pairs on that row (float64)."""
    T, K = slot.shape
    rows = y_f32.shape[0]
    W = np.zeros((T, rows), np.float64)
    for t in range(T):
        for k in range(K):
            r = int(slot[t, k])
            if r >= 0:
                W[t, r] += 1.0 if w is None else float(w[t, k])
    return W @ y_f32.astype(np.float64)


def rank_layout(idx, E: int, R: int, A: int, w=None):
    """Normal-mode layout by sorting: the distinct (rank, token) keys of the
    valid pairs, sorted, take consecutive rows; per row the rank-local ids."""
    idx = np.asarray(idx)
    T, K = idx.shape
    L = E // R
    keys = sorted({(int(e) // L, t) for t in range(T) for e in idx[t] if 0 <= e < E})
    rank_slot = -np.ones((T, R), np.int64)
    recv_src, recv_idx, recv_w = [], [], []
    for row, (r, t) in enumerate(keys):
        rank_slot[t, r] = row
        recv_src.append(t)
        recv_idx.append([int(e) - r * L if 0 <= e < E and int(e) // L == r else -1
                         for e in idx[t]])
        if w is not None:
            recv_w.append([float(w[t, k]) if 0 <= idx[t, k] < E and int(idx[t, k]) // L == r
                           else 0.0 for k in range(K)])
    counts = np.array([sum(1 for (r, _) in keys if r == q) for q in range(R)], np.int64)
    rank_offset = np.concatenate([[0], np.cumsum(counts)])
    ids = idx[(idx >= 0) & (idx < E)]
    cnt = np.bincount(ids, minlength=E)
    return dict(rank_slot=rank_slot, rank_offset=rank_offset, recv_src=np.array(recv_src),
                recv_topk_idx=np.array(recv_idx, np.int64).reshape(-1, K),
                recv_topk_weights=np.array(recv_w, np.float32).reshape(-1, K)
                if w is not None else None,
                recv_expert_count=(cnt + A - 1) // A * A)
