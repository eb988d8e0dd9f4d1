"""Top-k sparse multi-query attention oracle (float64).  Test infrastructure only.

Source: the decoder's sparse attention takes Q, the KV cache and an index; the
KV rows it attends to are fetched through a page table ([V32] section
实验方法和结果).  Every query head of a row shares the same latent KV rows
(multi-query).  The result depends on the index *set* only; the order of the
indices is a rounding effect of the blockwise merge, not part of the
definition ([V32] sections 实验方法和结果, 结论 and 进一步探索 eq. (1)(2)).

For row r, head h, over the multiset J_r = {idx[r, t] : idx[r, t] >= 0}:

    s_j = scale * q[r,h,:] . kv[j, :]            (all d_qk columns)
    o   = sum_{j in J_r} softmax(s)_j * kv[j, :d_v]  (V = first d_v columns)
    lse = max_j s_j + ln sum_j exp(s_j - max)

Negative entries are padding and are skipped; a repeated index counts with its
multiplicity; an empty set gives o = 0, lse = -inf.
"""
from __future__ import annotations

import numpy as np

from oracle.paging import paged_rows
from oracle.pool import run_units

__all__ = ["sparse_mqa", "sparse_mqa_paged"]


def sparse_mqa(q, kv_latent, topk_idx, d_v: int, scale: float, rows=None, workers: int = 1):
    """q [R, H, d_qk], kv_latent [n_kv, d_qk], topk_idx int [R, k].

    rows: optional subset of query rows to evaluate (others NaN).
    workers: host threads evaluating query rows (each row is independent).
    Returns out [R, H, d_v] float64 and lse [H, R] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv_latent, dtype=np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    n_rows, heads, d_qk = q.shape
    if kv.shape[1] != d_qk or not (0 < d_v <= d_qk):
        raise ValueError("bad latent dims")
    if idx.size and idx.max() >= kv.shape[0]:
        raise ValueError("index out of range")
    row_list = range(n_rows) if rows is None else sorted(set(int(r) for r in rows))
    fill = 0.0 if rows is None else np.nan
    out = np.full((n_rows, heads, d_v), fill)
    lse = np.full((heads, n_rows), fill)

    def row(r):
        sel = idx[r][idx[r] >= 0]
        if sel.size == 0:
            out[r] = 0.0
            lse[:, r] = -np.inf
            return
        kr = kv[sel]                                  # gathered rows [n, d_qk]
        logits = float(scale) * (q[r] @ kr.T)         # [H, n]
        m = logits.max(axis=1)
        e = np.exp(logits - m[:, None])
        l_sum = e.sum(axis=1)
        out[r] = (e @ kr[:, :d_v]) / l_sum[:, None]
        lse[:, r] = m + np.log(l_sum)

    run_units(row, row_list, workers)
    return out, lse


def sparse_mqa_paged(q, kv_cache, page_table, page_size: int, n_logical: int, topk_idx, d_v: int, scale: float,
                     rows=None):
    """sparse_mqa over the logical KV view of a paged cache: kv_cache holds
    physical rows [n_pages * page_size, d_qk]; indices are logical positions
    in [0, n_logical)."""
    kv = np.asarray(kv_cache)
    logical = kv[paged_rows(page_table, page_size, n_logical)]
    return sparse_mqa(q, logical, topk_idx, d_v, scale, rows=rows)
