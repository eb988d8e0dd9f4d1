"""Deterministic top-k index selection oracle.  Test infrastructure only.

Source: 「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」, sections
修改topk结果，输出后排序 and 用 torch.sort 替换 topk，输出对比: the indexer
picks the 2048 highest-scoring positions of each row of logits [323, 2590]; an
unstable top-k resolves equal scores at the edge of the selection either way,
so two identical requests selected index sets that differed by one, and the
fix was a stable sort.  The tie rule (equal keys go by their id, never by
where they happen to sit in memory) follows 「AMD MI250部署DeepSeek-V4-Flash：
先修正确性再谈性能」 section 4.2.

Definition, per row r with valid positions V_r = [start_r, start_r + len_r)
of the n columns (start 0 and len n when not given):

    position i ranks before position j  iff  x_i > x_j,
                                         or  x_i == x_j and i < j
    (a NaN ranks after every number; NaNs among themselves by position;
     -0.0 == +0.0, so they tie)

    out[r, t] = the position of rank t in V_r for t < min(k, len_r),
                -1 for t >= len_r.

The positions are absolute column indices of the row.  The result is unique:
the rank order is a strict total order on V_r.
"""
from __future__ import annotations

import numpy as np

__all__ = ["topk_indices"]


def topk_indices(logits, k: int, row_starts=None, row_lens=None):
    """logits [R, n] float32 (or float64 holding float32 values); k >= 1.

    row_starts, row_lens: optional int arrays [R] (defaults 0 and n); each
    row's valid span must lie within [0, n).  Returns int32 [R, k].
    """
    x = np.asarray(logits, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("logits must be [rows, n]")
    rows, n = x.shape
    if k < 1:
        raise ValueError("k must be >= 1")
    starts = np.zeros(rows, np.int64) if row_starts is None else np.asarray(row_starts, np.int64)
    lens = np.full(rows, n, np.int64) if row_lens is None else np.asarray(row_lens, np.int64)
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        s, ln = int(starts[r]), int(lens[r])
        if s < 0 or ln < 0 or s + ln > n:
            raise ValueError("row %d: span [%d, %d) outside [0, %d)" % (r, s, s + ln, n))
        if ln == 0:
            continue
        seg = x[r, s:s + ln] + 0.0                       # -0.0 becomes +0.0: they tie
        # Sort key: numbers by descending value, then NaNs; equal keys keep
        # their position order (a stable sort), i.e. ties go to the lower index.
        nan = np.isnan(seg)
        key = np.where(nan, 0.0, -seg)
        order = np.lexsort((np.arange(ln), key, nan))    # last key is primary
        m = min(k, ln)
        out[r, :m] = (order[:m] + s).astype(np.int32)
    return out
