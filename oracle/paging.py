"""Paged KV cache addressing.  Test infrastructure only.

Source: the sparse attention of 「推理引擎的“蝴蝶效应” -- 从V32 模型的输出不一致说起」
fetches its KV rows through a page table (section 实验方法和结果,
pagetable_1), and the prefill path of 「从 SGLang Kernel源码到 GPU Trace：
DeepSeek V4.1 Flash - Prefill」 keeps its KV in a paged cache of fixed-size
pages (section 2.2).  Logical position j of a sequence lives in its page
j // page_size at offset j % page_size; that page is physical page
table[j // page_size].
"""
from __future__ import annotations

import numpy as np

__all__ = ["paged_rows"]


def paged_rows(page_table, page_size: int, n_logical: int):
    """Physical cache row of each logical position 0 .. n_logical-1:
    page_table[j // page_size] * page_size + j % page_size."""
    pt = np.asarray(page_table, dtype=np.int64)
    j = np.arange(n_logical, dtype=np.int64)
    return pt[j // page_size] * page_size + j % page_size
