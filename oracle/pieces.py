"""Query-piece arithmetic of the vision encoder.  Test infrastructure only.

[3090] section 三: attention is computed qb query rows at a time; the S and P
buffers hold one piece (qb x N floats) and are reused piece after piece.  With
a buffer of about 12.497 million floats, N <= 3535 fits in one piece, while
N = 8547 gives qb = 1462 and 6 pieces.

The piece row count for a buffer of ``cap`` floats is floor(cap / N); the
pieces are [p*qb, min((p+1)*qb, N)) for p = 0 .. ceil(N/qb) - 1.
"""
from __future__ import annotations

from typing import List, Tuple

__all__ = ["piece_rows_for_capacity", "piece_ranges"]


def piece_rows_for_capacity(cap_floats: int, n: int) -> int:
    """Rows per piece when a qb x N float buffer must fit in ``cap_floats``."""
    if n <= 0:
        raise ValueError("n must be positive")
    return min(n, cap_floats // n)


def piece_ranges(n: int, qb: int) -> List[Tuple[int, int]]:
    """[start, end) row range of every piece of an n-row sequence (qb <= 0: one piece)."""
    if n <= 0:
        return []
    if qb <= 0 or qb >= n:
        return [(0, n)]
    return [(p, min(p + qb, n)) for p in range(0, n, qb)]
