"""Parallel evaluation of independent oracle units.  Test infrastructure only.

The oracle's definitions are evaluated one (sequence, head, block of rows) or
one query row at a time; those units share no state and write disjoint parts
of the output, so they may run on several host threads.  NumPy's matrix
products and ufuncs release the interpreter lock, so a thread pool spreads the
work over the host's cores; the BLAS library is limited to one thread per
worker meanwhile, so the workers do not oversubscribe the cores.  The order
units run in never changes a value: each unit's arithmetic is the same
sequence of operations whichever thread runs it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

__all__ = ["host_cores", "run_units"]


def host_cores() -> int:
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:          # not Linux
        return os.cpu_count() or 1


def run_units(fn, units, workers: int = 1):
    """Call fn(u) for every unit u, on ``workers`` threads (1: in order, here)."""
    units = list(units)
    if workers <= 1 or len(units) <= 1:
        for u in units:
            fn(u)
        return
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=min(workers, len(units))) as ex:
            for f in [ex.submit(fn, u) for u in units]:
                f.result()          # re-raise any worker's exception
