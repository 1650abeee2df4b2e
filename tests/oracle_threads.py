"""Row-parallel oracle calls for full-size checks (test helper).

The oracle's row epilogues treat rows independently, so a [rows, D] problem
splits into row blocks that a thread pool runs at once (each oracle call is
one C call through ctypes, which releases the GIL); the blocks partition the
output, so the result is the single-threaded one.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def threads():
    n = int(os.environ.get("OMP_NUM_THREADS", "16"))
    return max(1, min(16, n, len(os.sched_getaffinity(0))))


def by_rows(fn, rows, blocks=64):
    """np.concatenate([fn(a, b) for row blocks [a, b)]) on a thread pool."""
    step = max(1, -(-rows // blocks))
    cuts = [(a, min(a + step, rows)) for a in range(0, rows, step)]
    with ThreadPoolExecutor(threads()) as pool:
        parts = list(pool.map(lambda c: fn(*c), cuts))
    return np.concatenate(parts, axis=0)
