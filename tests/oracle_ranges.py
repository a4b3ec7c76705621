"""Running the oracle over independent ranges of a workload on several host
threads (test infrastructure).  Every step of the path works on independent
quantization blocks (the reorder moves whole slices), so a whole-output
comparison splits into ranges; the oracle's functions are ctypes calls, which
release the interpreter lock, so the ranges run in parallel.  Slicing and
dispatch only: no arithmetic of the method here."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def workers():
    env = os.environ.get("ZPQ_TEST_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    """[fn(i) for i in items], on a thread pool, in order."""
    with ThreadPoolExecutor(workers()) as ex:
        return list(ex.map(fn, items))


def source_ranges(flat, n_src, per_src, lo, hi):
    """Elements [lo, hi) of each of n_src equal sources laid out source-major
    in `flat` (per_src elements each), concatenated in source order."""
    return np.concatenate([flat[i * per_src + lo:i * per_src + hi] for i in range(n_src)])
