"""Running the oracle over independent ranges of a workload on several host
threads (test infrastructure).  Every step of the path works on independent
quantization blocks (the reorder moves whole slices), so a whole-output
comparison splits into ranges; the oracle's functions are ctypes calls, which
release the interpreter lock, so the ranges run in parallel.  Slicing and
dispatch only: no arithmetic of the method here."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


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


def slice_source(L, N):
    """Slice carried by each send position, from the oracle's reorder."""
    return oracle.reorder(np.arange(L * N, dtype=np.int64), L, N)


def oracle_send(g, dtype, L, N, B):
    """The oracle's reorder + INT4 quantization of the whole gradient, one
    send position per task: position p carries slice src[p], quantized on
    its own (its blocks do not depend on any other slice)."""
    W = L * N
    S = g.size // W
    src = slice_source(L, N)
    parts = pmap(lambda p: oracle.qgz_reorder_quant_i4(g[src[p] * S:(src[p] + 1) * S], dtype,
                                                       1, 1, B), range(W))
    return np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts])


def oracle_receive(codes, scales, K, chunk, B, ranges, out_dtype=None, divisor=1.0):
    """The oracle's hop-receive step over K source-major chunks, in `ranges`
    pieces of the chunk (whole blocks each); returns the concatenation."""
    R = chunk // ranges
    assert R * ranges == chunk and R % B == 0

    def one(r):
        lo, hi = r * R, (r + 1) * R
        ic = source_ranges(codes, K, chunk // 2, lo // 2, hi // 2)
        isc = source_ranges(scales, K, chunk // B, lo // B, hi // B)
        return oracle.qgz_dequant_reduce_requant_i4(ic, isc, K, R, B, out_dtype, divisor)
    parts = pmap(one, range(ranges))
    if out_dtype is None:
        return np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts])
    return np.concatenate(parts)
