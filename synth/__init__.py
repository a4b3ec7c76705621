"""Seeded synthetic inputs shared by the tests and the benchmark.

This module holds no quantization arithmetic: only the random generator
(synth.c, SplitMix64 counters + Box-Muller) and the recipes of the workloads.
Every value is a pure function of (seed, stream, element index).  Values are
drawn in double, rounded to fp32, then rounded to fp16 / bf16 by torch's CPU
conversion (round to nearest even).

Workloads (each stands in for GPT-style weight or gradient tensors; the
ZeRO++ pages train GPT models of 18B-138B parameters and publish no tensors):

  qwz_roundtrip  fp16 [2^20] ~ N(0, 0.02); 1049 seeded positions (0.1%)
                 replaced by N(0, 1) outliers; block 2048 of the 4096 blocks of
                 256 set to +0.
  qwz_layer      one GPT layer at hidden 8192, fp16, flattened in the order
                 QKV [8192x24576], out-proj [8192x8192], FFN-up [8192x32768],
                 FFN-down [32768x8192] (12*8192^2 = 805,306,368 elements),
                 all ~ N(0, 0.02); the rank-0 shard is the first 1/16.
  qgz_hop1       bf16 gradient [2^28]: per block of 128, x = 1e-3*sqrt(v)*z with
                 v = 10^U(-2, 2) (log-uniform in [1e-2, 1e2]).
  qgz_hop2       16 fp32 gradient slices [2^24] ~ N(0, 1e-3).
  qgz_fused      fp16 gradient of FFN [12288x49152] then QKV [12288x36864]
                 (1,056,964,608 elements), x = 1e-3*t_3; of its blocks of 64,
                 1% hold one constant 1e-3*t_3 value and 0.5% are all zero
                 (disjoint, seeded).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

SEEDS = {"qwz_roundtrip": 1, "qwz_layer": 2, "qgz_hop1": 3, "qgz_hop2": 4, "qgz_fused": 5}

QWZ_LAYER_SHAPES = [(8192, 24576), (8192, 8192), (8192, 32768), (32768, 8192)]
QGZ_FUSED_SHAPES = [(12288, 49152), (12288, 36864)]

CHUNK = 1 << 26


def threads():
    env = os.environ.get("ZPQ_SYNTH_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64, i64, d, vp, ci = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                               ctypes.c_void_p, ctypes.c_int)
        L.synth_normal.argtypes = [u64, u64, i64, i64, d, d, vp, ci]
        L.synth_student_t3.argtypes = [u64, u64, i64, i64, d, vp, ci]
        L.synth_blockvar_normal.argtypes = [u64, u64, i64, i64, i64, d, d, d, vp, ci]
        L.synth_u64.argtypes = [u64, u64, i64, i64, vp, ci]
        L.synth_uniform.argtypes = [u64, u64, i64, i64, vp, ci]
        for f in (L.synth_normal, L.synth_student_t3, L.synth_blockvar_normal,
                  L.synth_u64, L.synth_uniform):
            f.restype = None
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- raw distributions (fp32) ------------------------------------------------

def normal(seed, stream, n, mean, std, offset=0):
    out = np.empty(n, np.float32)
    lib().synth_normal(seed, stream, offset, n, mean, std, _p(out), threads())
    return out


def student_t3(seed, stream, n, scale, offset=0):
    out = np.empty(n, np.float32)
    lib().synth_student_t3(seed, stream, offset, n, scale, _p(out), threads())
    return out


def blockvar_normal(seed, stream, n, block, base, log10_lo, log10_hi, offset=0):
    out = np.empty(n, np.float32)
    lib().synth_blockvar_normal(seed, stream, offset, n, block, base, log10_lo, log10_hi,
                                _p(out), threads())
    return out


def u64(seed, stream, n, offset=0):
    out = np.empty(n, np.uint64)
    lib().synth_u64(seed, stream, offset, n, _p(out), threads())
    return out


def uniform(seed, stream, n, offset=0):
    out = np.empty(n, np.float64)
    lib().synth_uniform(seed, stream, offset, n, _p(out), threads())
    return out


def select(seed, stream, population, k, offset=0):
    """k distinct indices of range(population): those with the smallest keys,
    returned sorted."""
    keys = u64(seed, stream, population, offset)
    idx = np.argpartition(keys, k - 1)[:k] if k < population else np.arange(population)
    return np.sort(idx)


# ---- conversions to the 16-bit storage types ---------------------------------

def to_f16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float16).numpy()


def to_bf16_bits(x):
    """bf16 as raw uint16 bit patterns (numpy has no bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _chunked(n, gen, conv, out_dtype):
    out = np.empty(n, out_dtype)
    for o in range(0, n, CHUNK):
        m = min(CHUNK, n - o)
        out[o:o + m] = conv(gen(o, m))
    return out


# ---- workloads ---------------------------------------------------------------

QWZ_ROUNDTRIP = dict(n=1 << 20, block=256, outliers=1049, zero_block=2048)


def qwz_roundtrip():
    """fp16 [2^20]: N(0, 0.02), 1049 N(0, 1) outliers, one all-zero block."""
    c = QWZ_ROUNDTRIP
    s = SEEDS["qwz_roundtrip"]
    x = normal(s, 0, c["n"], 0.0, 0.02)
    pos = select(s, 1, c["n"], c["outliers"])
    x[pos] = normal(s, 2, c["n"], 0.0, 1.0)[pos]
    b, B = c["zero_block"], c["block"]
    x[b * B:(b + 1) * B] = 0.0
    return to_f16(x)


QWZ_LAYER = dict(n=sum(a * b for a, b in QWZ_LAYER_SHAPES), block=256, world=16)


def qwz_layer(offset=0, n=None):
    """fp16 elements [offset, offset+n) of the flattened layer."""
    s = SEEDS["qwz_layer"]
    total = QWZ_LAYER["n"]
    n = total - offset if n is None else n
    return _chunked(n, lambda o, m: normal(s, 0, m, 0.0, 0.02, offset + o), to_f16, np.float16)


def qwz_shard(rank=0):
    W = QWZ_LAYER["world"]
    S = QWZ_LAYER["n"] // W
    return qwz_layer(rank * S, S)


QGZ_HOP1 = dict(n=1 << 28, block=128, L=8, N=4)


def qgz_hop1(offset=0, n=None):
    """bf16 bits, elements [offset, offset+n) of the hop-1 gradient."""
    s = SEEDS["qgz_hop1"]
    c = QGZ_HOP1
    n = c["n"] - offset if n is None else n
    return _chunked(n, lambda o, m: blockvar_normal(s, 0, m, c["block"], 1e-3, -2.0, 2.0,
                                                    offset + o),
                    to_bf16_bits, np.uint16)


QGZ_HOP2 = dict(sources=16, chunk=1 << 24, block=128, divisor=16.0, out="bf16")


def qgz_hop2_source(i):
    """fp32 gradient slice of source rank i, N(0, 1e-3)."""
    s = SEEDS["qgz_hop2"]
    return normal(s, 200 + i, QGZ_HOP2["chunk"], 0.0, 1e-3)


QGZ_FUSED = dict(n=sum(a * b for a, b in QGZ_FUSED_SHAPES), block=64, L=8, N=48,
                 const_frac=0.01, zero_frac=0.005, out="f16")


def qgz_fused_special_blocks():
    """(constant block ids, their values as fp32, zero block ids), disjoint."""
    c = QGZ_FUSED
    s = SEEDS["qgz_fused"]
    nb = c["n"] // c["block"]
    n_const = int(round(c["const_frac"] * nb))
    n_zero = int(round(c["zero_frac"] * nb))
    keys = u64(s, 2, nb)
    order = np.argpartition(keys, n_const + n_zero)[:n_const + n_zero]
    order = order[np.argsort(keys[order], kind="stable")]
    const_ids = np.sort(order[:n_const])
    zero_ids = np.sort(order[n_const:])
    vals = student_t3(s, 3, nb, 1e-3)[const_ids]
    return const_ids, vals, zero_ids


def qgz_fused(offset=0, n=None, special=None):
    """fp16 elements [offset, offset+n) of the fused-qgZ gradient.  offset and
    n must be multiples of the block (64)."""
    c = QGZ_FUSED
    s = SEEDS["qgz_fused"]
    B = c["block"]
    n = c["n"] - offset if n is None else n
    assert offset % B == 0 and n % B == 0
    const_ids, vals, zero_ids = special if special is not None else qgz_fused_special_blocks()

    def gen(o, m):
        x = student_t3(s, 0, m, 1e-3, offset + o)
        b0, b1 = (offset + o) // B, (offset + o + m) // B
        xb = x.reshape(-1, B)
        lo, hi = np.searchsorted(const_ids, [b0, b1])
        xb[const_ids[lo:hi] - b0, :] = vals[lo:hi, None]
        lo, hi = np.searchsorted(zero_ids, [b0, b1])
        xb[zero_ids[lo:hi] - b0, :] = 0.0
        return x

    return _chunked(n, gen, to_f16, np.float16)
