"""CPU oracle for the ZeRO++ qwZ / qgZ quantization path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py.  The product package never imports it.

Thin ctypes wrapper over oracle/libzpq_ref.so (plain single-threaded C).
Arrays are numpy; fp16 arrays are np.float16, bf16 arrays are carried as raw
np.uint16 bit patterns, fp32 arrays are np.float32.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        sig = {
            "zpq_ref_f16_to_f32": ([vp, i64, vp], None),
            "zpq_ref_bf16_to_f32": ([vp, i64, vp], None),
            "zpq_ref_f32_to_f16": ([vp, i64, vp], None),
            "zpq_ref_f32_to_bf16": ([vp, i64, vp], None),
            "zpq_ref_block_quant": ([vp, i64, i32, i32, vp, vp], ctypes.c_int),
            "zpq_ref_block_dequant": ([vp, vp, i64, i32, vp], ctypes.c_int),
            "zpq_ref_pack_i4": ([vp, i64, vp], ctypes.c_int),
            "zpq_ref_unpack_i4": ([vp, i64, vp], ctypes.c_int),
            "zpq_ref_reorder": ([vp, i64, i64, i32, i32, vp], ctypes.c_int),
            "zpq_ref_reduce_add": ([vp, vp, i64], None),
            "zpq_ref_average": ([vp, i64, f32, vp], None),
            "zpq_ref_quant_i8": ([vp, ctypes.c_int, i64, i32, vp, vp], ctypes.c_int),
            "zpq_ref_dequant_i8": ([vp, vp, i64, i32, vp, ctypes.c_int], ctypes.c_int),
            "zpq_ref_qgz_reorder_quant_i4": ([vp, ctypes.c_int, i64, i32, i32, i32, vp, vp],
                                             ctypes.c_int),
            "zpq_ref_qgz_dequant_reduce_requant_i4": (
                [vp, vp, i32, i64, i32, vp, vp, vp, ctypes.c_int, f32], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")


def _raw16(x, dtype):
    """Input as (contiguous array, type code); bf16 must be np.uint16 bits."""
    if dtype == "f32":
        return _c(x, np.float32), F32
    if dtype == "f16":
        return _c(x, np.float16), F16
    if dtype == "bf16":
        return _c(x, np.uint16), BF16
    raise ValueError(dtype)


# ---- single steps ---------------------------------------------------------

def f16_to_f32(h):
    h = _c(h, np.float16)
    out = np.empty(h.shape, np.float32)
    lib().zpq_ref_f16_to_f32(_p(h), h.size, _p(out))
    return out


def bf16_to_f32(b):
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().zpq_ref_bf16_to_f32(_p(b), b.size, _p(out))
    return out


def f32_to_f16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().zpq_ref_f32_to_f16(_p(x), x.size, _p(out))
    return out.view(np.float16)


def f32_to_bf16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().zpq_ref_f32_to_bf16(_p(x), x.size, _p(out))
    return out


def widen(x, dtype):
    if dtype == "f32":
        return _c(x, np.float32).copy()
    if dtype == "f16":
        return f16_to_f32(x)
    if dtype == "bf16":
        return bf16_to_f32(x)
    raise ValueError(dtype)


def narrow(v, dtype):
    if dtype == "f32":
        return _c(v, np.float32).copy()
    if dtype == "f16":
        return f32_to_f16(v)
    if dtype == "bf16":
        return f32_to_bf16(v)
    raise ValueError(dtype)


def block_quant(x, block, qmax):
    x = _c(x, np.float32)
    codes = np.empty(x.size, np.int8)
    scales = np.empty(x.size // block if block > 0 else 0, np.float32)
    _check(lib().zpq_ref_block_quant(_p(x), x.size, block, qmax, _p(codes), _p(scales)))
    return codes, scales


def block_dequant(codes, scales, block):
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    out = np.empty(codes.size, np.float32)
    _check(lib().zpq_ref_block_dequant(_p(codes), _p(scales), codes.size, block, _p(out)))
    return out


def pack_i4(codes):
    codes = _c(codes, np.int8)
    out = np.empty(codes.size // 2, np.uint8)
    _check(lib().zpq_ref_pack_i4(_p(codes), codes.size, _p(out)))
    return out


def unpack_i4(packed, n=None):
    packed = _c(packed, np.uint8)
    n = packed.size * 2 if n is None else n
    out = np.empty(n, np.int8)
    _check(lib().zpq_ref_unpack_i4(_p(packed), n, _p(out)))
    return out


def reorder(x, L, N):
    """O7 on any fixed-size element type (a flat array)."""
    x = np.ascontiguousarray(x)
    out = np.empty_like(x)
    _check(lib().zpq_ref_reorder(_p(x), x.dtype.itemsize, x.size, L, N, _p(out)))
    return out


def reduce_add(acc, d):
    """acc <- fl32(acc + d), in place; returns acc."""
    if acc.dtype != np.float32 or not acc.flags.c_contiguous:
        raise TypeError("acc must be a contiguous float32 array")
    d = _c(d, np.float32)
    lib().zpq_ref_reduce_add(_p(acc), _p(d), acc.size)
    return acc


def average(acc, divisor):
    acc = _c(acc, np.float32)
    out = np.empty_like(acc)
    lib().zpq_ref_average(_p(acc), acc.size, ctypes.c_float(divisor), _p(out))
    return out


# ---- compositions mirroring the four libzpq entry points ------------------

def quant_i8(x, dtype, block):
    x, t = _raw16(x, dtype)
    codes = np.empty(x.size, np.int8)
    scales = np.empty(x.size // block, np.float32)
    _check(lib().zpq_ref_quant_i8(_p(x), t, x.size, block, _p(codes), _p(scales)))
    return codes, scales


def dequant_i8(codes, scales, block, out_dtype):
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    n = codes.size
    out = np.empty(n, {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[out_dtype])
    _check(lib().zpq_ref_dequant_i8(_p(codes), _p(scales), n, block, _p(out), DTYPES[out_dtype]))
    return out


def qgz_reorder_quant_i4(g, dtype, L, N, block):
    g, t = _raw16(g, dtype)
    n = g.size
    codes = np.empty(n // 2, np.uint8)
    scales = np.empty(n // block, np.float32)
    _check(lib().zpq_ref_qgz_reorder_quant_i4(_p(g), t, n, L, N, block, _p(codes), _p(scales)))
    return codes, scales


def qgz_dequant_reduce_requant_i4(in_codes, in_scales, K, chunk, block,
                                  out_dtype=None, divisor=1.0):
    """Mode I4 when out_dtype is None (returns codes, scales); mode FLOAT
    otherwise (returns the averaged values in out_dtype)."""
    in_codes = _c(in_codes, np.uint8)
    in_scales = _c(in_scales, np.float32)
    if in_codes.size != K * (chunk // 2) or in_scales.size != K * (chunk // block):
        raise ValueError("input sizes do not match K, chunk, block")
    L = lib()
    null = ctypes.c_void_p(0)
    if out_dtype is None:
        oc = np.empty(chunk // 2, np.uint8)
        os_ = np.empty(chunk // block, np.float32)
        _check(L.zpq_ref_qgz_dequant_reduce_requant_i4(
            _p(in_codes), _p(in_scales), K, chunk, block, _p(oc), _p(os_), null, 0,
            ctypes.c_float(1.0)))
        return oc, os_
    out = np.empty(chunk, {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[out_dtype])
    _check(L.zpq_ref_qgz_dequant_reduce_requant_i4(
        _p(in_codes), _p(in_scales), K, chunk, block, null, null, _p(out),
        DTYPES[out_dtype], ctypes.c_float(divisor)))
    return out
