"""Python binding of libzpq, the ZeRO++ block-quantized communication kernels
for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of libzpq.so,
called through its C ABI (include/zpq.h).  PyTorch supplies device memory and
the current stream.  There is no fallback: if libzpq.so is missing or a call
fails, an exception is raised.

Functions (names follow the C ABI):
  quant_i8(x, block)                         -> (codes int8 [n], scales f32 [n/block])
  dequant_i8(codes, scales, block, dtype)    -> y [n]
  qgz_reorder_quant_i4(grad, L, N, block)    -> (codes uint8 [n/2], scales f32 [n/block])
  qgz_dequant_reduce_requant_i4(codes, scales, n_src, chunk, block,
                                out_dtype=None, divisor=1.0)
      out_dtype None: hop-1 mode, -> (codes uint8 [chunk/2], scales f32 [chunk/block])
      out_dtype set : hop-2 mode, -> averaged values [chunk] of that dtype
Each also accepts preallocated outputs (out=...) so that timed loops allocate
nothing.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzpq.so")

ZPQ_F32, ZPQ_F16, ZPQ_BF16 = 0, 1, 2
STATUS = {0: "ok", 1: "null pointer", 2: "bad size", 3: "bad block", 4: "misaligned pointer",
          5: "bad dtype", 6: "bad output mode", 7: "launch failed", 8: "bad argument",
          9: "output overlaps input"}

EXPORTS = ("zpq_quant_i8", "zpq_dequant_i8", "zpq_quant_i8_tensor", "zpq_qgz_reorder_quant_i4",
           "zpq_qgz_dequant_reduce_requant_i4", "zpq_status_str", "zpq_abi_version")


class ZpqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: libzpq status {status} ({_status_str(status)})")


_lib = None


def lib():
    """The loaded libzpq (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m block_quantized_communication_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.zpq_quant_i8.argtypes = [vp, i32, i64, i32, vp, vp, vp]
        L.zpq_dequant_i8.argtypes = [vp, vp, i64, i32, vp, i32, vp]
        L.zpq_quant_i8_tensor.argtypes = [vp, i32, i64, vp, vp, vp]
        L.zpq_qgz_reorder_quant_i4.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp]
        L.zpq_qgz_dequant_reduce_requant_i4.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp, i32,
                                                        f32, vp]
        for f in (L.zpq_quant_i8, L.zpq_dequant_i8, L.zpq_quant_i8_tensor,
                  L.zpq_qgz_reorder_quant_i4, L.zpq_qgz_dequant_reduce_requant_i4):
            f.restype = ctypes.c_int
        L.zpq_status_str.argtypes = [ctypes.c_int]
        L.zpq_status_str.restype = ctypes.c_char_p
        L.zpq_abi_version.argtypes = []
        L.zpq_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _status_str(status):
    try:
        return lib().zpq_status_str(status).decode()
    except Exception:
        return STATUS.get(status, "unknown")


def _torch():
    import torch
    return torch


def dtype_code(dt):
    torch = _torch()
    codes = {torch.float32: ZPQ_F32, torch.float16: ZPQ_F16, torch.bfloat16: ZPQ_BF16}
    if dt not in codes:
        raise ValueError(f"unsupported element type {dt} (float32, float16 or bfloat16)")
    return codes[dt]


def torch_dtype(code):
    torch = _torch()
    return {ZPQ_F32: torch.float32, ZPQ_F16: torch.float16, ZPQ_BF16: torch.bfloat16}[code]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, where):
    if rc != 0:
        raise ZpqError(rc, where)


def _gpu(t, name, device=None):
    """t must be a contiguous tensor on a GPU (on `device` when given): the
    library receives raw device pointers and checks neither."""
    if not t.is_cuda or not t.is_contiguous() or (device is not None and t.device != device):
        where = "a GPU" if device is None else str(device)
        raise ValueError(f"{name}: need a contiguous tensor on {where}, got "
                         f"{tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    return t.device


def _need(t, dtype, numel, name, device):
    _gpu(t, name, device)
    if t.dtype != dtype or t.numel() != numel:
        raise ValueError(f"{name}: need {numel} elements of {dtype}, got {t.numel()} of {t.dtype}")


def _blocks(n, block):
    return n // block if block > 0 else 0       # a bad block is refused by the library


def quant_i8(x, block=256, out=None, stream=None):
    """qwZ INT8 block quantization: x (fp32/fp16/bf16, CUDA) -> (codes, scales)."""
    torch = _torch()
    dev = _gpu(x, "x")
    n = x.numel()
    if out is None:
        out = (torch.empty(n, dtype=torch.int8, device=dev),
               torch.empty(_blocks(n, block), dtype=torch.float32, device=dev))
    codes, scales = out
    _need(codes, torch.int8, n, "codes", dev)
    _need(scales, torch.float32, _blocks(n, block), "scales", dev)
    rc = lib().zpq_quant_i8(_ptr(x), dtype_code(x.dtype), n, block, _ptr(codes), _ptr(scales),
                            _stream(stream, dev))
    _check(rc, "zpq_quant_i8")
    return codes, scales


def quant_i8_tensor(x, out=None, stream=None):
    """Non-blocked INT8 quantization, one scale for all of x -> (codes, scale[1])."""
    torch = _torch()
    dev = _gpu(x, "x")
    n = x.numel()
    if out is None:
        out = (torch.empty(n, dtype=torch.int8, device=dev),
               torch.empty(1, dtype=torch.float32, device=dev))
    codes, scale = out
    _need(codes, torch.int8, n, "codes", dev)
    _need(scale, torch.float32, 1, "scale", dev)
    rc = lib().zpq_quant_i8_tensor(_ptr(x), dtype_code(x.dtype), n, _ptr(codes), _ptr(scale),
                                   _stream(stream, dev))
    _check(rc, "zpq_quant_i8_tensor")
    return codes, scale


def dequant_i8(codes, scales, block=256, dtype=None, out=None, stream=None):
    """qwZ INT8 block dequantization: (codes, scales) -> y of `dtype`."""
    torch = _torch()
    dev = _gpu(codes, "codes")
    n = codes.numel()
    _need(codes, torch.int8, n, "codes", dev)
    _need(scales, torch.float32, _blocks(n, block), "scales", dev)
    if out is None:
        out = torch.empty(n, dtype=dtype or torch.float16, device=dev)
    _need(out, out.dtype, n, "out", dev)
    rc = lib().zpq_dequant_i8(_ptr(codes), _ptr(scales), n, block, _ptr(out),
                              dtype_code(out.dtype), _stream(stream, dev))
    _check(rc, "zpq_dequant_i8")
    return out


def qgz_reorder_quant_i4(grad, local_ranks, nodes, block=128, out=None, stream=None):
    """qgZ slice reorder + INT4 block quantization -> (codes [n/2], scales [n/block])."""
    torch = _torch()
    dev = _gpu(grad, "grad")
    n = grad.numel()
    if out is None:
        out = (torch.empty(n // 2, dtype=torch.uint8, device=dev),
               torch.empty(_blocks(n, block), dtype=torch.float32, device=dev))
    codes, scales = out
    _need(codes, torch.uint8, n // 2, "codes", dev)
    _need(scales, torch.float32, _blocks(n, block), "scales", dev)
    rc = lib().zpq_qgz_reorder_quant_i4(_ptr(grad), dtype_code(grad.dtype), n, local_ranks, nodes,
                                        block, _ptr(codes), _ptr(scales), _stream(stream, dev))
    _check(rc, "zpq_qgz_reorder_quant_i4")
    return codes, scales


def qgz_dequant_reduce_requant_i4(in_codes, in_scales, n_src, chunk, block=128, out_dtype=None,
                                  divisor=1.0, out=None, stream=None):
    """qgZ receive side of one all-to-all hop.  Hop 1 (out_dtype None and out
    None or a (codes, scales) pair): -> (codes [chunk/2], scales [chunk/block]);
    hop 2: -> values [chunk] of out_dtype (or of out's type)."""
    torch = _torch()
    dev = _gpu(in_codes, "in_codes")
    _need(in_codes, torch.uint8, n_src * (chunk // 2), "in_codes", dev)
    _need(in_scales, torch.float32, n_src * _blocks(chunk, block), "in_scales", dev)
    if out_dtype is None and (out is None or isinstance(out, tuple)):
        if out is None:
            out = (torch.empty(chunk // 2, dtype=torch.uint8, device=dev),
                   torch.empty(_blocks(chunk, block), dtype=torch.float32, device=dev))
        oc, os_ = out
        _need(oc, torch.uint8, chunk // 2, "out_codes", dev)
        _need(os_, torch.float32, _blocks(chunk, block), "out_scales", dev)
        rc = lib().zpq_qgz_dequant_reduce_requant_i4(
            _ptr(in_codes), _ptr(in_scales), n_src, chunk, block, _ptr(oc), _ptr(os_),
            ctypes.c_void_p(0), 0, ctypes.c_float(1.0), _stream(stream, dev))
        _check(rc, "zpq_qgz_dequant_reduce_requant_i4")
        return oc, os_
    if out is None:
        out = torch.empty(chunk, dtype=out_dtype, device=dev)
    _need(out, out.dtype, chunk, "out", dev)
    rc = lib().zpq_qgz_dequant_reduce_requant_i4(
        _ptr(in_codes), _ptr(in_scales), n_src, chunk, block, ctypes.c_void_p(0),
        ctypes.c_void_p(0), _ptr(out), dtype_code(out.dtype), ctypes.c_float(divisor),
        _stream(stream, dev))
    _check(rc, "zpq_qgz_dequant_reduce_requant_i4")
    return out


def abi_version():
    return int(lib().zpq_abi_version())
