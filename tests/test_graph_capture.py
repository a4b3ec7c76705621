"""The library under HIP graph capture: it allocates nothing, never
synchronizes and records no memset, so the whole qwZ + qgZ chain can be
captured once and replayed.  Each replay follows eager work (new inputs
copied in, an eager run of the same chain into other buffers, a device
synchronize) and must equal that eager result bit for bit."""
import numpy as np
import pytest

import block_quantized_communication_amd as zpq

pytestmark = pytest.mark.gpu


def chain(x, g, L, N, B, out):
    """qwZ quantize + dequantize of x, qgZ send + both hops of g, into `out`."""
    import torch
    n = g.numel()
    zpq.quant_i8(x, 256, out=(out["c8"], out["s8"]))
    zpq.dequant_i8(out["c8"], out["s8"], 256, out=out["y8"])
    zpq.quant_i8_tensor(x, out=(out["ct"], out["st"]))
    zpq.qgz_reorder_quant_i4(g, L, N, B, out=(out["c4"], out["s4"]))
    zpq.qgz_dequant_reduce_requant_i4(out["c4"], out["s4"], L, n // L, B,
                                      out=(out["c5"], out["s5"]))
    zpq.qgz_dequant_reduce_requant_i4(out["c5"], out["s5"], N, n // (L * N), B,
                                      out_dtype=torch.float16, divisor=float(L * N),
                                      out=out["y5"])


def buffers(n, g_n, L, N, B):
    import torch
    e = lambda k, dt: torch.empty(k, dtype=dt, device="cuda")
    return {"c8": e(n, torch.int8), "s8": e(n // 256, torch.float32), "y8": e(n, torch.float16),
            "ct": e(n, torch.int8), "st": e(1, torch.float32),
            "c4": e(g_n // 2, torch.uint8), "s4": e(g_n // B, torch.float32),
            "c5": e(g_n // L // 2, torch.uint8), "s5": e(g_n // L // B, torch.float32),
            "y5": e(g_n // (L * N), torch.float16)}


def same(a, b):
    import torch
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_captured_chain_replays_equal_eager():
    import torch
    n, L, N, B = 1 << 20, 4, 2, 64
    gn = L * N * B * 2048
    gen = torch.Generator(device="cuda").manual_seed(21)
    x = (torch.randn(n, generator=gen, device="cuda") * 0.02).half()
    g = (torch.randn(gn, generator=gen, device="cuda") * 1e-3).half()
    graph_out, eager_out = buffers(n, gn, L, N, B), buffers(n, gn, L, N, B)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up outside the capture
        chain(x, g, L, N, B, graph_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(x, g, L, N, B, graph_out)
    torch.cuda.synchronize()
    for rep in range(4):
        print(f"graph replay {rep}", flush=True)
        x.copy_((torch.randn(n, generator=gen, device="cuda") * (0.01 * (rep + 1))).half())
        g.copy_((torch.randn(gn, generator=gen, device="cuda") * 1e-3).half())
        for t in graph_out.values():
            t.view(torch.uint8).fill_(0xA5)          # stale contents must be overwritten
        chain(x, g, L, N, B, eager_out)              # eager result, other buffers
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = [k for k in graph_out if not same(graph_out[k], eager_out[k])]
        assert not bad, f"replay {rep}: {bad} differ from the eager run"
