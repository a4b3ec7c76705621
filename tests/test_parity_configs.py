"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every output byte of every kernel is compared with the
oracle.

The oracle recomputes each output from the generator's input through every
preceding step (slice reorder, INT4 quantization, hop-1 reduction), so no
oracle input ever comes from the GPU.  It runs over independent ranges on
host threads (tests/oracle_ranges.py): whole send positions for the reorder
and quantization, block ranges of the received chunks for the hop kernels.
Simulated all-to-alls: the hop-1 receive buffer of rank (node 0, local 0) is
stood in by that rank's own L send chunks, and the hop-2 receive buffer by
the N send positions of its own hop-1 result (same shapes and statistics as
the chunks other ranks would send).
"""
import time

import numpy as np
import pytest

import block_quantized_communication_amd as zpq
import oracle
import synth
from oracle_ranges import oracle_receive, oracle_send, pmap
from parity_util import assert_bits_equal, from_device

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def dev(a, bf16=False):
    t = torch().from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch().bfloat16)
    return t.cuda()


def say(msg):
    import resource
    rss = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 2 ** 20
    print(f"[{time.strftime('%H:%M:%S')} peak RSS {rss:.1f} GiB] {msg}", flush=True)


def test_qwz_roundtrip_full():
    c = synth.QWZ_ROUNDTRIP
    x = synth.qwz_roundtrip()
    print(f"qwz_roundtrip n={x.size}", flush=True)
    codes, scales = zpq.quant_i8(dev(x), c["block"])
    y = zpq.dequant_i8(codes, scales, c["block"], torch().float16)
    rc, rs = oracle.quant_i8(x, "f16", c["block"])
    assert_bits_equal(from_device(codes), rc, "codes")
    assert_bits_equal(from_device(scales), rs, "scales")
    assert_bits_equal(from_device(y), oracle.dequant_i8(rc, rs, c["block"], "f16"), "dequant")
    # the all-zero block decodes to +0
    b, B = c["zero_block"], c["block"]
    assert (from_device(y)[b * B:(b + 1) * B].view(np.uint16) == 0).all()


def test_qwz_layer_shard_and_gathered():
    c = synth.QWZ_LAYER
    B, W = c["block"], c["world"]
    n = c["n"]
    S = n // W
    say(f"qwz_layer n={n} shard={S}: generating")
    layer = synth.qwz_layer()
    xd = dev(layer)
    # rank 0's shard
    sc, ss = zpq.quant_i8(xd[:S], B)
    # the gathered buffer: W shards quantized by their ranks and concatenated;
    # shard boundaries are block boundaries, so it is the whole-layer
    # quantization (one launch stands in for the W ranks)
    gc, gs = zpq.quant_i8(xd, B)
    T = torch()
    assert T.equal(gc[:S], sc) and T.equal(gs[:S // B].view(T.int32), ss.view(T.int32))
    y = zpq.dequant_i8(gc, gs, B, T.float16)
    del xd
    gch, gsh, yh = from_device(gc), from_device(gs), from_device(y)
    say("qwz_layer: oracle over 48 ranges")
    R = 1 << 24
    assert n % R == 0

    def one(r0):
        ec, es = oracle.quant_i8(layer[r0:r0 + R], "f16", B)
        return ec, es, oracle.dequant_i8(ec, es, B, "f16")
    parts = pmap(one, range(0, n, R))
    ec = np.concatenate([p[0] for p in parts])
    es = np.concatenate([p[1] for p in parts])
    assert_bits_equal(gch, ec, "gathered codes")
    assert_bits_equal(gsh, es, "gathered scales")
    assert_bits_equal(yh, np.concatenate([p[2] for p in parts]), "dequant")
    assert_bits_equal(from_device(sc), ec[:S], "shard codes")
    assert_bits_equal(from_device(ss), es[:S // B], "shard scales")
    say("qwz_layer: every byte equal")


def test_qgz_hop1():
    c = synth.QGZ_HOP1
    L, N, B, n = c["L"], c["N"], c["block"], c["n"]
    chunk = n // L
    say(f"qgz_hop1 n={n} L={L} N={N} B={B}: generating")
    g = synth.qgz_hop1()
    c1, s1 = zpq.qgz_reorder_quant_i4(dev(g, bf16=True), L, N, B)
    c2, s2 = zpq.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)
    c1h, s1h, c2h, s2h = (from_device(t) for t in (c1, s1, c2, s2))
    say("qgz_hop1: oracle send buffer")
    ec1, es1 = oracle_send(g, "bf16", L, N, B)
    assert_bits_equal(c1h, ec1, "send codes")
    assert_bits_equal(s1h, es1, "send scales")
    say("qgz_hop1: oracle hop-1 receive (source i = send chunk i)")
    ec2, es2 = oracle_receive(ec1, es1, L, chunk, B, 64)
    assert_bits_equal(c2h, ec2, "hop-1 codes")
    assert_bits_equal(s2h, es2, "hop-1 scales")
    say("qgz_hop1: every byte equal")


def test_qgz_hop2_full():
    c = synth.QGZ_HOP2
    K, chunk, B = c["sources"], c["chunk"], c["block"]
    print(f"qgz_hop2 K={K} chunk={chunk} B={B}", flush=True)
    codes, scales = [], []
    for i in range(K):
        q, s = oracle.block_quant(synth.qgz_hop2_source(i), B, 7)
        codes.append(oracle.pack_i4(q))
        scales.append(s)
    codes = np.concatenate(codes)
    scales = np.concatenate(scales)
    y = zpq.qgz_dequant_reduce_requant_i4(dev(codes), dev(scales), K, chunk, B,
                                           out_dtype=torch().bfloat16, divisor=c["divisor"])
    ref = oracle.qgz_dequant_reduce_requant_i4(codes, scales, K, chunk, B, "bf16", c["divisor"])
    assert_bits_equal(from_device(y), ref, "averaged gradient")


def test_qgz_fused_both_hops():
    c = synth.QGZ_FUSED
    L, N, B, n = c["L"], c["N"], c["block"], c["n"]
    W = L * N
    S = n // W
    chunk = n // L
    say(f"qgz_fused n={n} L={L} N={N} B={B}: generating")
    g = synth.qgz_fused()
    say("qgz_fused: running the three kernels")
    gd = dev(g)
    c1, s1 = zpq.qgz_reorder_quant_i4(gd, L, N, B)
    del gd
    c2, s2 = zpq.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)
    y = zpq.qgz_dequant_reduce_requant_i4(c2, s2, N, S, B, out_dtype=torch().float16,
                                           divisor=float(W))
    c1h, s1h, c2h, s2h, yh = (from_device(t) for t in (c1, s1, c2, s2, y))
    del c1, s1, c2, s2, y
    say("qgz_fused: oracle send buffer (384 positions)")
    ec1, es1 = oracle_send(g, "f16", L, N, B)
    del g
    assert_bits_equal(c1h, ec1, "send codes")
    assert_bits_equal(s1h, es1, "send scales")
    say("qgz_fused: oracle hop-1 receive")
    ec2, es2 = oracle_receive(ec1, es1, L, chunk, B, 48)
    assert_bits_equal(c2h, ec2, "hop-1 codes")
    assert_bits_equal(s2h, es2, "hop-1 scales")
    say("qgz_fused: oracle hop-2 receive and average")
    ey = oracle_receive(ec2, es2, N, S, B, 16, "f16", float(W))
    assert_bits_equal(yh, ey, "averaged")
    say("qgz_fused: every byte equal")
