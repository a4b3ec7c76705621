"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.

Where the oracle is fast enough the whole output is compared (qwZ round
trip, the qwZ shard, qgZ hop 2).  Elsewhere sampled blocks are compared: the
oracle recomputes each sampled output block from the generator's input
through every preceding step (slice reorder, INT4 quantization, hop-1
reduction), so no oracle input ever comes from the GPU.  Simulated
all-to-alls: the hop-1 receive buffer of rank (node 0, local 0) is stood in by
that rank's own L send chunks, and the hop-2 receive buffer by the N send
positions of its own hop-1 result (same shapes and statistics as the chunks
other ranks would send).
"""
import numpy as np
import pytest

import block_quantized_communication_amd as zpq
import oracle
import synth
from parity_util import assert_bits_equal, from_device

pytestmark = pytest.mark.gpu

NSAMPLE = 48


def torch():
    import torch as t
    return t


def dev(a, bf16=False):
    t = torch().from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch().bfloat16)
    return t.cuda()


def gather_bytes(t, starts, width):
    """Bytes [s, s + width) of a flat CUDA uint8/int8 tensor for each start."""
    T = torch()
    idx = (T.as_tensor(np.asarray(starts, np.int64))[:, None] + T.arange(width)[None, :]).cuda()
    return t.view(T.uint8)[idx.ravel()].cpu().numpy()


def gather_f32(t, idx):
    T = torch()
    return t[T.as_tensor(np.asarray(idx, np.int64)).cuda()].cpu().numpy()


def sample_blocks(rng, nblocks, extra=()):
    s = set(int(v) for v in rng.integers(0, nblocks, NSAMPLE))
    s |= {0, nblocks - 1} | {int(v) for v in extra}
    return np.array(sorted(s), np.int64)


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
    print(f"qwz_layer n={n} shard={S}", flush=True)
    layer = synth.qwz_layer()
    xd = dev(layer)
    # rank 0's shard: full comparison
    sc, ss = zpq.quant_i8(xd[:S], B)
    rc, rs = oracle.quant_i8(layer[:S], "f16", B)
    assert_bits_equal(from_device(sc), rc, "shard codes")
    assert_bits_equal(from_device(ss), rs, "shard scales")
    # the gathered buffer: W shards quantized by their ranks and concatenated;
    # shard boundaries are block boundaries, so it is the whole-layer
    # quantization (one launch stands in for the W ranks)
    gc, gs = zpq.quant_i8(xd, B)
    T = torch()
    assert T.equal(gc[:S], sc) and T.equal(gs[:S // B].view(T.int32), ss.view(T.int32))
    y = zpq.dequant_i8(gc, gs, B, T.float16)
    del xd
    rng = np.random.default_rng(2)
    nb = n // B
    blocks = sample_blocks(rng, nb, extra=[r * (S // B) for r in range(W)] +
                           [r * (S // B) - 1 for r in range(1, W)])
    xs = np.concatenate([layer[b * B:(b + 1) * B] for b in blocks])
    ec, es = oracle.quant_i8(xs, "f16", B)
    ey = oracle.dequant_i8(ec, es, B, "f16")
    assert_bits_equal(gather_bytes(gc, blocks * B, B).view(np.int8), ec, "gathered codes")
    assert_bits_equal(gather_f32(gs, blocks), es, "gathered scales")
    gy = from_device(y)
    assert_bits_equal(np.concatenate([gy[b * B:(b + 1) * B] for b in blocks]), ey, "dequant")


def slice_source(L, N):
    """Slice carried by each send position, from the oracle's reorder."""
    return oracle.reorder(np.arange(L * N, dtype=np.int64), L, N)


def oracle_send_blocks(g, dtype, L, N, B, positions):
    """Oracle INT4 codes/scales of the send-order blocks starting at the given
    positions: each block is gathered from its source slice (the reorder) and
    quantized on its own (blocks are independent)."""
    n = g.size
    S = n // (L * N)
    src = slice_source(L, N)
    pos = np.asarray(positions, np.int64)
    start = src[pos // S] * S + pos % S
    xs = np.concatenate([g[s:s + B] for s in start])
    return oracle.qgz_reorder_quant_i4(xs, dtype, 1, 1, B)      # L = N = 1: no reorder


def test_qgz_hop1():
    c = synth.QGZ_HOP1
    L, N, B, n = c["L"], c["N"], c["block"], c["n"]
    chunk = n // L
    print(f"qgz_hop1 n={n} L={L} N={N} B={B}", flush=True)
    g = synth.qgz_hop1()
    c1, s1 = zpq.qgz_reorder_quant_i4(dev(g, bf16=True), L, N, B)
    c2, s2 = zpq.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)
    rng = np.random.default_rng(3)
    S = n // (L * N)
    # K3, sampled send blocks (including every slice's first and last block)
    blocks = sample_blocks(rng, n // B, extra=[p * S // B for p in range(L * N)] +
                           [(p + 1) * S // B - 1 for p in range(L * N)])
    ec, es = oracle_send_blocks(g, "bf16", L, N, B, blocks * B)
    assert_bits_equal(gather_bytes(c1, blocks * B // 2, B // 2), ec, "send codes")
    assert_bits_equal(gather_f32(s1, blocks), es, "send scales")
    # K4 hop 1, sampled output blocks: source i is send chunk i
    ob = sample_blocks(rng, chunk // B)
    pos = np.array([i * chunk + b * B for i in range(L) for b in ob], np.int64)
    ic, isc = oracle_send_blocks(g, "bf16", L, N, B, pos)         # [i][t] order
    rc, rs = oracle.qgz_dequant_reduce_requant_i4(ic, isc, L, ob.size * B, B)
    assert_bits_equal(gather_bytes(c2, ob * B // 2, B // 2), rc, "hop-1 codes")
    assert_bits_equal(gather_f32(s2, ob), rs, "hop-1 scales")


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
    print(f"qgz_fused n={n} L={L} N={N} B={B}: generating", flush=True)
    g = synth.qgz_fused()
    print("qgz_fused: running the three kernels", flush=True)
    gd = dev(g)
    c1, s1 = zpq.qgz_reorder_quant_i4(gd, L, N, B)
    del gd
    c2, s2 = zpq.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)
    y = zpq.qgz_dequant_reduce_requant_i4(c2, s2, N, S, B, out_dtype=torch().float16,
                                           divisor=float(W))
    torch().cuda.synchronize()
    print("qgz_fused: sampled oracle chain", flush=True)
    rng = np.random.default_rng(5)
    ob = sample_blocks(rng, S // B)
    T = ob.size
    # level 1: send blocks at i*chunk + m*S + b*B, ordered [m][i][t]
    pos = np.array([i * chunk + m * S + b * B for m in range(N) for i in range(L) for b in ob],
                   np.int64)
    ec1, es1 = oracle_send_blocks(g, "f16", L, N, B, pos)
    assert_bits_equal(gather_bytes(c1, pos // 2, B // 2), ec1, "send codes")
    assert_bits_equal(gather_f32(s1, pos // B), es1, "send scales")
    # level 2: per node position m, reduce the L sources over the T blocks
    cb, sb = (B // 2) * T, T
    ec2, es2 = [], []
    for m in range(N):
        ic = ec1[m * L * cb:(m + 1) * L * cb]
        isc = es1[m * L * sb:(m + 1) * L * sb]
        rc, rs = oracle.qgz_dequant_reduce_requant_i4(ic, isc, L, T * B, B)
        ec2.append(rc)
        es2.append(rs)
    pos2 = np.array([m * S + b * B for m in range(N) for b in ob], np.int64)
    assert_bits_equal(gather_bytes(c2, pos2 // 2, B // 2), np.concatenate(ec2), "hop-1 codes")
    assert_bits_equal(gather_f32(s2, pos2 // B), np.concatenate(es2), "hop-1 scales")
    # level 3: average over the N hop-2 sources
    ey = oracle.qgz_dequant_reduce_requant_i4(np.concatenate(ec2), np.concatenate(es2), N,
                                              T * B, B, "f16", float(W))
    gy = from_device(y)
    assert_bits_equal(np.concatenate([gy[b * B:(b + 1) * B] for b in ob]), ey, "averaged")
