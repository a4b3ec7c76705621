"""GPU parity past 2^31 elements: every kernel indexes elements with 64-bit
offsets (the hop-receive kernel takes chunks of up to 2^32 elements with
32-bit byte offsets).  Inputs are drawn on the GPU by torch's seeded
generator (not by the kernels under test); sampled blocks -- the first and
last, those around element 2^31, and random ones -- are copied back and
compared with the oracle bit for bit."""
import numpy as np
import pytest

import block_quantized_communication_amd as zpq
import oracle
from parity_util import assert_bits_equal

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + (1 << 14)       # elements


def torch():
    import torch as t
    return t


def gen(seed):
    T = torch()
    return T.Generator(device="cuda").manual_seed(seed)


def blocks_around_2p31(rng, nblocks, B):
    b31 = (1 << 31) // B
    s = {0, 1, nblocks - 2, nblocks - 1, b31 - 2, b31 - 1, b31, b31 + 1}
    s |= {int(v) for v in rng.integers(0, nblocks, 24)}
    return np.array(sorted(s), np.int64)


def rows(t, blocks, width):
    """Rows [b*width, (b+1)*width) of flat tensor t, for each block b, on the host."""
    T = torch()
    idx = (T.as_tensor(blocks)[:, None] * width + T.arange(width)[None, :]).cuda()
    return t[idx.ravel()].cpu()


def test_quant_dequant_i8_past_2p31():
    T = torch()
    B = 256
    print(f"quant/dequant_i8 n={BIG}", flush=True)
    x = (T.randn(BIG, generator=gen(11), device="cuda") * 0.02).half()
    codes, scales = zpq.quant_i8(x, B)
    y = zpq.dequant_i8(codes, scales, B, T.float16)
    T.cuda.synchronize()
    bl = blocks_around_2p31(np.random.default_rng(11), BIG // B, B)
    xs = rows(x, bl, B).numpy()
    ec, es = oracle.quant_i8(xs, "f16", B)
    assert_bits_equal(rows(codes, bl, B).numpy(), ec, "codes")
    assert_bits_equal(scales[T.as_tensor(bl).cuda()].cpu().numpy(), es, "scales")
    assert_bits_equal(rows(y, bl, B).numpy(), oracle.dequant_i8(ec, es, B, "f16"), "dequant")


def test_qgz_reorder_quant_i4_past_2p31():
    T = torch()
    L, N, B = 2, 2, 64
    n = BIG
    S = n // (L * N)
    print(f"qgz_reorder_quant_i4 n={n} L={L} N={N}", flush=True)
    g = (T.randn(n, generator=gen(12), device="cuda") * 1e-3).bfloat16()
    codes, scales = zpq.qgz_reorder_quant_i4(g, L, N, B)
    T.cuda.synchronize()
    bl = blocks_around_2p31(np.random.default_rng(12), n // B, B)
    src = oracle.reorder(np.arange(L * N, dtype=np.int64), L, N)   # slice at each position
    pos = bl * B
    start = src[pos // S] * S + pos % S                             # source element of each block
    xs = rows(g.view(T.int16), start // B, B).numpy().view(np.uint16)
    assert (start % B == 0).all()
    ec, es = oracle.qgz_reorder_quant_i4(xs, "bf16", 1, 1, B)        # blocks are independent
    assert_bits_equal(rows(codes, bl, B // 2).numpy(), ec, "codes")
    assert_bits_equal(scales[T.as_tensor(bl).cuda()].cpu().numpy(), es, "scales")


@pytest.mark.parametrize("mode", ["i4", "bf16"])
def test_dequant_reduce_past_2p31(mode):
    T = torch()
    K, B = 2, 128
    c = BIG                                    # chunk elements, below the 2^32 limit
    print(f"dequant_reduce mode={mode} K={K} chunk={c}", flush=True)
    codes = T.randint(0, 256, (K * c // 2,), generator=gen(13), device="cuda", dtype=T.uint8)
    scales = T.rand(K * c // B, generator=gen(14), device="cuda") * 1e-3
    if mode == "i4":
        oc, os_ = zpq.qgz_dequant_reduce_requant_i4(codes, scales, K, c, B)
    else:
        y = zpq.qgz_dequant_reduce_requant_i4(codes, scales, K, c, B, out_dtype=T.bfloat16,
                                               divisor=16.0)
    T.cuda.synchronize()
    bl = blocks_around_2p31(np.random.default_rng(13), c // B, B)
    # the sampled output blocks' sources, source-major as the kernel receives them
    ic = np.concatenate([rows(codes, i * (c // B) + bl, B // 2).numpy() for i in range(K)])
    isc = np.concatenate([scales[T.as_tensor(i * (c // B) + bl).cuda()].cpu().numpy()
                          for i in range(K)])
    m = bl.size * B
    if mode == "i4":
        rc, rs = oracle.qgz_dequant_reduce_requant_i4(ic, isc, K, m, B)
        assert_bits_equal(rows(oc, bl, B // 2).numpy(), rc, "codes")
        assert_bits_equal(os_[T.as_tensor(bl).cuda()].cpu().numpy(), rs, "scales")
    else:
        ry = oracle.qgz_dequant_reduce_requant_i4(ic, isc, K, m, B, "bf16", 16.0)
        got = rows(y.view(T.int16), bl, B).numpy().view(np.uint16)
        assert_bits_equal(got, ry, "values")


def test_dequant_i8_beyond_one_dispatch_grid():
    """2^35 + 2^12 elements: 2^24 + 2 workgroup tiles of 2048 elements, more
    than one dispatch can launch (2^32 - 1 work-items); the grid is capped and
    the first workgroups take a second tile.  Sampled: the first and last
    blocks, random blocks and every block of the three tiles that the second
    pass covers (with the XCD-contiguous tile order, tiles 2^21, 2^22 + 1 and
    2^24 + 1).  Needs about 97 GB of device memory."""
    T = torch()
    B, n = 256, (1 << 35) + (1 << 12)
    T.cuda.empty_cache()
    print(f"dequant_i8 n={n}: drawing codes", flush=True)
    codes = T.randint(-128, 128, (n,), generator=gen(15), device="cuda", dtype=T.int8)
    scales = T.rand(n // B, generator=gen(16), device="cuda") * 0.01
    y = zpq.dequant_i8(codes, scales, B, T.float16)
    T.cuda.synchronize()
    tiles = [1 << 21, (1 << 22) + 1, (1 << 24) + 1]
    s = {0, 1, n // B - 1} | {int(v) for v in np.random.default_rng(15).integers(0, n // B, 32)}
    s |= {t * 8 + k for t in tiles for k in range(-1, 9)}
    bl = np.array(sorted(b for b in s if 0 <= b < n // B), np.int64)
    cs = rows(codes, bl, B).numpy()
    ss = scales[T.as_tensor(bl).cuda()].cpu().numpy()
    assert_bits_equal(rows(y, bl, B).numpy(), oracle.dequant_i8(cs, ss, B, "f16"), "dequant")
    del codes, scales, y
    T.cuda.empty_cache()
