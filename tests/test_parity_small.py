"""GPU parity of every libzpq entry point against the CPU oracle, bit for bit,
at sizes the oracle handles in seconds: several workgroup tiles plus a ragged
tail, every element type and block size, adversarial blocks, edge cases."""
import numpy as np
import pytest

import block_quantized_communication_amd as zpq
import oracle
from parity_util import (adversarial_f32, as_dtype, assert_bits_equal,
                         assert_equal_nan_aware, from_device, to_device)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]
BLOCKS = [32, 64, 128, 256, 512]
# Largest workgroup tile of the quantize kernels: fp32 inputs hold 16 elements per
# lane, two tiles per lane (8192 elements); 16-bit inputs hold 8 per lane (4096).
# Sizes below are multiples of it plus a ragged tail, so they span several tiles
# of every element type.
TILE = 256 * 16 * 2


def torch_dt(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("block", BLOCKS)
def test_quant_i8(dtype, block):
    rng = np.random.default_rng(block * 7 + len(dtype))
    for nblocks in (1, 3, 2 * TILE // block + 5):          # ragged tails
        n = nblocks * block
        x = as_dtype(adversarial_f32(rng, n, block), dtype)
        print(f"quant_i8 dtype={dtype} block={block} n={n}", flush=True)
        codes, scales = zpq.quant_i8(to_device(x, dtype), block)
        rc, rs = oracle.quant_i8(x, dtype, block)
        assert_bits_equal(from_device(scales), rs, "scales")
        assert_bits_equal(from_device(codes), rc, "codes")


@pytest.mark.parametrize("out", DTYPES)
@pytest.mark.parametrize("block", [32, 256, 512])
def test_dequant_i8(out, block):
    rng = np.random.default_rng(block + len(out))
    n = (2 * TILE // block + 3) * block
    codes = rng.integers(-128, 128, n).astype(np.int8)        # -128 too: any int8 decodes
    s = rng.standard_normal(n // block).astype(np.float32) * np.float32(0.01)
    s[::7] = 0.0
    s[1::7] = np.float32(3e-41)                                # subnormal scales
    s[2::7] = np.float32(2.6e36)                               # 127 * s near FLT_MAX
    s[3::7] = np.abs(s[3::7]) * np.float32(1e-3)               # fp16-subnormal outputs
    print(f"dequant_i8 out={out} block={block} n={n}", flush=True)
    y = zpq.dequant_i8(to_device(codes), to_device(s), block, torch_dt(out))
    assert_bits_equal(from_device(y), oracle.dequant_i8(codes, s, block, out), "values")


def test_quant_dequant_roundtrip_f16_all_values():
    """Every finite fp16 value inside blocks of every scale class."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    h = h[: h.size - h.size % 256]
    rng = np.random.default_rng(1)
    x = rng.permutation(h)
    codes, scales = zpq.quant_i8(to_device(x), 256)
    rc, rs = oracle.quant_i8(x, "f16", 256)
    assert_bits_equal(from_device(codes), rc, "codes")
    assert_bits_equal(from_device(scales), rs, "scales")
    y = zpq.dequant_i8(codes, scales, 256, torch_dt("f16"))
    assert_bits_equal(from_device(y), oracle.dequant_i8(rc, rs, 256, "f16"), "dequant")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("block", [32, 64, 128, 512])
@pytest.mark.parametrize("L,N", [(1, 1), (2, 2), (3, 2), (8, 4), (2, 5)])
def test_qgz_reorder_quant_i4(dtype, block, L, N):
    rng = np.random.default_rng(block + 10 * L + N)
    W = L * N
    for per_slice_blocks in (1, TILE // block + 3):          # slices shorter / longer than a tile
        n = W * per_slice_blocks * block
        x = as_dtype(adversarial_f32(rng, n, block), dtype)
        print(f"reorder_quant_i4 dtype={dtype} block={block} L={L} N={N} n={n}", flush=True)
        codes, scales = zpq.qgz_reorder_quant_i4(to_device(x, dtype), L, N, block)
        rc, rs = oracle.qgz_reorder_quant_i4(x, dtype, L, N, block)
        assert_bits_equal(from_device(scales), rs, "scales")
        assert_bits_equal(from_device(codes), rc, "codes")


def random_received(rng, K, chunk, block, huge=False):
    """K received INT4 chunks: random nibbles and scales of every class.
    Without `huge`, nibbles cover all 16 values (-8 included: any nibble
    decodes) and some scales exceed 2^100 (up to 1e32).  With `huge`, some scales exceed FLT_MAX/8 (so 8*s overflows)
    and nibbles stay in [-7, 7], as the quantizer produces, so that every true
    sum stays finite."""
    if huge:
        q = rng.integers(-7, 8, K * chunk).astype(np.int8)
        codes = ((q[0::2] & 0xF) | ((q[1::2] & 0xF) << 4)).astype(np.uint8)
    else:
        codes = rng.integers(0, 256, K * chunk // 2).astype(np.uint8)
    nb = chunk // block
    s = (np.abs(rng.standard_normal((K, nb))) * 10.0 ** rng.uniform(-4, 1, (K, 1))).astype(
        np.float32)
    s[:, ::9] = 0.0
    s[:, 1::9] = np.float32(1e-40)
    if not huge:
        s[:, 3::9] = np.float32(1e32)            # s * 2^24 overflows fp32; sums stay finite
        s[:, 4::9] = np.float32(3e30)            # just above 2^100
    if huge:
        s[0, 2::9] = np.float32(4.5e37)         # 8 * s overflows; 7 * s does not
        s[1:, 2::9] = 0.0                        # keep the true sums finite
    return codes, s.ravel()


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("K", [1, 2, 3, 5, 8, 16, 48, 97])
def test_dequant_reduce_requant_i4(block, K):
    rng = np.random.default_rng(block * 100 + K)
    chunk = (256 * 16 // block * 3 + 1) * block               # several tiles + ragged
    for huge in (False, True):
        if huge and K < 2:
            continue
        codes, s = random_received(rng, K, chunk, block, huge)
        print(f"dequant_reduce_requant_i4 block={block} K={K} chunk={chunk} huge={huge}",
              flush=True)
        oc, os_ = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk,
                                                     block)
        rc, rs = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block)
        assert_bits_equal(from_device(os_), rs, "scales")
        assert_bits_equal(from_device(oc), rc, "codes")


@pytest.mark.parametrize("out", DTYPES)
@pytest.mark.parametrize("block", [32, 64, 128, 512])
@pytest.mark.parametrize("K,divisor", [(1, 1.0), (3, 3.0), (16, 16.0), (48, 384.0),
                                       (8, 0.5), (5, 2.0 ** 50), (4, 1e-30), (3, 2.0 ** -126),
                                       (2, 2.0 ** 126), (2, 2.0 ** 127), (97, 97.0)])
def test_dequant_reduce_average(out, block, K, divisor):
    rng = np.random.default_rng(block + K)
    chunk = (256 * 16 // block * 2 + 3) * block
    for huge in (False, True):
        if huge and K < 2:
            continue
        codes, s = random_received(rng, K, chunk, block, huge)
        print(f"dequant_reduce_average out={out} block={block} K={K} div={divisor} "
              f"huge={huge}", flush=True)
        y = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk, block,
                                               out_dtype=torch_dt(out), divisor=divisor)
        ref = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block, out, divisor)
        assert_bits_equal(from_device(y), ref, "values")


@pytest.mark.parametrize("out", DTYPES)
@pytest.mark.parametrize("divisor", [1.0, 384.0, 0.5])
def test_dequant_reduce_average_overflowing_sums(out, divisor):
    """Sums that overflow, together with a source whose 8*s overflows fp32.
    Sources 0 and 1 have scales 4e37 (7 * s is finite, two such terms sum past
    FLT_MAX), source 2 has 4.3e37 (> FLT_MAX/8; -8 * s = -inf already in the
    definition).  Per element the definition gives +inf, -inf, NaN
    (+inf + -inf) or a finite value; the average must equal the oracle's,
    NaN where the oracle has NaN."""
    rng = np.random.default_rng(404)
    K, block = 3, 64
    chunk = (256 * 16 // block * 2 + 3) * block
    nb = chunk // block
    codes = rng.integers(0, 256, K * chunk // 2).astype(np.uint8)
    c = codes.reshape(K, chunk // 2)
    c[0:2, : chunk // 4] = 0x77          # code 7 in both nibbles: 2 * 7 * 4e37 overflows
    c[2, : chunk // 8] = 0x88            # code -8 with s > FLT_MAX/8: -inf term
    s = np.empty((K, nb), np.float32)
    s[0:2] = np.float32(4e37)
    s[2] = np.float32(4.3e37)
    s[:, nb - 5:] = rng.uniform(1e-3, 1.0, (K, 5)).astype(np.float32)   # ordinary tail blocks
    s = s.ravel()
    print(f"dequant_reduce_average overflowing sums out={out} divisor={divisor}", flush=True)
    y = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk, block,
                                           out_dtype=torch_dt(out), divisor=divisor)
    ref = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block, out, divisor)
    got = from_device(y)
    if out == "bf16":
        inf_pos = (ref == 0x7F80).sum()
        nan_pos = (((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)).sum()
    else:
        inf_pos = np.isposinf(ref).sum()
        nan_pos = np.isnan(ref).sum()
    assert inf_pos > 0 and nan_pos > 0, (inf_pos, nan_pos)   # the case is really exercised
    assert_equal_nan_aware(got, ref, out, "values")


@pytest.mark.parametrize("out", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("tail", [0, 128 * 3])
@pytest.mark.parametrize("divisor", [3.0, 16.0, 2.0 ** 127, 2.0 ** -126])
def test_dequant_reduce_average_long_chunk(out, tail, divisor):
    """A chunk long enough for the hop-2 launch with 16 elements per lane
    (short chunks take 8 per lane): 2^23 + 2^16 elements, 3 sources; with a
    tail, the last wave is partly empty and writes its outputs lane by lane
    (whole waves write theirs as coalesced 1 KB stores).  Powers of two take
    the multiply by 2^-k at this width: 2^127 makes subnormal and zero
    averages, 2^-126 overflowing ones."""
    rng = np.random.default_rng(77 + tail)
    K, block, chunk = 3, 128, (1 << 23) + (1 << 16) + tail
    codes, s = random_received(rng, K, chunk, block)
    print(f"dequant_reduce_average long chunk out={out} K={K} chunk={chunk} tail={tail} "
          f"div={divisor}", flush=True)
    y = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk, block,
                                           out_dtype=torch_dt(out), divisor=divisor)
    ref = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block, out, divisor)
    assert_bits_equal(from_device(y), ref, "values")


def requant_near_ties(rng, nblocks, block):
    """Received chunks whose fp32 sums land on and next to every rounding
    boundary of the hop-1 requantization.  Per block: element 0 is the block
    maximum a (so the requantized scale is s = fl32(a/7)); the others are the
    fp32 values nearest to (k + 1/2) * s, k = 0..6, and their neighbours up to
    4 ulp away, both signs.  Each value X is a multiple of 2^E (E = the exponent
    of a minus 27: every fp32 value of magnitude >= a/16 is one) and is built
    exactly as the sum of 10 sources: source i has scale 2^(E + 3(9 - i)) and
    code = the i-th base-8 digit of X / 2^E (sign of X), so every product and
    every partial sum is exact and the kernel's sum is X itself."""
    K = 10
    codes = np.zeros((K, nblocks * block), np.int8)
    scales = np.zeros((K, nblocks), np.float32)
    for b in range(nblocks):
        a = np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(-60, 60)))
        E = int(np.floor(np.log2(float(a)))) - 27
        s = np.float32(np.float32(a) / np.float32(7.0))
        vals = [a]
        for k in range(7):
            x0 = np.float32((k + 0.5) * float(s))
            lo = hi = x0
            vals += [x0, -x0]
            for _ in range(4):
                lo = np.nextafter(lo, np.float32(0))
                hi = np.nextafter(hi, np.float32(np.inf))
                vals += [lo, -lo, hi, -hi]
        vals = vals[:block] + [np.float32(0.0)] * (block - len(vals[:block]))
        for i in range(K):
            scales[i, b] = np.float32(2.0 ** (E + 3 * (9 - i)))
        for j, x in enumerate(vals):
            m = int(round(abs(float(x)) / 2.0 ** E))
            assert m * 2.0 ** E == abs(float(x)) and m < 1 << 30
            sign = -1 if x < 0 else 1
            for i in range(K):
                codes[i, b * block + j] = sign * ((m >> (3 * (9 - i))) & 7)
    packed = ((codes[:, 0::2].astype(np.int32) & 0xF) |
              ((codes[:, 1::2].astype(np.int32) & 0xF) << 4)).astype(np.uint8)
    return K, packed.ravel(), scales.ravel()


def test_requant_near_ties():
    """Hop-1 requantization of sums on and next to every rounding boundary
    (ties to even, values a few ulp either side), in 64 blocks of 128 with
    maxima across 120 binades: bit-exact against the oracle."""
    rng = np.random.default_rng(2024)
    block, nblocks = 128, 64
    K, codes, s = requant_near_ties(rng, nblocks, block)
    chunk = nblocks * block
    print(f"requant near ties K={K} chunk={chunk} block={block}", flush=True)
    oc, os_ = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk, block)
    rc, rs = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block)
    assert_bits_equal(from_device(os_), rs, "scales")
    assert_bits_equal(from_device(oc), rc, "codes")


@pytest.mark.parametrize("waves", [1023, 1025])
@pytest.mark.parametrize("mode", ["i4", "f16"])
def test_dequant_reduce_ragged_last_wave(mode, waves):
    """Receive launches of 1023 and 1025 waves (a last workgroup with 3 of
    its 4 waves busy, and one with 1) whose last wave is partly empty: a
    ragged tail of 3 blocks."""
    rng = np.random.default_rng(waves)
    K = 5
    block, epl = (128, 32) if mode == "i4" else (64, 8)      # the launch's elements per lane
    chunk = (waves - 1) * 64 * epl + 3 * block
    codes, s = random_received(rng, K, chunk, block)
    print(f"dequant_reduce ragged last wave mode={mode} waves={waves} chunk={chunk}",
          flush=True)
    if mode == "i4":
        oc, os_ = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk,
                                                     block)
        rc, rs = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block)
        assert_bits_equal(from_device(os_), rs, "scales")
        assert_bits_equal(from_device(oc), rc, "codes")
    else:
        y = zpq.qgz_dequant_reduce_requant_i4(to_device(codes), to_device(s), K, chunk, block,
                                               out_dtype=torch_dt("f16"), divisor=5.0)
        ref = oracle.qgz_dequant_reduce_requant_i4(codes, s, K, chunk, block, "f16", 5.0)
        assert_bits_equal(from_device(y), ref, "values")


def test_requant_single_source_is_identity():
    """Hop-1 requantization of one source returns the quantizer's own codes
    and scales (requantization is idempotent)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_t(3, 128 * 999) * 1e-3).astype(np.float32)
    codes, scales = zpq.qgz_reorder_quant_i4(to_device(x), 1, 1, 128)
    oc, os_ = zpq.qgz_dequant_reduce_requant_i4(codes, scales, 1, x.size, 128)
    assert_bits_equal(from_device(oc), from_device(codes), "codes")
    assert_bits_equal(from_device(os_), from_device(scales), "scales")


def test_empty_inputs_are_noops():
    import torch
    e = torch.empty(0, device="cuda")
    c, s = zpq.quant_i8(e.half(), 256)
    assert c.numel() == 0 and s.numel() == 0
    y = zpq.dequant_i8(c, s, 256, torch.float16)
    assert y.numel() == 0


def test_outputs_untouched_outside_range():
    """Canaries around every output: nothing is written past the end."""
    import torch
    rng = np.random.default_rng(5)
    n, block = 3 * 256 + 4096, 256
    x = to_device(as_dtype(adversarial_f32(rng, n, block), "f16"))
    guard = 4096
    cbuf = torch.full((n + 2 * guard,), 0x5A, dtype=torch.int8, device="cuda")
    sbuf = torch.full((n // block + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    zpq.quant_i8(x, block, out=(cbuf[guard:guard + n], sbuf[guard:guard + n // block]))
    torch.cuda.synchronize()
    assert (cbuf[:guard] == 0x5A).all() and (cbuf[guard + n:] == 0x5A).all()
    assert (sbuf[:guard] == 7.0).all() and (sbuf[guard + n // block:] == 7.0).all()
    # INT4 paths
    g = to_device(as_dtype(adversarial_f32(rng, 8 * 4 * 128 * 3, 128), "bf16"), "bf16")
    m = g.numel()
    cb = torch.full((m // 2 + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((m // 128 + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    zpq.qgz_reorder_quant_i4(g, 8, 4, 128, out=(cb[guard:guard + m // 2],
                                                sb[guard:guard + m // 128]))
    torch.cuda.synchronize()
    assert (cb[:guard] == 0xA5).all() and (cb[guard + m // 2:] == 0xA5).all()
    assert (sb[:guard] == 7.0).all() and (sb[guard + m // 128:] == 7.0).all()
    chunk = m // 8
    ob = torch.full((chunk // 2 + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    osb = torch.full((chunk // 128 + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    zpq.qgz_dequant_reduce_requant_i4(cb[guard:guard + m // 2], sb[guard:guard + m // 128], 8,
                                       chunk, 128, out=(ob[guard:guard + chunk // 2],
                                                        osb[guard:guard + chunk // 128]))
    vb = torch.full((chunk + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    zpq.qgz_dequant_reduce_requant_i4(cb[guard:guard + m // 2], sb[guard:guard + m // 128], 8,
                                       chunk, 128, out_dtype=torch.float32, divisor=8.0,
                                       out=vb[guard:guard + chunk])
    torch.cuda.synchronize()
    assert (ob[:guard] == 0xA5).all() and (ob[guard + chunk // 2:] == 0xA5).all()
    assert (osb[:guard] == 7.0).all() and (osb[guard + chunk // 128:] == 7.0).all()
    assert (vb[:guard] == 7.0).all() and (vb[guard + chunk:] == 7.0).all()


def test_deterministic_repeat():
    import torch
    rng = np.random.default_rng(8)
    g = to_device(as_dtype(adversarial_f32(rng, 8 * 48 * 64 * 5, 64), "f16"))
    a = zpq.qgz_reorder_quant_i4(g, 8, 48, 64)
    b = zpq.qgz_reorder_quant_i4(g, 8, 48, 64)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_16bit_absmax(dtype):
    """One block per positive finite fp16 / bf16 value a: [a, -a/3, a/7, 0, ...]
    through the INT8 and the INT4 quantizer (scale, absmax code, a few
    others) -- every scale the 16-bit inputs can produce."""
    bits = np.arange(1, 0x7F80 if dtype == "bf16" else 0x7C00, dtype=np.uint32).astype(np.uint16)
    a = oracle.bf16_to_f32(bits) if dtype == "bf16" else bits.view(np.float16).astype(np.float32)
    B = 32
    x32 = np.zeros((a.size, B), np.float32)
    x32[:, 0] = a
    x32[:, 1] = -a / 3
    x32[:, 2] = a / 7
    x32[:, 5] = a * 0.5
    x = as_dtype(x32.ravel(), dtype)
    if dtype == "bf16":
        x.reshape(-1, B)[:, 0] = bits          # exact absmax bits
    else:
        x.view(np.uint16).reshape(-1, B)[:, 0] = bits
    xd = to_device(x, dtype)
    codes, scales = zpq.quant_i8(xd, B)
    rc, rs = oracle.quant_i8(x, dtype, B)
    assert_bits_equal(from_device(scales), rs, "INT8 scales")
    assert_bits_equal(from_device(codes), rc, "INT8 codes")
    c4, s4 = zpq.qgz_reorder_quant_i4(xd, 1, 1, B)
    rc4, rs4 = oracle.qgz_reorder_quant_i4(x, dtype, 1, 1, B)
    assert_bits_equal(from_device(s4), rs4, "INT4 scales")
    assert_bits_equal(from_device(c4), rc4, "INT4 codes")


def test_ring_reduce_scatter_chain_matches_oracle():
    """The compressed-ring chain of the hop-count study (K = 2 requantization
    per hop, 15 hops) on the GPU equals the oracle's chain bit for bit."""
    import synth
    S, B, W = 4096, 128, 16
    g = np.stack([synth.blockvar_normal(40, 1000 + r, S, B, 1e-3, -2.0, 2.0) for r in range(W)])
    qg = [zpq.qgz_reorder_quant_i4(to_device(g[r]), 1, 1, B) for r in range(W)]
    qo = [oracle.qgz_reorder_quant_i4(g[r], "f32", 1, 1, B) for r in range(W)]
    pc, ps = qg[0]
    oc, os_ = qo[0]
    import torch
    for r in range(1, W):
        pc, ps = zpq.qgz_dequant_reduce_requant_i4(torch.cat([pc, qg[r][0]]),
                                                   torch.cat([ps, qg[r][1]]), 2, S, B)
        oc, os_ = oracle.qgz_dequant_reduce_requant_i4(np.concatenate([oc, qo[r][0]]),
                                                       np.concatenate([os_, qo[r][1]]), 2, S, B)
    assert_bits_equal(from_device(pc), oc, "ring codes")
    assert_bits_equal(from_device(ps), os_, "ring scales")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind", ["outliers", "adversarial", "tiny", "zero", "max_last"])
def test_quant_i8_tensor(dtype, kind):
    """Per-tensor INT8 quantization equals the oracle's block quantizer with
    one block spanning the tensor, from one tile to more tiles than the
    absmax pass has workgroups."""
    rng = np.random.default_rng(len(kind) * 3 + len(dtype))
    for n in (16, 3 * 4096 + 16, (1 << 18) + 48, 3 << 20, (9 << 20) + 16):   # last: > 2048 tiles
        if kind == "outliers":
            x = (rng.standard_normal(n) * 0.02).astype(np.float32)
            pos = rng.integers(0, n, max(1, n // 1000))
            x[pos] = rng.standard_normal(pos.size).astype(np.float32)
        elif kind == "adversarial":
            x = adversarial_f32(rng, n, 16)
        elif kind == "tiny":                  # scale below 2^-100 (f32) / subnormal inputs
            x = (rng.standard_normal(n) * 1e-40).astype(np.float32)
        elif kind == "zero":
            x = np.zeros(n, np.float32)
        else:                                  # the tensor's max in its very last element
            x = rng.uniform(-1, 1, n).astype(np.float32)
            x[-1] = -3.0
        xs = as_dtype(x, dtype)
        print(f"quant_i8_tensor dtype={dtype} kind={kind} n={n}", flush=True)
        codes, scale = zpq.quant_i8_tensor(to_device(xs, dtype))
        rc, rs = oracle.quant_i8(xs, dtype, n)
        assert_bits_equal(from_device(scale), rs, "scale")
        assert_bits_equal(from_device(codes), rc, "codes")


def boundary_blocks(dtype, qmax, B):
    """One block per positive finite 16-bit absmax a (sign alternating by
    block): a itself, then for each k < qmax the two values of the type on
    either side of the rounding boundary (k + 1/2) * fl32(a / qmax), clipped to
    a; zero padding.  Returns the blocks as 16-bit patterns."""
    import torch
    top = 0x7F80 if dtype == "bf16" else 0x7C00
    a_bits = np.arange(1, top, dtype=np.uint32).astype(np.uint16)
    a32 = oracle.bf16_to_f32(a_bits) if dtype == "bf16" else a_bits.view(np.float16).astype(np.float32)
    s = (a32 / np.float32(qmax)).astype(np.float32)
    k = np.arange(qmax, dtype=np.float64)
    t = (k[None, :] + 0.5) * s[:, None].astype(np.float64)          # [A, qmax]
    tt = torch.from_numpy(t.astype(np.float32).ravel())
    if dtype == "bf16":
        near = tt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        near = tt.to(torch.float16).numpy().view(np.uint16)
    near = near.reshape(t.shape).astype(np.int32)
    cand = np.stack([near - 1, near, near + 1], axis=2).reshape(len(a_bits), -1)
    cand = np.clip(cand, 0, a_bits.astype(np.int32)[:, None])          # |x| <= a
    need = 1 + cand.shape[1]
    assert need <= B, (need, B)
    blocks = np.zeros((len(a_bits), B), np.uint16)
    blocks[:, 0] = a_bits
    blocks[:, 1:need] = cand.astype(np.uint16)
    blocks[1::2] |= np.uint16(0x8000)                                    # negative blocks
    blocks[1::2][blocks[1::2] == 0x8000] = 0                             # no -0 padding
    return blocks.ravel()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rounding_boundaries_every_absmax(dtype):
    """The inputs where a quotient off by one ulp would change a code: for
    every 16-bit absmax, the values next to each rounding boundary, through
    the INT8 quantizer (qmax 127) and the INT4 quantizer (qmax 7)."""
    for qmax, B in ((127, 512), (7, 32)):
        bits = boundary_blocks(dtype, qmax, B)
        x = bits if dtype == "bf16" else bits.view(np.float16)
        print(f"rounding boundaries dtype={dtype} qmax={qmax} n={bits.size}", flush=True)
        xd = to_device(x, dtype)
        if qmax == 127:
            codes, scales = zpq.quant_i8(xd, B)
            rc, rs = oracle.quant_i8(x, dtype, B)
        else:
            codes, scales = zpq.qgz_reorder_quant_i4(xd, 1, 1, B)
            rc, rs = oracle.qgz_reorder_quant_i4(x, dtype, 1, 1, B)
        assert_bits_equal(from_device(scales), rs, "scales")
        assert_bits_equal(from_device(codes), rc, "codes")


def test_explicit_side_stream():
    """Every entry point enqueues on the stream it is given: the whole chain
    on a side stream (default priority), then one synchronize, equals the
    oracle."""
    import torch
    rng = np.random.default_rng(91)
    s = torch.cuda.Stream()
    n, B, L, N = 8 * 4096, 128, 2, 2
    x = as_dtype((rng.standard_normal(n) * 0.02).astype(np.float32), "bf16")
    xd = to_device(x, "bf16")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c8, s8 = zpq.quant_i8(xd, B, stream=s)
        y8 = zpq.dequant_i8(c8, s8, B, torch.bfloat16, stream=s)
        ct, st_ = zpq.quant_i8_tensor(xd, stream=s)
        c4, s4 = zpq.qgz_reorder_quant_i4(xd, L, N, B, stream=s)
        c5, s5 = zpq.qgz_dequant_reduce_requant_i4(c4, s4, L, n // L, B, stream=s)
        y5 = zpq.qgz_dequant_reduce_requant_i4(c5, s5, N, n // (L * N), B, out_dtype=torch.float32,
                                                divisor=4.0, stream=s)
    s.synchronize()
    rc8, rs8 = oracle.quant_i8(x, "bf16", B)
    assert_bits_equal(from_device(c8), rc8, "codes")
    assert_bits_equal(from_device(y8), oracle.dequant_i8(rc8, rs8, B, "bf16"), "dequant")
    rct, rst = oracle.quant_i8(x, "bf16", n)
    assert_bits_equal(from_device(ct), rct, "per-tensor codes")
    assert_bits_equal(from_device(st_), rst, "per-tensor scale")
    rc4, rs4 = oracle.qgz_reorder_quant_i4(x, "bf16", L, N, B)
    assert_bits_equal(from_device(c4), rc4, "INT4 codes")
    rc5, rs5 = oracle.qgz_dequant_reduce_requant_i4(rc4, rs4, L, n // L, B)
    assert_bits_equal(from_device(c5), rc5, "hop-1 codes")
    ry = oracle.qgz_dequant_reduce_requant_i4(rc5, rs5, N, n // (L * N), B, "f32", 4.0)
    assert_bits_equal(from_device(y5), ry, "hop-2 values")
