"""Pins of the oracle's block quantizer (steps O2-O6) against facts fixed
outside the oracle itself.

The ZeRO++ pages say only that weights (INT8) and gradients (INT4) are
quantized block-wise (summary page, atlas.scime.ai, "Approach" and
"Surprising findings"; index page, mlsanity.com, "Abstract (arXiv)").  The
quantizer is fixed as: s = fl32(absmax/qmax), q = clamp(rne(fl32(x/s)),
-qmax, qmax), q = 0 where s == 0, d = fl32(q*s).

Pins:
  golden     hand-derived blocks (tests/golden/quant_blocks.json)
  brute      exact rational arithmetic (Python Fractions) with an independent
             round-to-binary32, on tiny random blocks
  division   fl32(x/s) == fl32(fl64(x)/fl64(s)) (double rounding is harmless
             for division when 53 >= 2*24+2; Figueroa 1995), numpy fp64 route
  absmax     every positive finite fp16 / bf16 absmax gets code +-qmax and
             round-trips exactly in its own type (exhaustive)
  bound      |x - d| <= s/2 + (2*qmax + 1/2) * 2^-24 * s for normal s
  special    all-zero blocks, constant blocks, scale underflow
  idempotent Q(D(Q(x))) == Q(x) for codes and scales
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---- golden ------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("quant_blocks.json")["cases"], ids=lambda c: c["name"])
def test_golden_blocks(case):
    x = np.array(case["x"], np.float32)
    codes, scales = oracle.block_quant(x, case["block"], case["qmax"])
    assert codes.tolist() == case["codes"]
    assert scales.tolist() == case["scales"]
    if "packed" in case:
        assert oracle.pack_i4(codes).tolist() == case["packed"]
        assert oracle.unpack_i4(np.array(case["packed"], np.uint8)).tolist() == case["codes"]
    if case["qmax"] == 127:
        c2, s2 = oracle.quant_i8(x, "f32", case["block"])
        assert c2.tolist() == case["codes"] and s2.tolist() == case["scales"]


@pytest.mark.parametrize("case", _load("quant_blocks.json")["dequant"], ids=lambda c: c["name"])
def test_golden_dequant(case):
    y = oracle.dequant_i8(np.array(case["codes"], np.int8), np.array(case["scales"], np.float32),
                          case["block"], "f16")
    assert y.view(np.uint16).tolist() == case["f16_bits"]


# ---- brute force with exact rationals -------------------------------------------

def rn32(v: Fraction) -> Fraction:
    """Round a rational to the nearest binary32 value, ties to even (no
    overflow handling needed for the magnitudes used here)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    m = round(a / quantum)          # Fraction.__round__ ties to even
    r = m * quantum
    return r if v > 0 else -r


def brute_quant(xs, qmax):
    fx = [Fraction(float(v)) for v in xs]
    a = max(abs(v) for v in fx)
    s = rn32(a / qmax)
    if s == 0:
        return [0] * len(xs), s
    codes = []
    for v in fx:
        t = rn32(v / s)
        k = round(t)                # ties to even
        codes.append(max(-qmax, min(qmax, k)))
    return codes, s


@pytest.mark.parametrize("qmax", [127, 7])
def test_brute_force_tiny_blocks(qmax):
    rng = np.random.default_rng(100 + qmax)
    for trial in range(400):
        block = int(rng.choice([2, 4, 8]))
        kind = trial % 4
        if kind == 0:
            x = rng.standard_normal(block)
        elif kind == 1:
            x = rng.standard_normal(block) * 10.0 ** rng.uniform(-30, 30)
        elif kind == 2:
            # exact ties: x = (k + 1/2) * s for a representable s
            s = np.float32(rng.uniform(0.1, 10))
            ks = rng.integers(-qmax, qmax, size=block)
            x = (ks + 0.5) * np.float64(s)
            x[0] = qmax * np.float64(s)
        else:
            x = rng.integers(-300, 300, size=block) / 4.0
        x = x.astype(np.float32)
        codes, scales = oracle.block_quant(x, block, qmax)
        ref_codes, ref_s = brute_quant(x, qmax)
        assert codes.tolist() == ref_codes, (x, codes, ref_codes)
        assert Fraction(float(scales[0])) == ref_s


# ---- division semantics through fp64 ----------------------------------------------

def fp64_route(x, block, qmax):
    xb = x.astype(np.float64).reshape(-1, block)
    a = np.abs(xb).max(axis=1)
    s = (a / qmax).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xb / s.astype(np.float64)[:, None]).astype(np.float32)
    q = np.clip(np.rint(t), -qmax, qmax)
    q[s == 0] = 0
    return q.astype(np.int8).ravel(), s


@pytest.mark.parametrize("qmax,block", [(127, 256), (7, 128), (7, 64), (127, 32)])
def test_division_route_fp64(qmax, block):
    rng = np.random.default_rng(qmax * 1000 + block)
    parts = [
        rng.standard_normal(block * 512) * 0.02,
        rng.standard_t(3, block * 512) * 1e-3,
        (rng.standard_normal(block * 256) * np.repeat(10.0 ** rng.uniform(-2, 2, 256), block)),
        rng.standard_normal(block * 64) * 1e-30,
        rng.standard_normal(block * 64) * 1e30,
    ]
    x = np.concatenate(parts).astype(np.float32)
    codes, scales = oracle.block_quant(x, block, qmax)
    ref_codes, ref_s = fp64_route(x, block, qmax)
    assert np.array_equal(scales.view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(codes, ref_codes)


def test_division_route_all_fp16_values():
    """Every fp16 x against several scales, through the fp64 route."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    xf = h.astype(np.float32)
    for a in [np.float16(65504), np.float16(1.0), np.float16(0.0999), np.float16(6.1e-5)]:
        for qmax in (127, 7):
            keep = np.abs(xf) <= np.float32(a)
            x = xf[keep]
            x = x[: x.size - x.size % 2]
            # blocks of two: (a, x_i) so the block scale is fl(a/qmax)
            blk = np.empty(2 * x.size, np.float32)
            blk[0::2] = np.float32(a)
            blk[1::2] = x
            codes, scales = oracle.block_quant(blk, 2, qmax)
            ref_codes, ref_s = fp64_route(blk, 2, qmax)
            assert np.array_equal(codes, ref_codes)
            assert np.array_equal(scales, ref_s)


# ---- absmax element: code +-qmax, exact round trip (exhaustive) -------------------

def _positive_finite(dtype):
    bits = np.arange(1, 1 << 15, dtype=np.uint32).astype(np.uint16)
    if dtype == "f16":
        v = bits.view(np.float16)
        v = v[np.isfinite(v)]
        return v, v.astype(np.float32)
    f = oracle.bf16_to_f32(bits)
    keep = np.isfinite(f)
    return bits[keep], f[keep]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("qmax", [127, 7])
def test_absmax_code_and_roundtrip_exhaustive(dtype, qmax):
    raw, a = _positive_finite(dtype)
    for sign in (1.0, -1.0):
        blk = np.zeros(2 * a.size, np.float32)
        blk[0::2] = sign * a
        codes, scales = oracle.block_quant(blk, 2, qmax)
        assert (codes[0::2] == sign * qmax).all()
        assert (codes[1::2] == 0).all()
        d = oracle.block_dequant(codes, scales, 2)[0::2]
        back = oracle.narrow(d, dtype)
        if dtype == "f16":
            assert np.array_equal(back.view(np.uint16), (sign * raw.astype(np.float32)).astype(
                np.float16).view(np.uint16))
        else:
            ref = raw if sign > 0 else (raw | np.uint16(0x8000))
            assert np.array_equal(back, ref)


# ---- error bound -------------------------------------------------------------------

@pytest.mark.parametrize("dtype,qmax,block", [("f16", 127, 256), ("bf16", 7, 128),
                                              ("f16", 7, 64), ("f32", 7, 128)])
def test_error_bound(dtype, qmax, block):
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(block * 2000) * 0.02,
                        rng.standard_t(3, block * 2000) * 1e-3]).astype(np.float32)
    x = oracle.widen(oracle.narrow(x, dtype), dtype)
    codes, scales = oracle.block_quant(x, block, qmax)
    d = oracle.block_dequant(codes, scales, block).astype(np.float64)
    s = np.repeat(scales.astype(np.float64), block)
    normal = s >= np.finfo(np.float32).tiny
    bound = s / 2 + (2 * qmax + 0.5) * 2.0 ** -24 * s
    err = np.abs(x.astype(np.float64) - d)
    assert (err[normal] <= bound[normal]).all()
    # non-vacuous: errors close to the half step do occur
    assert (err[normal] / s[normal]).max() > 0.45


# ---- special blocks --------------------------------------------------------------

def test_all_zero_block_gives_zero_scale_codes_and_plus_zero():
    x = np.zeros(512, np.float32)
    x[256:] = -0.0
    for qmax in (127, 7):
        codes, scales = oracle.block_quant(x, 256, qmax)
        assert (codes == 0).all() and (scales == 0).all()
        d = oracle.block_dequant(codes, scales, 256)
        assert (d.view(np.uint32) == 0).all()          # +0.0, not -0.0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_constant_block(dtype):
    rng = np.random.default_rng(3)
    vals = oracle.widen(oracle.narrow(rng.standard_t(3, 300).astype(np.float32) * 1e-3, dtype),
                        dtype)
    vals = vals[vals != 0]
    for qmax in (127, 7):
        x = np.repeat(vals, 64)
        codes, scales = oracle.block_quant(x, 64, qmax)
        assert (np.abs(codes) == qmax).all()
        d = oracle.block_dequant(codes, scales, 64)
        assert np.array_equal(oracle.narrow(d, dtype), oracle.narrow(x, dtype))


def test_scale_underflow_gives_zero_codes():
    # absmax 1e-44 (fp32 subnormal): a/127 underflows to 0
    x = np.array([1e-44, -5e-45, 0, 1e-45], np.float32)
    codes, scales = oracle.block_quant(x, 4, 127)
    assert scales[0] == 0 and (codes == 0).all()
    # tiny but nonzero subnormal scale: codes stay inside [-qmax, qmax]
    x = np.array([1e-40, -7e-41, 3e-41, 0], np.float32)
    codes, scales = oracle.block_quant(x, 4, 7)
    assert scales[0] > 0 and (np.abs(codes) <= 7).all()


def test_nonfinite_input_rejected():
    x = np.array([1.0, np.inf, 0, 0], np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.block_quant(x, 4, 127)


# ---- requantization idempotence ----------------------------------------------------

@pytest.mark.parametrize("qmax,block", [(127, 256), (7, 128), (7, 64)])
def test_requant_idempotent(qmax, block):
    rng = np.random.default_rng(qmax + block)
    x = np.concatenate([rng.standard_normal(block * 3000) * 0.02,
                        rng.standard_t(3, block * 3000) * 1e-3,
                        rng.standard_normal(block * 500) * 1e20]).astype(np.float32)
    c1, s1 = oracle.block_quant(x, block, qmax)
    d = oracle.block_dequant(c1, s1, block)
    c2, s2 = oracle.block_quant(d, block, qmax)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_pack_unpack_roundtrip_all_nibble_pairs():
    q = np.array([(a, b) for a in range(-8, 8) for b in range(-8, 8)], np.int8).ravel()
    p = oracle.pack_i4(q)
    assert p.size == 256 and sorted(p.tolist()) == list(range(256))
    assert np.array_equal(oracle.unpack_i4(p), q)
