"""Pins of the oracle's conversions (steps O1 and O6).

The oracle converts between fp32 and fp16 / bf16 with code written from the
IEEE 754 binary16 definition and the bfloat16 layout.  Pinned against
independent implementations, exhaustively:
  - fp16 -> fp32 and fp32 -> fp16 against numpy's own converter (round to
    nearest even), every one of the 2^16 / 2^32 bit patterns;
  - bf16 -> fp32 against the definition (the top half of a binary32), and
    fp32 -> bf16 against the integer rounding formula
    (bits + 0x7FFF + lsb) >> 16, every one of the 2^32 bit patterns, plus a
    sample against torch's converter.
NaN payloads are outside the domain (inputs are finite); only NaN-ness is
compared for them.
"""
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

import oracle

CHUNK = 1 << 20


def _all_f32(lo):
    return np.arange(lo, lo + CHUNK, dtype=np.uint32).view(np.float32)


def _check_f16_chunk(lo):
    x = _all_f32(lo)
    got = oracle.f32_to_f16(x).view(np.uint16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    bad = (got != ref) & ~nan
    bad |= nan & ~np.isnan(got.view(np.float16))
    return int(bad.sum())


def _check_bf16_chunk(lo):
    x = _all_f32(lo)
    got = oracle.f32_to_bf16(x)
    u = x.view(np.uint32)
    # (u + 0x7FFF + lsb) >> 16 without 32-bit overflow: split off the top half
    hi = u >> 16
    lo = u & 0xFFFF
    ref = (hi + ((lo + 0x7FFF + (hi & 1)) >> 16)).astype(np.uint16)
    nan = np.isnan(x)
    bad = (got != ref) & ~nan
    bad |= nan & ~np.isnan(oracle.bf16_to_f32(got))
    return int(bad.sum())


def _run_span(args):
    fn, lo, hi = args
    return sum(fn(c) for c in range(lo, hi, CHUNK))


def _pool_sum(fn):
    spans = [(fn, lo, lo + (1 << 28)) for lo in range(0, 1 << 32, 1 << 28)]
    with ProcessPoolExecutor(max_workers=8) as ex:
        return sum(ex.map(_run_span, spans))


def test_f16_to_f32_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    got = oracle.f16_to_f32(h)
    ref = h.astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    assert np.isnan(got[nan]).all()


def test_bf16_to_f32_exhaustive():
    b = np.arange(1 << 16, dtype=np.uint32)
    got = oracle.bf16_to_f32(b.astype(np.uint16))
    assert np.array_equal(got.view(np.uint32), b << 16)


@pytest.mark.slow
def test_f32_to_f16_exhaustive():
    assert _pool_sum(_check_f16_chunk) == 0


@pytest.mark.slow
def test_f32_to_bf16_exhaustive():
    assert _pool_sum(_check_bf16_chunk) == 0


def test_f32_to_bf16_vs_torch_sample():
    import torch
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), ref)


def test_conversion_edge_values():
    # round-to-nearest-even boundaries named by the definitions
    f16_cases = {
        65504.0: 0x7BFF,            # largest finite fp16
        65519.99609375: 0x7BFF,     # just below the overflow midpoint
        65520.0: 0x7C00,            # midpoint 65504|65536 ties to even -> inf
        2.0 ** -24: 0x0001,         # smallest subnormal
        2.0 ** -25: 0x0000,         # half of it ties to even (0)
        3 * 2.0 ** -26: 0x0001,     # 0.75 of it rounds up
        2.0 ** -14: 0x0400,         # smallest normal
        1.0 + 2.0 ** -11: 0x3C00,   # tie between 1 and 1+2^-10 -> even (1)
        1.0 + 3 * 2.0 ** -11: 0x3C02,  # tie -> even (1+2^-9)
        -0.0: 0x8000,
    }
    for v, bits in f16_cases.items():
        got = int(oracle.f32_to_f16(np.array([v], np.float32)).view(np.uint16)[0])
        assert got == bits, (v, hex(got), hex(bits))
    bf16_cases = {
        1.0 + 2.0 ** -8: 0x3F80,        # tie -> even
        1.0 + 3 * 2.0 ** -8: 0x3F82,    # tie -> even (upwards)
        3.3895313892515355e38: 0x7F7F,  # largest finite bf16
        float(np.finfo(np.float32).max): 0x7F80,  # rounds past the top -> inf
        2.0 ** -133: 0x0001,            # smallest bf16 subnormal
        2.0 ** -134: 0x0000,            # half of it ties to even
    }
    for v, bits in bf16_cases.items():
        got = int(oracle.f32_to_bf16(np.array([v], np.float32))[0])
        assert got == bits, (v, hex(got), hex(bits))
