"""Pins of the oracle's qgZ steps (O7 reorder, O8 reduce, O9 average and the
two compositions) against facts fixed outside the oracle.

The ZeRO++ summary page (atlas.scime.ai, "Approach", "Surprising findings")
describes qgZ as a two-hop all-to-all (intra-node, then inter-node) of INT4
gradients, with the gradient slices reordered beforehand so each ends at the
right rank, and with dequantization before reduction; the LIT-102 anthology
record ("Key takeaways") adds that the reduction is local and in higher
precision and that it replaces reduce-scatter (also the index page's
"Abstract (arXiv)").

Pins:
  golden      hand-derived permutations and a reduction whose fp32 result
              depends on the summation order (tests/golden/qgz_examples.json)
  placement   every element tagged with (source rank, index) and pushed
              through the reorder and two simulated all-to-alls as plain
              copies: rank r must end with exactly slice r of every source
  bijection   the reorder is a permutation of slices; identity iff L or N is 1
  N=L=1       the whole qgZ path is the INT4 quantize/dequantize round trip
  K=1         hop-1 requantization of a single source returns its input
  exact sums  power-of-two scales make every partial sum exact: the result
              equals the rational sum
  bound       end-to-end error against the exact fp64 mean stays inside the
              sum of the per-step bounds
  volume      byte accounting: 3M -> 0.75M as the block grows
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "qgz_examples.json")) as f:
    QGZ = json.load(f)


def slice_order(L, N):
    """Slice id carried by each send position, via the oracle's reorder."""
    return oracle.reorder(np.arange(L * N, dtype=np.int32), L, N)


# ---- reorder -----------------------------------------------------------------------

@pytest.mark.parametrize("case", QGZ["reorder"]["cases"], ids=lambda c: f"L{c['L']}N{c['N']}")
def test_golden_reorder(case):
    assert slice_order(case["L"], case["N"]).tolist() == case["slice_at_position"]


@pytest.mark.parametrize("L,N", [(a, b) for a in range(1, 6) for b in range(1, 6)] + [(8, 4),
                                                                                      (8, 48)])
def test_reorder_is_bijection(L, N):
    p = slice_order(L, N)
    assert sorted(p.tolist()) == list(range(L * N))
    assert (np.array_equal(p, np.arange(L * N))) == (L == 1 or N == 1)


def simulate_placement(L, N, S):
    """Tags through reorder + hop-1 all-to-all + hop-2 all-to-all (copies
    only).  Returns recv[r] = array [N][L][S] of tags at rank r."""
    W = L * N
    n = W * S
    send1 = {}
    for r in range(W):
        tags = np.arange(n, dtype=np.int64) + r * n      # tag = src * n + index
        send1[r] = oracle.reorder(tags, L, N)
    # hop 1: rank (m, j) gets chunk j of every local rank (m, i), source-major
    chunk1 = n // L
    recv1 = {}
    for m in range(N):
        for j in range(L):
            recv1[m * L + j] = np.stack([send1[m * L + i][j * chunk1:(j + 1) * chunk1]
                                         for i in range(L)])          # [L][N*S]
    # hop 2: rank (m', j) gets position m' of the chunk held by rank (m, j)
    recv2 = {}
    for mp in range(N):
        for j in range(L):
            recv2[mp * L + j] = np.stack([recv1[m * L + j][:, mp * S:(mp + 1) * S]
                                          for m in range(N)])         # [N][L][S]
    return recv2, n


@pytest.mark.parametrize("L,N,S", [(2, 2, 3), (3, 2, 2), (2, 3, 4), (4, 3, 1), (1, 5, 2),
                                   (5, 1, 2), (3, 4, 2)])
def test_final_owner_simulation(L, N, S):
    recv, n = simulate_placement(L, N, S)
    for r, got in recv.items():
        for m in range(N):
            for i in range(L):
                src = m * L + i
                expect = src * n + r * S + np.arange(S)
                assert np.array_equal(got[m, i], expect), (r, m, i)


# ---- reduction order: golden ------------------------------------------------------

def _golden_reduce_inputs():
    g = QGZ["reduce_order"]
    codes = np.array(g["codes_by_source"], np.uint8).ravel()
    scales = np.array(g["scales_by_source"], np.float32).ravel()
    return g, codes, scales


def test_golden_reduce_order_float():
    g, codes, scales = _golden_reduce_inputs()
    for key, div in (("divisor_1", 1.0), ("divisor_4", 4.0)):
        y = oracle.qgz_dequant_reduce_requant_i4(codes, scales, g["K"], g["chunk"], g["block"],
                                                 "f32", div)
        assert y.tolist() == g["float_out"][key]
    yb = oracle.qgz_dequant_reduce_requant_i4(codes, scales, g["K"], g["chunk"], g["block"],
                                              "bf16", 1.0)
    assert yb.tolist() == g["bf16_bits_divisor_1"]


def test_golden_reduce_order_requant():
    g, codes, scales = _golden_reduce_inputs()
    oc, os_ = oracle.qgz_dequant_reduce_requant_i4(codes, scales, g["K"], g["chunk"], g["block"])
    assert oc.tolist() == g["i4_out"]["codes"]
    assert os_.view(np.uint32).tolist() == g["i4_out"]["scales_bits"]


# ---- special cases -------------------------------------------------------------------

@pytest.mark.parametrize("dtype,block", [("bf16", 128), ("f16", 64), ("f32", 32)])
def test_qgz_single_rank_is_roundtrip(dtype, block):
    """N = L = 1: reorder is the identity, hop 1 and hop 2 have one source and
    the divisor is 1, so the path is INT4 quantize then dequantize."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(block * 300) * 1e-3).astype(np.float32)
    g = oracle.narrow(x, dtype)
    c, s = oracle.qgz_reorder_quant_i4(g, dtype, 1, 1, block)
    # hop 1 with K = 1: requantization returns the input (idempotence)
    c1, s1 = oracle.qgz_dequant_reduce_requant_i4(c, s, 1, x.size, block)
    assert np.array_equal(c1, c) and np.array_equal(s1.view(np.uint32), s.view(np.uint32))
    y = oracle.qgz_dequant_reduce_requant_i4(c1, s1, 1, x.size, block, "f32", 1.0)
    q, s_ref = oracle.block_quant(oracle.widen(g, dtype), block, 7)
    d_ref = oracle.block_dequant(q, s_ref, block)
    assert np.array_equal(y.view(np.uint32), d_ref.view(np.uint32))


def test_exact_sums_equal_rational_sum():
    """Scales that are powers of two and few sources: every partial sum is
    exactly representable, so the fp32 result equals the rational sum."""
    rng = np.random.default_rng(9)
    K, chunk, block = 6, 256, 64
    q = rng.integers(-7, 8, size=(K, chunk)).astype(np.int8)
    s = (2.0 ** rng.integers(-4, 5, size=(K, chunk // block))).astype(np.float32)
    codes = np.concatenate([oracle.pack_i4(q[i]) for i in range(K)])
    y = oracle.qgz_dequant_reduce_requant_i4(codes, s.ravel(), K, chunk, block, "f32", 1.0)
    for e in range(chunk):
        exact = sum(Fraction(int(q[i, e])) * Fraction(float(s[i, e // block])) for i in range(K))
        assert Fraction(float(y[e])) == exact
    # with a power-of-two divisor the average is exact too
    y8 = oracle.qgz_dequant_reduce_requant_i4(codes, s.ravel(), K, chunk, block, "f32", 8.0)
    assert np.array_equal(y8, y / np.float32(8))


def test_source_order_matters_and_is_rank_order():
    """Permuting the sources changes the fp32 result in general; the oracle's
    result equals a left-to-right fp32 sum in the given order."""
    rng = np.random.default_rng(21)
    K, chunk, block = 8, 4096, 128
    x = (rng.standard_normal((K, chunk)) * 10.0 ** rng.uniform(-3, 3, (K, 1))).astype(np.float32)
    qs = [oracle.block_quant(x[i], block, 7) for i in range(K)]
    codes = np.concatenate([oracle.pack_i4(c) for c, _ in qs])
    scales = np.concatenate([s for _, s in qs])
    y = oracle.qgz_dequant_reduce_requant_i4(codes, scales, K, chunk, block, "f32", 1.0)
    acc = np.zeros(chunk, np.float32)
    for c, s in qs:
        acc = acc + oracle.block_dequant(c, s, block)      # numpy fp32 adds
    assert np.array_equal(y.view(np.uint32), acc.view(np.uint32))
    perm = rng.permutation(K)
    codes_p = np.concatenate([oracle.pack_i4(qs[i][0]) for i in perm])
    scales_p = np.concatenate([qs[i][1] for i in perm])
    y_p = oracle.qgz_dequant_reduce_requant_i4(codes_p, scales_p, K, chunk, block, "f32", 1.0)
    assert not np.array_equal(y, y_p)


# ---- end-to-end error bound against the exact mean ---------------------------------------

def p4(s, qmax=7):
    return s / 2 + (2 * qmax + 0.5) * 2.0 ** -24 * s


@pytest.mark.parametrize("L,N,S,block", [(2, 2, 256, 64), (4, 2, 128, 128), (2, 3, 256, 32)])
def test_end_to_end_error_bound(L, N, S, block):
    W = L * N
    n = W * S
    u = 2.0 ** -24
    rng = np.random.default_rng(L * 100 + N)
    # slice s of every rank is centred on 10*s, so a misplaced slice shows up
    centre = np.repeat(np.arange(W) * 10.0, S)
    grads = [(centre + rng.standard_normal(n)).astype(np.float32) for _ in range(W)]
    send1 = [oracle.qgz_reorder_quant_i4(g, "f32", L, N, block) for g in grads]
    c1 = n // L
    send2, recv_scales1 = {}, {}
    for m in range(N):
        for j in range(L):
            codes = np.concatenate([send1[m * L + i][0][j * c1 // 2:(j + 1) * c1 // 2]
                                    for i in range(L)])
            scales = np.concatenate([send1[m * L + i][1][j * c1 // block:(j + 1) * c1 // block]
                                     for i in range(L)])
            send2[m * L + j] = oracle.qgz_dequant_reduce_requant_i4(codes, scales, L, c1, block)
            recv_scales1[m * L + j] = scales.reshape(L, -1)
    exact = np.mean(np.stack(grads).astype(np.float64), axis=0)
    for mp in range(N):
        for j in range(L):
            r = mp * L + j
            codes = np.concatenate([send2[m * L + j][0][mp * S // 2:(mp + 1) * S // 2]
                                    for m in range(N)])
            scales = np.concatenate([send2[m * L + j][1][mp * S // block:(mp + 1) * S // block]
                                     for m in range(N)])
            y = oracle.qgz_dequant_reduce_requant_i4(codes, scales, N, S, block, "f32", float(W))
            # per-element bound
            bound = np.zeros(S)
            sum_abs2 = np.zeros(S)
            for m in range(N):
                s1 = recv_scales1[m * L + j][:, mp * S // block:(mp + 1) * S // block]
                src = np.repeat(p4(s1.astype(np.float64)), block, axis=1)      # [L][S]
                s2 = np.repeat(scales[m * S // block:(m + 1) * S // block].astype(np.float64),
                               block)
                # |terms| of the hop-1 sum are at most |x| + its error
                hop1_terms = np.abs(np.stack([grads[m * L + i][r * S:(r + 1) * S]
                                              for i in range(L)]).astype(np.float64)) + src
                bound += src.sum(0) + (L - 1) * u * hop1_terms.sum(0) * 1.01 + p4(s2)
                sum_abs2 += hop1_terms.sum(0) + p4(s2)
            bound += (N - 1) * u * sum_abs2 * 1.01
            bound = bound / W + u * np.abs(y.astype(np.float64)) * 1.01
            err = np.abs(y.astype(np.float64) - exact[r * S:(r + 1) * S])
            assert (err <= bound).all(), (r, (err / bound).max())


# ---- byte accounting -----------------------------------------------------------------

def test_volume_accounting():
    v = QGZ["volume"]
    fp16 = 2.0
    # ZeRO-3: fwd all-gather, bwd all-gather, reduce-scatter, each M fp16 values
    assert 3 * fp16 / fp16 == v["zero3_units"]

    def ratio(bits, block):           # bytes per element incl. one fp32 scale per block
        return (bits / 8 + 4.0 / block) / fp16

    # qwZ INT8 forward + hpZ (no cross-node backward gather) + qgZ INT4
    for block in (1 << 20,):
        assert abs(ratio(8, block) + 0 + ratio(4, block) - v["zeropp_units"]) < 1e-5
    assert abs(ratio(8, 256) - 0.5078125) < 1e-12
    assert abs(ratio(4, 128) - 0.265625) < 1e-12
    assert abs(ratio(4, 64) - 0.28125) < 1e-12
    # sizes the oracle actually produces
    x = np.zeros(1024, np.float16)
    c, s = oracle.quant_i8(x, "f16", 256)
    assert c.nbytes + s.nbytes == ratio(8, 256) * x.nbytes
    c4, s4 = oracle.qgz_reorder_quant_i4(x, "f16", 2, 2, 128)
    assert c4.nbytes + s4.nbytes == ratio(4, 128) * x.nbytes


# ---- averaging division and output rounding -----------------------------------------

@pytest.mark.parametrize("divisor", [3.0, 6.0, 384.0, 7.5, 1e-3])
def test_average_division_fp64_route(divisor):
    """fl32(acc / W) == fl32(fl64(acc) / fl64(W)) (division double-rounding
    is harmless), with acc taken from the same call at divisor 1; fp16 / bf16
    outputs are the fp32 average rounded to nearest even (numpy / torch)."""
    import torch
    rng = np.random.default_rng(int(divisor * 1000))
    K, chunk, block = 5, 8192, 64
    x = (rng.standard_t(3, (K, chunk)) * 1e-3).astype(np.float32)
    qs = [oracle.block_quant(x[i], block, 7) for i in range(K)]
    codes = np.concatenate([oracle.pack_i4(c) for c, _ in qs])
    scales = np.concatenate([s for _, s in qs])
    acc = oracle.qgz_dequant_reduce_requant_i4(codes, scales, K, chunk, block, "f32", 1.0)
    y = oracle.qgz_dequant_reduce_requant_i4(codes, scales, K, chunk, block, "f32", divisor)
    ref = (acc.astype(np.float64) / np.float64(np.float32(divisor))).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
    y16 = oracle.qgz_dequant_reduce_requant_i4(codes, scales, K, chunk, block, "f16", divisor)
    assert np.array_equal(y16.view(np.uint16), ref.astype(np.float16).view(np.uint16))
    yb = oracle.qgz_dequant_reduce_requant_i4(codes, scales, K, chunk, block, "bf16", divisor)
    refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, refb)
