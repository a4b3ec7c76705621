"""The range-split oracle runs that the full-size GPU parity tests use
(send positions on their own, hop-receive chunks in block ranges, on host
threads) equal the oracle's whole-tensor compositions, bit for bit."""
import numpy as np
import pytest

import oracle
import synth
import oracle_ranges as cfg


@pytest.mark.parametrize("L,N,B,per", [(2, 3, 64, 4096), (8, 4, 128, 2048), (3, 5, 32, 640)])
def test_ranges_equal_whole(L, N, B, per):
    W = L * N
    n = W * per
    g = synth.qgz_fused(0, n)
    c1, s1 = cfg.oracle_send(g, "f16", L, N, B)
    w1 = oracle.qgz_reorder_quant_i4(g, "f16", L, N, B)
    assert np.array_equal(c1, w1[0]) and np.array_equal(s1.view(np.uint32), w1[1].view(np.uint32))
    chunk = n // L
    c2, s2 = cfg.oracle_receive(c1, s1, L, chunk, B, 4)
    w2 = oracle.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)
    assert np.array_equal(c2, w2[0]) and np.array_equal(s2.view(np.uint32), w2[1].view(np.uint32))
    S = n // W
    y = cfg.oracle_receive(c2, s2, N, S, B, 2, "f16", float(W))
    w3 = oracle.qgz_dequant_reduce_requant_i4(c2, s2, N, S, B, "f16", float(W))
    assert np.array_equal(y.view(np.uint16), w3.view(np.uint16))
