"""The pages' structural argument for qgZ, measured with the oracle: a
compressed reduce-scatter requantizes the running sum at every hop, so its
error grows with the number of ranks, while qgZ's two-hop all-to-all
quantizes every value twice whatever the world size (LIT-102 anthology
record, Key takeaways; ZeRO++ summary page, Approach)."""
import numpy as np
import pytest

import oracle
import synth

S, B = 1 << 12, 128


def study(W):
    g = np.stack([synth.blockvar_normal(40, 1000 + r, S, B, 1e-3, -2.0, 2.0) for r in range(W)])
    exact = g.astype(np.float64).mean(0)
    q = [oracle.qgz_reorder_quant_i4(g[r], "f32", 1, 1, B) for r in range(W)]
    pc, ps = q[0]
    for r in range(1, W):
        pc, ps = oracle.qgz_dequant_reduce_requant_i4(np.concatenate([pc, q[r][0]]),
                                                      np.concatenate([ps, q[r][1]]), 2, S, B)
    ring = oracle.qgz_dequant_reduce_requant_i4(pc, ps, 1, S, B, "f32", float(W))
    L = min(W, 8)
    N = W // L
    hop1 = [oracle.qgz_dequant_reduce_requant_i4(
        np.concatenate([q[m * L + i][0] for i in range(L)]),
        np.concatenate([q[m * L + i][1] for i in range(L)]), L, S, B) for m in range(N)]
    qgz = oracle.qgz_dequant_reduce_requant_i4(np.concatenate([h[0] for h in hop1]),
                                               np.concatenate([h[1] for h in hop1]), N, S, B,
                                               "f32", float(W))
    scale = np.sqrt(np.mean(exact ** 2))

    def err(y):
        return np.sqrt(np.mean((y.astype(np.float64) - exact) ** 2)) / scale
    return err(qgz), err(ring)


def test_ring_error_compounds_qgz_does_not():
    q8, r8 = study(8)
    q64, r64 = study(64)
    assert r8 > q8 and r64 > r8 * 1.5            # the ring's error grows with its hops
    assert r64 > 2.5 * q64                       # ... and ends far above qgZ's
    assert abs(q64 - q8) < 0.1 * q8              # qgZ's stays flat


def test_single_hop_cases_agree():
    q2, r2 = study(2)
    assert q2 == pytest.approx(r2, rel=0, abs=0)  # W = 2: both are one hop over two sources
