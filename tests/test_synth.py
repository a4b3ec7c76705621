"""The seeded input generator: deterministic, thread-count independent, and
drawing the workloads' stated distributions and structure."""
import numpy as np

import synth


def test_counter_based_and_thread_independent(monkeypatch):
    monkeypatch.setenv("ZPQ_SYNTH_THREADS", "1")
    a = synth.student_t3(9, 0, 200_000, 1e-3)
    b = synth.normal(9, 1, 200_000, 0.0, 2.0)
    monkeypatch.setenv("ZPQ_SYNTH_THREADS", "7")
    assert np.array_equal(a, synth.student_t3(9, 0, 200_000, 1e-3))
    assert np.array_equal(b, synth.normal(9, 1, 200_000, 0.0, 2.0))
    # any slice can be regenerated on its own
    assert np.array_equal(a[123_456:150_000], synth.student_t3(9, 0, 26_544, 1e-3, 123_456))
    # streams and seeds are independent
    assert not np.array_equal(b, synth.normal(9, 2, 200_000, 0.0, 2.0))
    assert not np.array_equal(b, synth.normal(10, 1, 200_000, 0.0, 2.0))


def test_distribution_moments():
    z = synth.normal(1, 0, 1 << 21, 0.0, 0.02)
    assert abs(z.mean()) < 1e-4 and abs(z.std() / 0.02 - 1) < 3e-3
    t = synth.student_t3(1, 0, 1 << 21, 1.0).astype(np.float64)
    # Student t, 3 dof: median of |t| is 0.7649, P(|t| > 3.182) = 0.05
    assert abs(np.median(np.abs(t)) - 0.7649) < 0.005
    assert abs(np.mean(np.abs(t) > 3.182) - 0.05) < 0.002
    v = synth.blockvar_normal(1, 0, 1 << 21, 128, 1.0, -2.0, 2.0).reshape(-1, 128)
    logvar = np.log10(v.astype(np.float64).var(axis=1))
    assert logvar.min() > -2.6 and logvar.max() < 2.6          # ~U(-2, 2) plus noise
    assert abs(np.median(logvar)) < 0.1


def test_qwz_roundtrip_structure():
    x = synth.qwz_roundtrip()
    c = synth.QWZ_ROUNDTRIP
    assert x.dtype == np.float16 and x.size == c["n"]
    blocks = x.reshape(-1, c["block"])
    zero = np.nonzero((blocks == 0).all(axis=1))[0]
    assert zero.tolist() == [c["zero_block"]]
    # outliers present: P(|N(0,1)| > 0.2) = 0.84 of 1049; N(0, 0.02) never reaches 10 sigma
    assert 800 < (np.abs(x) > 0.2).sum() <= 1049
    assert synth.select(1, 1, c["n"], c["outliers"]).size == c["outliers"]


def test_qgz_fused_special_blocks():
    const_ids, vals, zero_ids = synth.qgz_fused_special_blocks()
    nb = synth.QGZ_FUSED["n"] // synth.QGZ_FUSED["block"]
    assert nb == 16_515_072
    assert const_ids.size == round(0.01 * nb) and zero_ids.size == round(0.005 * nb)
    assert np.intersect1d(const_ids, zero_ids).size == 0
    special = (const_ids, vals, zero_ids)
    b = int(const_ids[0])
    x = synth.qgz_fused(b * 64, 64 * 4, special).reshape(-1, 64)
    assert (x[0] == x[0, 0]).all()
    z = int(zero_ids[0])
    y = synth.qgz_fused(z * 64, 64, special)
    assert (y == 0).all()


def test_workload_sizes():
    assert synth.QWZ_LAYER["n"] == 805_306_368 == 12 * 8192 ** 2
    assert synth.QWZ_LAYER["n"] % (16 * 256) == 0
    assert synth.QGZ_FUSED["n"] == 1_056_964_608
    assert synth.QGZ_FUSED["n"] % (8 * 48 * 64) == 0
    assert synth.QGZ_HOP1["n"] % (8 * 4 * 128) == 0
