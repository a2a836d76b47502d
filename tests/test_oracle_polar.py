"""Pins for the oracle's polar baseline (paper section 3.5, reading R8).

The magnitude quantizer is checked against the Rayleigh mean (closed form), against numerical
integration of the centroid condition (scipy's quad, not the oracle's closed-form integrals),
and against a Lloyd run on samples of the density.  The index is checked against brute force
over every level and every phase bin.  The table is checked by its polar coordinates.  The
comparison the paper reports (joint 2D coding beats polar coding at equal bits) is checked on
circular Gaussian pairs.
"""
import math

import numpy as np
import pytest
import scipy.integrate


def _rayleigh_pdf(r):
    return r * math.exp(-0.5 * r * r)


def test_one_level_is_the_rayleigh_mean(orc):
    levels, thr = orc.rayleigh_lloyd_max(0)
    assert thr.size == 0
    assert abs(levels[0] - math.sqrt(math.pi / 2)) < 1e-14


@pytest.mark.parametrize("ba", [1, 2, 3, 4, 5, 6])
def test_levels_are_centroids_of_their_cells(orc, ba):
    """Lloyd-Max conditions: every level is the mean of the density over its cell (integrated
    numerically here), and every threshold is the midpoint of its two levels.  The iteration stops
    after at most 10000 rounds (reading R8), where 64 levels are still settling at the 1e-7 level."""
    levels, thr = orc.rayleigh_lloyd_max(ba)
    na = 1 << ba
    assert np.all(np.diff(levels) > 0)
    np.testing.assert_allclose(thr, 0.5 * (levels[:-1] + levels[1:]), rtol=0, atol=1e-15)
    edges = [0.0] + list(thr) + [np.inf]
    for i in range(na):
        a, b = edges[i], edges[i + 1]
        mass = scipy.integrate.quad(_rayleigh_pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        mom = scipy.integrate.quad(lambda r: r * _rayleigh_pdf(r), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        tol = 1e-9 if ba <= 4 else 1e-6
        assert abs(levels[i] - mom / mass) < tol * levels[i], (i, levels[i], mom / mass)


@pytest.mark.parametrize("ba", [2, 4])
def test_levels_match_lloyd_on_samples(orc, ba):
    """A plain 1D Lloyd on 2^20 Rayleigh samples lands on the same levels, within the sampling
    noise (largest for the sparse top cell)."""
    rng = np.random.default_rng(5)
    r = np.sort(np.sqrt(-2.0 * np.log1p(-rng.random(1 << 20))))
    csum = np.concatenate([[0.0], np.cumsum(r)])
    na = 1 << ba
    lv = np.quantile(r, (np.arange(na) + 0.5) / na)
    for _ in range(20000):
        t = 0.5 * (lv[:-1] + lv[1:])
        e = np.concatenate([[0], np.searchsorted(r, t), [len(r)]])
        lv = (csum[e[1:]] - csum[e[:-1]]) / (e[1:] - e[:-1])
    levels, _ = orc.rayleigh_lloyd_max(ba)
    np.testing.assert_allclose(levels, lv, rtol=5e-3, atol=0)


@pytest.mark.parametrize("ba,bp", [(5, 6), (4, 4), (1, 1), (3, 7)])
def test_polar_index_is_nearest_level_and_nearest_phase(orc, ba, bp):
    rng = np.random.default_rng(ba * 16 + bp)
    p = (rng.standard_normal((4000, 2)) * 1.3).astype(np.float32)
    p[:11] = [[0, 0], [1, 0], [0, 1], [-1, 0], [0, -1], [1e-30, -1e-30], [5, 5], [-3, 1e-6],
              [-0.0, 0.0], [-0.0, -0.0], [0.0, -0.0]]   # a zero pair has phase 0 whatever its signs
    levels, thr = orc.rayleigh_lloyd_max(ba)
    idx = orc.polar_index(p, ba, bp, thr)
    na, n_ph = 1 << ba, 1 << bp
    ia, ip = idx % na, idx // na
    r = np.hypot(p[:, 0].astype(np.float64), p[:, 1].astype(np.float64))
    # magnitude: the nearest level (ties to the lower one); skip points within 1e-12 of a threshold
    d = np.abs(r[:, None] - levels[None, :])
    near = np.argmin(d, axis=1)
    far = np.ones(len(r), bool) if thr.size == 0 else np.min(np.abs(r[:, None] - thr[None, :]), axis=1) > 1e-12
    assert far.sum() > 3900
    np.testing.assert_array_equal(ia[far], near[far])
    # phase: the bin centre 2 pi j / Np nearest in angle; skip points within 1e-12 rad of a bin edge
    th = np.arctan2(p[:, 1].astype(np.float64), p[:, 0].astype(np.float64))
    centres = 2 * np.pi * np.arange(n_ph) / n_ph
    ang = np.abs((th[:, None] - centres[None, :] + np.pi) % (2 * np.pi) - np.pi)
    jn = np.argmin(ang, axis=1)
    edge = np.abs(((th * n_ph / (2 * np.pi) + 0.5) % 1.0) - 0.0)
    ok = (np.minimum(edge, 1 - edge) > 1e-12) & (r > 0)
    np.testing.assert_array_equal(ip[ok], jn[ok])
    assert np.all(ip[r == 0] == 0)


def test_polar_table_layout(orc):
    ba, bp = 5, 6
    levels, _ = orc.rayleigh_lloyd_max(ba)
    cb = orc.polar_table(ba, bp, levels).astype(np.float64)
    na, n_ph = 1 << ba, 1 << bp
    assert cb.shape == (na * n_ph, 2)
    k = np.arange(na * n_ph)
    ia, ip = k % na, k // na
    np.testing.assert_allclose(np.hypot(cb[:, 0], cb[:, 1]), levels[ia], rtol=2e-7)
    th = np.arctan2(cb[:, 1], cb[:, 0])
    want = (2 * np.pi * ip / n_ph + np.pi) % (2 * np.pi) - np.pi
    dth = np.abs((th - want + np.pi) % (2 * np.pi) - np.pi)
    assert dth.max() < 1e-6


def test_encode_polar_uses_the_polar_index(orc):
    rng = np.random.default_rng(9)
    d_in, block, ba, bp = 256, 64, 5, 6
    w = (rng.standard_normal((6, d_in)) * 0.02).astype(np.float32)
    w[2] = 0
    s = (np.sqrt(np.abs(rng.standard_normal(d_in))) + 0.1).astype(np.float32)
    sb = rng.integers(0, 2**32, size=d_in // 32, dtype=np.uint64).astype(np.uint32)
    sig, _ = orc.calibrate(w, s, sb, block)
    levels, thr = orc.rayleigh_lloyd_max(ba)
    e = orc.encode_polar(w, s, sb, block, ba, bp, thr, sig, want_p=True)
    idx = orc.polar_index(e["p"].reshape(-1, 2), ba, bp, thr).reshape(6, d_in // 2)
    idx[2] = 0   # a zero row encodes every index as 0
    np.testing.assert_array_equal(e["idx"], idx)
    for i in range(6):
        np.testing.assert_array_equal(orc.unpack_row(e["codes"][i], ba + bp, d_in), e["idx"][i])
    # the QAM-W encoder's front end and norms are shared
    qe = orc.encode(w, s, sb, block, orc.polar_table(ba, bp, levels), ba + bp, sig, want_p=True)
    np.testing.assert_array_equal(qe["norm"], e["norm"])
    np.testing.assert_array_equal(qe["p"], e["p"])


def test_joint_2d_beats_polar_at_equal_bits(orc):
    """Section 5 / abstract: joint 2D coding beats polar (magnitude x phase) coding at equal bits.
    On circular Gaussian pairs, a K = 256 Lloyd codebook has lower mean squared error than the
    4 + 4 bit polar quantizer."""
    rng = np.random.default_rng(11)
    train = rng.standard_normal((1 << 14, 2)).astype(np.float32)
    cb, _, _ = orc.lloyd(train, 8, 30)
    test = rng.standard_normal((1 << 14, 2)).astype(np.float32)
    qi, _ = orc.nearest(test, cb)
    mse_2d = np.mean(np.sum((test - cb[qi]) ** 2, axis=1))
    levels, thr = orc.rayleigh_lloyd_max(4)
    table = orc.polar_table(4, 4, levels)
    pi_ = orc.polar_index(test, 4, 4, thr)
    mse_polar = np.mean(np.sum((test - table[pi_]) ** 2, axis=1))
    assert mse_2d < mse_polar, (mse_2d, mse_polar)
