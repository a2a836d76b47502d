"""Pins for the oracle's scalar (d = 1) ablation (paper section 2, reading R10): each coordinate of
the scaled pair is coded with the Lloyd-Max quantizer of the standard normal density.

Checked against what the mathematics fixes: one bit gives the half-normal means +-sqrt(2/pi); every
level is the conditional mean of its cell by numerical integration (scipy's quad, not the oracle's
closed form); the levels are symmetric; a plain Lloyd on normal samples lands on them; the index is
the brute-force nearest level; nearest-codeword search over the product table agrees with the two
scalar indices; and the paper's point that joint 2D coding beats scalar coding at equal bits holds
on circular Gaussian pairs.
"""
import math

import numpy as np
import pytest
import scipy.integrate


def _pdf(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def test_one_bit_is_the_half_normal_mean(orc):
    levels, thr = orc.gauss_lloyd_max(1)
    np.testing.assert_allclose(levels, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-15)
    assert thr[0] == 0.0


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6])
def test_levels_are_centroids_and_symmetric(orc, b):
    levels, thr = orc.gauss_lloyd_max(b)
    L = 1 << b
    assert np.all(np.diff(levels) > 0)
    np.testing.assert_allclose(levels, -levels[::-1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(thr, 0.5 * (levels[:-1] + levels[1:]), rtol=0, atol=1e-15)
    edges = [-np.inf] + list(thr) + [np.inf]
    tol = 1e-9 if b <= 4 else 1e-6
    for i in range(L):
        a, c = edges[i], edges[i + 1]
        mass = scipy.integrate.quad(_pdf, a, c, epsabs=1e-15, epsrel=1e-13)[0]
        mom = scipy.integrate.quad(lambda x: x * _pdf(x), a, c, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(levels[i] - mom / mass) < tol * max(1.0, abs(levels[i])), (i, levels[i], mom / mass)


@pytest.mark.parametrize("b", [2, 3])
def test_levels_match_lloyd_on_samples(orc, b):
    rng = np.random.default_rng(8)
    z = rng.standard_normal(1 << 19)
    x = np.sort(np.concatenate([z, -z]))   # a symmetric sample: no drift from its mean
    csum = np.concatenate([[0.0], np.cumsum(x)])
    L = 1 << b
    lv = np.quantile(x, (np.arange(L) + 0.5) / L)
    for _ in range(5000):
        t = 0.5 * (lv[:-1] + lv[1:])
        e = np.concatenate([[0], np.searchsorted(x, t), [len(x)]])
        lv = (csum[e[1:]] - csum[e[:-1]]) / (e[1:] - e[:-1])
    levels, _ = orc.gauss_lloyd_max(b)
    np.testing.assert_allclose(levels, lv, rtol=0, atol=5e-3)


@pytest.mark.parametrize("b", [1, 3, 4, 6])
def test_index_is_the_nearest_level(orc, b):
    levels, thr = orc.gauss_lloyd_max(b)
    rng = np.random.default_rng(b)
    p = (rng.standard_normal(3000) * 1.4).astype(np.float32)
    p[:4] = [0.0, -0.0, 1e-30, -7.5]
    got = orc.scalar_index(p, b, thr)
    d = np.abs(p.astype(np.float64)[:, None] - levels[None, :])
    far = np.min(np.abs(p.astype(np.float64)[:, None] - thr[None, :]), axis=1) > 1e-12
    np.testing.assert_array_equal(got[far], np.argmin(d, axis=1)[far])
    assert got[0] == got[1] == (1 << b) // 2 - 1 + (1 if thr[(1 << b) // 2 - 1] < 0 else 0)   # 0 sits on the middle threshold: lower level


@pytest.mark.parametrize("b", [2, 4])
def test_product_table_search_is_the_pair_of_scalar_indices(orc, b):
    levels, thr = orc.gauss_lloyd_max(b)
    cb = orc.scalar_table(b, levels)
    L = 1 << b
    np.testing.assert_array_equal(cb[:, 0], np.tile(levels.astype(np.float32), L))
    np.testing.assert_array_equal(cb[:, 1], np.repeat(levels.astype(np.float32), L))
    rng = np.random.default_rng(40 + b)
    p = rng.standard_normal((4000, 2)).astype(np.float32)
    ix, iy = orc.scalar_index(p[:, 0], b, thr), orc.scalar_index(p[:, 1], b, thr)
    nn, _ = orc.nearest(p, cb)
    far = (np.min(np.abs(p[:, :1].astype(np.float64) - thr[None, :]), axis=1) > 1e-6) & \
          (np.min(np.abs(p[:, 1:].astype(np.float64) - thr[None, :]), axis=1) > 1e-6)
    np.testing.assert_array_equal(nn[far], (ix + L * iy)[far])


def test_encode_scalar_uses_the_scalar_indices(orc):
    rng = np.random.default_rng(12)
    d_in, block, b = 256, 64, 4
    w = (rng.standard_normal((5, d_in)) * 0.02).astype(np.float32)
    w[1] = 0
    s = (np.sqrt(np.abs(rng.standard_normal(d_in))) + 0.1).astype(np.float32)
    sb = rng.integers(0, 2**32, size=d_in // 32, dtype=np.uint64).astype(np.uint32)
    sig, _ = orc.calibrate(w, s, sb, block)
    levels, thr = orc.gauss_lloyd_max(b)
    e = orc.encode_scalar(w, s, sb, block, b, thr, sig, want_p=True)
    pp = e["p"].reshape(5, d_in // 2, 2)
    want = orc.scalar_index(pp[..., 0], b, thr).reshape(5, -1) + (orc.scalar_index(pp[..., 1], b, thr).reshape(5, -1) << b)
    want[1] = 0
    np.testing.assert_array_equal(e["idx"], want)
    qe = orc.encode(w, s, sb, block, orc.scalar_table(b, levels), 2 * b, sig)
    np.testing.assert_array_equal(qe["norm"], e["norm"])


def test_joint_2d_beats_scalar_at_equal_bits(orc):
    """Sections 1-2: joint 2D coding recovers the pair structure scalar codebooks discard; at 8 bits
    per pair a K = 256 Lloyd codebook has lower MSE on circular Gaussian pairs than 4 + 4 scalar
    Lloyd-Max."""
    rng = np.random.default_rng(13)
    cb, _, _ = orc.lloyd(rng.standard_normal((1 << 14, 2)).astype(np.float32), 8, 30)
    test = rng.standard_normal((1 << 14, 2)).astype(np.float32)
    qi, _ = orc.nearest(test, cb)
    mse_2d = np.mean(np.sum((test - cb[qi]) ** 2, axis=1))
    levels, thr = orc.gauss_lloyd_max(4)
    table = orc.scalar_table(4, levels)
    si = orc.scalar_index(test[:, 0], 4, thr) + 16 * orc.scalar_index(test[:, 1], 4, thr)
    mse_1d = np.mean(np.sum((test - table[si]) ** 2, axis=1))
    assert mse_2d < mse_1d, (mse_2d, mse_1d)


def test_index_ties_go_to_the_lower_level(orc):
    thr = np.array([-1.0, 0.0, 0.5], dtype=np.float64)   # exactly representable in fp32
    p = np.array([-1.0, 0.0, 0.5, 0.5000001, -1.0000001, 3.0], dtype=np.float32)
    np.testing.assert_array_equal(orc.scalar_index(p, 2, thr), [0, 1, 2, 3, 0, 3])
