"""Pins for the oracle's activation-aware channel scale (reading R11: s_j = r_j^alpha, r_j the RMS of
input channel j over the calibration activations) and for the output-error identity that motivates
it, ||X dW^T||_F^2 = Tr(dW M dW^T) with M = X^T X (the layer-output trace identity the pages state).

The scale is checked against closed forms (constant channels, alpha = 0 and 1, the scaling law
r(cX) = |c| r(X)), a dead channel, and numpy's own RMS; the identity is checked on a codec error dW
from the oracle's encoder and decoder, and the point of the scale -- that it lowers the output
error on activations with strong channels -- on a seeded case.
"""
import numpy as np
import pytest


def test_closed_forms(orc):
    T, d = 37, 12
    x = np.tile(np.arange(1, d + 1, dtype=np.float32) * np.float32(0.5), (T, 1))
    x[::2] *= -1                                     # the sign does not matter
    s0, r = orc.act_scale(x, 0.0)
    np.testing.assert_allclose(r, 0.5 * np.arange(1, d + 1), rtol=1e-15)
    np.testing.assert_array_equal(s0, np.ones(d, np.float32))
    s1, _ = orc.act_scale(x, 1.0)
    np.testing.assert_array_equal(s1, (0.5 * np.arange(1, d + 1)).astype(np.float32))
    s3, _ = orc.act_scale(x, 0.3)
    np.testing.assert_array_equal(s3, np.power(0.5 * np.arange(1, d + 1), 0.3).astype(np.float32))


def test_rms_matches_numpy_and_scales(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 64)) * np.exp(rng.standard_normal(64))).astype(np.float32)
    x[:, 5] = 0                                      # a dead channel
    s, r = orc.act_scale(x, 0.3)
    np.testing.assert_allclose(r, np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0)), rtol=1e-14)
    assert s[5] == 1.0 and r[5] == 0.0
    _, r2 = orc.act_scale(4 * x, 0.3)                # powers of two: exact
    np.testing.assert_array_equal(r2, 4 * r)


def test_trace_identity_and_the_point_of_the_scale(orc):
    """||X dW^T||^2 = Tr(dW X^T X dW^T) for the codec's own error, and activation-aware scales lower
    that error when a few channels carry most of the activation energy."""
    rng = np.random.default_rng(11)
    T, d_out, d_in, block, bits = 256, 48, 256, 64, 7
    rho = np.exp(0.5 * rng.standard_normal(d_in))
    rho[rng.choice(d_in, 4, replace=False)] *= 30     # strong channels
    x = (rng.standard_normal((T, d_in)) * rho).astype(np.float32)
    w = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    sb = rng.integers(0, 2**32, size=d_in // 32, dtype=np.uint64).astype(np.uint32)
    cb, _, _ = orc.lloyd(rng.standard_normal((1 << 14, 2)).astype(np.float32), bits, 20)

    def out_err(s):
        sig, _ = orc.calibrate(w, s, sb, block)
        e = orc.encode(w, s, sb, block, cb, bits, sig)
        wh = orc.decode(e["codes"], e["norm"], d_in, sig, cb, bits, s, sb, block, want_f64=True)["f64"]
        dw = wh - w.astype(np.float64)
        xd = x.astype(np.float64)
        lhs = np.sum((xd @ dw.T) ** 2)
        rhs = np.trace(dw @ (xd.T @ xd) @ dw.T)
        assert abs(lhs - rhs) <= 1e-9 * lhs
        return lhs

    s_aw, _ = orc.act_scale(x, 0.3)
    e_plain, e_aw = out_err(np.ones(d_in, np.float32)), out_err(s_aw)
    assert e_aw < 0.8 * e_plain, (e_aw, e_plain)
