"""Pins for the CPU oracle: facts fixed by the QAM-W paper and by mathematics.

Each test checks the oracle against something other than itself: values the
paper prints, closed forms, invariants (Lemma 1), library routines for special
cases (scipy's Hadamard matrix, cKDTree, numpy's float16, torch's bfloat16),
or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.spatial

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _signs(d_in, seed=7):
    bits = _rng(seed).integers(0, 2**32, size=(d_in + 31) // 32, dtype=np.uint64).astype(np.uint32)
    j = np.arange(d_in)
    eps = np.where((bits[j >> 5] >> (j & 31).astype(np.uint32)) & 1, -1.0, 1.0)
    return bits, eps


def _rot_independent(u, eps, b):
    """y = blockdiag(H_b) (eps . u) built from scipy's Sylvester Hadamard matrix."""
    H = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    v = (u * eps).reshape(u.shape[0], -1, b)
    return np.einsum("ik,rtk->rti", H, v).reshape(u.shape)


# ----------------------------------------------------------------------------- rotation (section 3.3, Lemma 1)

@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024])
def test_hadamard_is_orthonormal(orc, b):
    H = orc.hadamard(b)
    err = np.abs(H @ H.T - np.eye(b)).max()
    if int(math.log2(b)) % 2 == 0:  # 1/sqrt(b) is a power of two: exact
        assert err == 0.0
    else:
        assert err <= 1e-15


@pytest.mark.parametrize("b", [2, 8, 64, 128, 256, 1024])
def test_hadamard_matches_scipy(orc, b):
    H = orc.hadamard(b)
    np.testing.assert_array_equal(np.sign(H), scipy.linalg.hadamard(b))
    assert np.all(np.abs(np.abs(H) - 1.0 / math.sqrt(b)) <= 1e-17)


@pytest.mark.parametrize("b,d_in", [(64, 512), (128, 1024), (256, 512), (2, 10), (1024, 2048)])
def test_rotation_is_isometry_and_matches_independent(orc, b, d_in):
    rng = _rng(b)
    w = (rng.standard_normal((9, d_in)) * 0.02).astype(np.float32)
    w[3] *= 1e3
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    bits, eps = _signs(d_in, b)
    y, r, st = orc.front_end(w, s, bits, b)
    assert st == 0
    a = w.astype(np.float64) * s.astype(np.float64)
    np.testing.assert_allclose(r, np.linalg.norm(a, axis=1), rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, rtol=0, atol=2e-14)  # Lemma 1
    y_ref = _rot_independent(a / np.linalg.norm(a, axis=1, keepdims=True), eps, b)
    np.testing.assert_allclose(y, y_ref, rtol=0, atol=1e-14)


def test_default_block_rule_printed_instances(orc):
    g = json.load(open(os.path.join(GOLDEN, "paper_values.json")))["default_block"]["cases"]
    for d_in, b in g:
        assert orc.default_block(d_in) == b
    assert orc.default_block(4096) == 1024 and orc.default_block(5120) == 1024
    assert orc.default_block(13824) == 512 and orc.default_block(11008) == 256 and orc.default_block(6) == 2


# ----------------------------------------------------------------------------- bitrate (section 3.7 eq. 3)

def test_bpw_printed_instances(orc):
    g = json.load(open(os.path.join(GOLDEN, "paper_values.json")))
    for d_in, bits, printed in g["bpw"]["cases"]:
        assert round(orc.bpw(d_in, bits), 2) == printed
    cb = g["codebook_bytes"]
    assert (1 << cb["bits"]) * 2 * 4 <= cb["max_bytes"]


@pytest.mark.parametrize("d_out,d_in,bits", [(4096, 4096, 11), (11008, 4096, 11), (4096, 11008, 11),
                                             (5120, 5120, 11), (13824, 5120, 7), (256, 512, 8)])
def test_stored_bytes_equal_eq3(orc, d_out, d_in, bits):
    stride = orc.row_stride(d_in, bits)
    assert stride % 16 == 0 and stride * 8 >= d_in // 2 * bits
    total_bits = (stride * d_out + 2 * d_out) * 8
    assert total_bits / (d_out * d_in) == pytest.approx(orc.bpw(d_in, bits), rel=0, abs=1e-12)


# ----------------------------------------------------------------------------- packing (section 3.1 step 6)

def test_pack_hand_worked_examples(orc):
    for line in open(os.path.join(GOLDEN, "pack_examples.txt")):
        if line.startswith("#") or not line.strip():
            continue
        bits, d_in, idx, hexrow = line.split()
        bits, d_in = int(bits), int(d_in)
        idx = np.array([int(x) for x in idx.split(",")], dtype=np.int32)
        row = orc.pack_row(idx, bits, d_in)
        assert row.tobytes().hex() == hexrow
        np.testing.assert_array_equal(orc.unpack_row(row, bits, d_in), idx)


@pytest.mark.parametrize("bits", list(range(1, 17)))
def test_pack_roundtrip(orc, bits):
    d_in = 2 * 173
    idx = _rng(bits).integers(0, 1 << bits, size=d_in // 2).astype(np.int32)
    row = orc.pack_row(idx, bits, d_in)
    np.testing.assert_array_equal(orc.unpack_row(row, bits, d_in), idx)
    used = (d_in // 2 * bits + 7) // 8
    assert not row[used:].any()
    # the stream read as one little-endian integer holds index k at bit k*bits
    big = int.from_bytes(row.tobytes(), "little")
    for k in (0, 1, 57, d_in // 2 - 1):
        assert (big >> (k * bits)) & ((1 << bits) - 1) == idx[k]


# ----------------------------------------------------------------------------- number formats

def _interesting_f32(n=200000):
    rng = _rng(3)
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    extra = np.array([0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e-8, 5.96e-8, 2.98e-8, 6.1035e-05,
                      1.0009765625, 1.00048828125, 1.000732421875, 3.0e38, -2.5, np.inf, -np.inf],
                     dtype=np.float32)
    scaled = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-9, 6, 50000)).astype(np.float32)
    return np.concatenate([f, extra, scaled])


def test_f16_rounding_matches_numpy(orc):
    xs = _interesting_f32()
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([orc.f16_from_f32(float(x)) for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    h = h[np.isfinite(h.view(np.float16))]
    back = np.array([orc.f32_from_f16(int(v)) for v in h], dtype=np.float32)
    np.testing.assert_array_equal(back, h.view(np.float16).astype(np.float32))


def test_bf16_rounding_matches_torch(orc):
    import torch
    xs = _interesting_f32()
    ref = torch.from_numpy(xs.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_from_f32(float(x)) for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------------------- nearest codeword (section 3.6)

def test_nearest_matches_kdtree_away_from_ties(orc):
    rng = _rng(11)
    cb = rng.standard_normal((2048, 2)).astype(np.float32)
    p = (rng.standard_normal((200000, 2)) * 1.3).astype(np.float32)
    idx, d = orc.nearest(p, cb)
    tree = scipy.spatial.cKDTree(cb.astype(np.float64))
    dd, ii = tree.query(p.astype(np.float64), k=2)
    clear = (dd[:, 1] ** 2 - dd[:, 0] ** 2) > 1e-5 * dd[:, 0] ** 2 + 1e-12
    assert clear.mean() > 0.999
    np.testing.assert_array_equal(idx[clear], ii[clear, 0])
    np.testing.assert_allclose(d[clear], dd[clear, 0] ** 2, rtol=1e-5, atol=1e-12)


def test_nearest_exact_ties_go_to_lowest_index(orc):
    cb = np.array([[1.0, 1.0], [-1.0, 1.0], [-1.0, -1.0], [1.0, -1.0], [1.0, 1.0]], dtype=np.float32)
    probes = np.array([[0.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [0.0, -1.0], [1.0, 0.0], [1.0, 1.0], [0.5, 0.5]],
                      dtype=np.float32)
    idx, _ = orc.nearest(probes, cb)
    np.testing.assert_array_equal(idx, [0, 0, 1, 2, 0, 0, 0])


def test_nearest_every_codeword_maps_to_itself(orc):
    rng = _rng(12)
    cb = rng.standard_normal((4096, 2)).astype(np.float32)
    idx, d = orc.nearest(cb, cb)
    np.testing.assert_array_equal(idx, np.arange(4096))
    assert not d.any()


# ----------------------------------------------------------------------------- Lloyd (section 3.6 eq. 2)

@pytest.fixture(scope="module")
def gauss_pts(synth):
    return synth.points(0x51414D5700000000, 4, 1 << 16)


def test_lloyd_k1_is_sample_mean(orc, gauss_pts):
    # Two identical starting codewords: every point ties and goes to index 0, so one iteration gives
    # the K=1 quantizer (centroid = sample mean) and cell 1, being empty, keeps its value.
    pts = gauss_pts.astype(np.float64)
    cbk, ek, stk = orc.lloyd(gauss_pts, 1, 1, init=np.array([[0.3, -0.2], [0.3, -0.2]], np.float32))
    assert stk == 0
    mean = pts.mean(axis=0)
    np.testing.assert_allclose(cbk[0], mean.astype(np.float32), rtol=0, atol=1e-7)
    np.testing.assert_array_equal(cbk[1], np.array([0.3, -0.2], np.float32))
    # distortion of the K=1 quantizer at the centroid is the total variance (~2 for the unit circular Gaussian)
    _, e2, _ = orc.lloyd(gauss_pts, 1, 1, init=np.stack([cbk[0], cbk[0]]))
    mse = e2[0] / 2**32 / len(pts)
    c0 = cbk[0].astype(np.float64)
    ref = ((gauss_pts.astype(np.float32) - cbk[0]).astype(np.float32) ** 2).astype(np.float64).sum(axis=1).mean()
    assert mse == pytest.approx(ref, rel=1e-6)
    assert mse == pytest.approx(((pts - c0) ** 2).sum(axis=1).mean(), rel=1e-5)
    assert mse == pytest.approx(2.0, abs=0.05)


def test_lloyd_k2_closed_form(orc, gauss_pts):
    cb, e, st = orc.lloyd(gauss_pts, 1, 30)
    r = np.linalg.norm(cb.astype(np.float64), axis=1)
    np.testing.assert_allclose(r, math.sqrt(2 / math.pi), atol=0.012)
    np.testing.assert_allclose(cb[0], -cb[1], atol=0.02)
    assert e[-1] / 2**32 / len(gauss_pts) == pytest.approx(2 - 2 / math.pi, abs=0.012)


def test_lloyd_centroid_condition_and_assignment(orc, gauss_pts):
    bits, t = 6, 8
    prev, _, _ = orc.lloyd(gauss_pts, bits, t - 1)
    cur, e, _ = orc.lloyd(gauss_pts, bits, t)
    idx, _ = orc.nearest(gauss_pts, prev)
    tree = scipy.spatial.cKDTree(prev.astype(np.float64))
    dd, ii = tree.query(gauss_pts.astype(np.float64), k=2)
    clear = (dd[:, 1] ** 2 - dd[:, 0] ** 2) > 1e-5 * dd[:, 0] ** 2
    np.testing.assert_array_equal(idx[clear], ii[clear, 0])
    pts = gauss_pts.astype(np.float64)
    for j in range(1 << bits):
        m = idx == j
        if m.any():
            ref = pts[m].mean(axis=0).astype(np.float32)
            assert np.all(np.abs(cur[j] - ref) <= np.spacing(np.abs(ref)) * 1.0)
        else:
            np.testing.assert_array_equal(cur[j], prev[j])


def test_lloyd_mse_non_increasing_and_resume(orc, gauss_pts):
    cb, e, _ = orc.lloyd(gauss_pts, 7, 12)
    mse = e.astype(np.float64)
    assert np.all(mse[1:] <= mse[:-1] * (1 + 1e-6))
    a, ea, _ = orc.lloyd(gauss_pts, 7, 5)
    b, eb, _ = orc.lloyd(gauss_pts, 7, 7, init=a)
    np.testing.assert_array_equal(b, cb)
    np.testing.assert_array_equal(np.concatenate([ea, eb]), e)


@pytest.mark.parametrize("bits", [7, 8])
def test_lloyd_high_rate_band(orc, gauss_pts, bits):
    K = 1 << bits
    _, e, _ = orc.lloyd(gauss_pts, bits, 40)
    mse = e[-1] / 2**32 / len(gauss_pts)
    zador = 2 * (5 / (36 * math.sqrt(3))) * 8 * math.pi / K  # 2 * G_hex * (2 pi e^{..}) high-rate estimate
    assert 0.8 * zador <= mse <= 1.2 * zador


def test_lloyd_point_range_flag(orc):
    pts = np.zeros((1024, 2), np.float32)
    pts[:, 0] = np.linspace(-1, 1, 1024)
    pts[5, 1] = 1e6
    _, _, st = orc.lloyd(pts, 4, 1)
    assert st & 8


# ----------------------------------------------------------------------------- calibration (section 3.4 eq. 1)

def test_calibration_isotropic_gaussian_rows(orc):
    rng = _rng(21)
    d_in, n = 2048, 1024
    w = rng.standard_normal((n, d_in)).astype(np.float32)
    s = np.ones(d_in, np.float32)
    bits, _ = _signs(d_in)
    sigma, st = orc.calibrate(w, s, bits, 128)
    z = sigma.astype(np.float64) * math.sqrt(d_in)
    assert abs(z.mean() - 1.0) < 0.005
    assert np.abs(z - 1.0).max() < 0.1


def test_calibration_recovers_planted_per_pair_sigma(orc):
    """Rows whose rotated pairs are circular Gaussians with a planted sigma_k per pair."""
    rng = _rng(22)
    d_in, n, b = 1024, 1024, 64
    kk = np.arange(d_in // 2)
    sig = 0.5 + (kk % 7) * 0.25 + (kk // 100) * 0.1
    sig = sig / math.sqrt(2 * (sig**2).sum())  # unit expected row norm
    y = rng.standard_normal((n, d_in)) * np.repeat(sig, 2)
    bits, eps = _signs(d_in, 3)
    H = scipy.linalg.hadamard(b) / math.sqrt(b)
    u = np.einsum("ik,rtk->rti", H.T, y.reshape(n, -1, b)).reshape(n, d_in) * eps  # u = R_fwd^T y
    sigma, _ = orc.calibrate(u.astype(np.float32), np.ones(d_in, np.float32), bits, b)
    ratio = sigma / sig
    assert np.abs(ratio - 1).max() < 0.1
    assert abs(ratio.mean() - 1) < 0.01
    assert np.corrcoef(sigma, sig)[0, 1] > 0.99


def test_calibration_skips_zero_rows_and_falls_back(orc):
    rng = _rng(23)
    d_in = 256
    w = rng.standard_normal((40, d_in)).astype(np.float32)
    s = np.ones(d_in, np.float32)
    bits, _ = _signs(d_in)
    s1, _ = orc.calibrate(w, s, bits, 64)
    w2 = np.concatenate([w[:10], np.zeros((7, d_in), np.float32), w[10:]])
    s2, _ = orc.calibrate(w2, s, bits, 64)
    np.testing.assert_array_equal(s1, s2)
    s3, _ = orc.calibrate(np.zeros((5, d_in), np.float32), s, bits, 64)
    np.testing.assert_array_equal(s3, np.float32(1 / math.sqrt(d_in)))


# ----------------------------------------------------------------------------- encode / decode (sections 3.1, 3.2)

def _tiny_problem(seed=31, d_out=12, d_in=64, b=16, bits=6):
    rng = _rng(seed)
    w = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    w[4] = 0.0
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    cb = rng.standard_normal((1 << bits, 2)).astype(np.float32)
    bits_w, eps = _signs(d_in, seed)
    return w, s, cb, bits_w, eps, b, bits


def test_encode_is_bruteforce_nearest_of_rotated_pairs(orc):
    """Independent recomputation: scipy Hadamard rotation, fp64 distances, argmin."""
    w, s, cb, sbits, eps, b, bits = _tiny_problem()
    sigma, _ = orc.calibrate(w, s, sbits, b)
    enc = orc.encode(w, s, sbits, b, cb, bits, sigma, want_p=True)
    a = w.astype(np.float64) * s
    r = np.linalg.norm(a, axis=1)
    nz = r > 0
    y = np.zeros_like(a)
    y[nz] = _rot_independent(a[nz] / r[nz, None], eps, b)
    p = (y.reshape(len(w), -1, 2) / sigma[None, :, None].astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(enc["p"].reshape(p.shape)[nz], p[nz])
    d = ((p[:, :, None, :].astype(np.float64) - cb[None, None].astype(np.float64)) ** 2).sum(-1)
    srt = np.sort(d, axis=-1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-5 * srt[..., 0]
    ref_idx = d.argmin(-1)
    assert clear[nz].mean() > 0.99
    np.testing.assert_array_equal(enc["idx"][nz][clear[nz]], ref_idx[nz][clear[nz]])
    # zero row: norm 0, all indices 0
    assert enc["norm"][4] == 0 and not enc["idx"][4].any()
    # stored norm is f16(fl32(r))
    np.testing.assert_array_equal(enc["norm"][nz], r[nz].astype(np.float32).astype(np.float16).view(np.uint16))


def test_decode_inverts_rotation_to_codewords(orc):
    """Re-rotating the decoded row recovers sigma_k * c[idx_k] (spec check on tiny inputs)."""
    w, s, cb, sbits, eps, b, bits = _tiny_problem(41)
    sigma, _ = orc.calibrate(w, s, sbits, b)
    enc = orc.encode(w, s, sbits, b, cb, bits, sigma)
    dec = orc.decode(enc["codes"], enc["norm"], w.shape[1], sigma, cb, bits, s, sbits, b, want_f64=True)
    rn = enc["norm"].view(np.float16).astype(np.float64)
    nz = rn > 0
    assert not dec["f64"][~nz].any() and not dec["bf16"][~nz].any()
    back = _rot_independent(dec["f64"][nz] * s / rn[nz, None], eps, b).reshape(nz.sum(), -1, 2)
    expect = sigma[None, :, None].astype(np.float64) * cb[enc["idx"][nz]].astype(np.float64)
    np.testing.assert_allclose(back, expect, rtol=0, atol=1e-13)
    # float and bf16 outputs are roundings of the double result
    np.testing.assert_array_equal(dec["f32"], dec["f64"].astype(np.float32))


def test_parseval_identity(orc, synth):
    """Lemma 1: the weighted reconstruction error equals the error of the rotated pairs."""
    c = synth.config(0)
    m = c.matrices[0]
    w = m.weights(0, 64)
    s = m.channel_scale()
    sbits = orc.sign_mask(0x51414D57, m.d_in)
    pts = synth.points(c.seed, 4, 1 << 12)
    cb, _, _ = orc.lloyd(pts, 8, 5)
    sigma, _ = orc.calibrate(w, s, sbits, c.block)
    enc = orc.encode(w, s, sbits, c.block, cb, 8, sigma)
    dec = orc.decode(enc["codes"], enc["norm"], m.d_in, sigma, cb, 8, s, sbits, c.block, want_f64=True)
    y, r, _ = orc.front_end(w, s, sbits, c.block)
    rn = enc["norm"].view(np.float16).astype(np.float64)
    lhs = (((w.astype(np.float64) - dec["f64"]) * s) ** 2).sum(axis=1)
    q = sigma[None, :, None].astype(np.float64) * cb[enc["idx"]].astype(np.float64)
    rhs = ((r[:, None] * y - rn[:, None] * q.reshape(len(w), -1)) ** 2).sum(axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10)


def test_reconstruction_improves_with_codebook_size(orc, synth):
    c = synth.config(1)
    m = c.matrices[0]
    w = m.weights(0, 48)
    s = m.channel_scale()
    sbits = orc.sign_mask(0x51414D57, m.d_in)
    pts = synth.points(c.seed, 4, 1 << 14)
    errs, dist = [], []
    for bits in (4, 6, 8):
        cb, e, _ = orc.lloyd(pts, bits, 15)
        dist.append(e[-1] / 2**32 / len(pts))
        sigma, _ = orc.calibrate(w, s, sbits, c.block)
        enc = orc.encode(w, s, sbits, c.block, cb, bits, sigma, want_idx=False)
        dec = orc.decode(enc["codes"], enc["norm"], m.d_in, sigma, cb, bits, s, sbits, c.block)
        wf = synth.bf16_bits_to_f32(w).astype(np.float64)
        errs.append(np.linalg.norm((dec["f32"] - wf) * s) / np.linalg.norm(wf * s))
    assert errs[0] > errs[1] > errs[2]
    # pairs are near unit circular Gaussians (E|p|^2 = 2), so the relative error is about sqrt(D/2)
    for err, d in zip(errs, dist):
        assert 0.7 < err / math.sqrt(d / 2) < 1.5


def test_status_flags(orc):
    d_in = 64
    rng = _rng(51)
    w = (rng.standard_normal((4, d_in))).astype(np.float32)
    s = np.ones(d_in, np.float32)
    sbits, _ = _signs(d_in)
    cb = rng.standard_normal((16, 2)).astype(np.float32)
    sig = np.ones(d_in // 2, np.float32)
    assert orc.encode(w, s, sbits, 16, cb, 4, sig)["status"] == 0
    w2 = w.copy()
    w2[1, 3] = np.nan
    assert orc.encode(w2, s, sbits, 16, cb, 4, sig)["status"] & 1
    s2 = s.copy()
    s2[5] = 0.0
    assert orc.encode(w, s2, sbits, 16, cb, 4, sig)["status"] & 2
    w3 = w.copy()
    w3[2] *= 1e4
    assert orc.encode(w3, s, sbits, 16, cb, 4, sig)["status"] == 4
