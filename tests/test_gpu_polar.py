"""GPU parity of the polar baseline (paper section 3.5) against the CPU oracle.

Covers the Rayleigh Lloyd-Max codebook (levels, thresholds, product table), the polar index of
crafted and random pairs (axes, diagonals, signed zeros, infinities, NaN, points on the magnitude
thresholds and on the phase-bin edges), the polar encoder on ragged and full-size matrices, the
decode of polar codes, and the bad-threshold flag.

Comparison rules:
  * levels and thresholds: within 1e-10 relative.  The oracle takes the first moment of a cell as
    a difference of erf values, which loses about 1e-12 relative in the sparse top cell of 256
    levels; the slowly converging iteration carries such differences along (a CPU run of the
    kernel's erfc form lands 5e-12 from the oracle at 256 levels, 4e-14 at 32).
  * table entries: within two fp32 ulps of the radius (the angle is exact on the GPU and
    rounded to double in the oracle, and the level differs as above).
  * indices: equal, except at near-ties: a differing magnitude index must be the neighbouring
    level with fl64(px^2 + py^2) within 1e-6 relative of the threshold between them, and a
    differing phase index the neighbouring bin with theta Np / (2 pi) + 1/2 within 1e-6 Np of an
    integer (both bounds cover a one-ulp difference of the fp32 pair, and exact ties).
"""
import math

import numpy as np
import pytest
import torch

from helpers import (DEV, assert_bf16_within_1ulp, gpu_decode, log, t, unpack_rows, w_tensor)

pytestmark = pytest.mark.gpu

CODEBOOKS = [(1, 1), (2, 3), (3, 7), (4, 4), (5, 6), (6, 6), (7, 5), (8, 4)]


def check_polar(gidx, ridx, p, ba, bp, thr):
    """Polar indices equal except at near-ties; returns the number of differing pairs."""
    gidx = np.asarray(gidx).ravel()
    ridx = np.asarray(ridx).ravel()
    mism = gidx != ridx
    n = int(mism.sum())
    if n == 0:
        return 0
    na, n_ph = 1 << ba, 1 << bp
    pm = np.asarray(p, np.float32).reshape(-1, 2)[mism].astype(np.float64)
    g, r = gidx[mism], ridx[mism]
    ga, gp, ra, rp = g % na, g // na, r % na, r // na
    r2 = pm[:, 0] * pm[:, 0] + pm[:, 1] * pm[:, 1]
    t2 = np.asarray(thr, np.float64) ** 2
    da = ga != ra
    if da.any():
        assert np.all(np.abs(ga[da] - ra[da]) == 1), (ga[da][:5], ra[da][:5])
        lo = np.minimum(ga[da], ra[da])
        gap = np.abs(r2[da] - t2[lo])
        assert np.all(gap <= 1e-6 * t2[lo]), "magnitude index differs away from a threshold: %s" % gap[:5]
    dp = gp != rp
    if dp.any():
        step = (gp[dp] - rp[dp]) % n_ph
        assert np.all((step == 1) | (step == n_ph - 1)), (gp[dp][:5], rp[dp][:5])
        v = np.arctan2(pm[dp, 1], pm[dp, 0]) * n_ph / (2 * np.pi) + 0.5
        gap = np.abs(v - np.round(v))
        assert np.all(gap <= 1e-6 * n_ph), "phase index differs away from a bin edge: %s" % gap[:5]
    return n


@pytest.mark.parametrize("ba,bp", CODEBOOKS, ids=["%d+%d" % c for c in CODEBOOKS])
def test_polar_codebook_matches_oracle(q, orc, ba, bp):
    log("polar codebook ba=%d bp=%d" % (ba, bp))
    lv, thr, tab = q.polar_codebook(ba, bp)
    torch.cuda.synchronize()
    lv, thr, tab = lv.cpu().numpy(), thr.cpu().numpy(), tab.cpu().numpy()
    lv_r, thr_r = orc.rayleigh_lloyd_max(ba)
    tab_r = orc.polar_table(ba, bp, lv_r)
    rel = np.abs(lv - lv_r) / lv_r
    log("  levels: max rel diff %.3g" % rel.max())
    assert rel.max() <= 1e-10
    np.testing.assert_allclose(thr, thr_r, rtol=1e-10, atol=0)
    np.testing.assert_array_equal(thr, 0.5 * (lv[:-1] + lv[1:]))   # exactly the midpoints
    assert np.all(np.diff(lv) > 0)
    ia = np.arange(tab.shape[0]) % (1 << ba)
    atol = (lv_r[ia] * 2.0 ** -22)[:, None]
    assert np.all(np.abs(tab.astype(np.float64) - tab_r) <= atol)


def _crafted_points(ba, bp, thr, seed):
    rng = np.random.default_rng(seed)
    n_ph = 1 << bp
    pts = [rng.standard_normal((3000, 2)) * 1.3, rng.standard_normal((500, 2)) * 1e-3,
           rng.standard_normal((500, 2)) * 40.0]
    ax = np.array([[1, 0], [0, 1], [-1, 0], [0, -1], [1, 1], [-1, 1], [-1, -1], [1, -1], [2.5, 2.5], [-0.5, 0.5]])
    pts.append(ax)
    zeros = np.array([[0.0, 0.0], [-0.0, 0.0], [0.0, -0.0], [-0.0, -0.0], [0.0, 3.0], [-0.0, 3.0], [-0.0, -3.0],
                      [3.0, -0.0], [-3.0, -0.0], [-3.0, 0.0]])
    pts.append(zeros)
    inf = np.inf
    specials = np.array([[inf, 0], [-inf, 0], [0, inf], [0, -inf], [inf, inf], [-inf, inf], [inf, -inf],
                         [-inf, -inf], [inf, 5.0], [-2.0, -inf], [np.nan, 1.0], [1.0, np.nan], [np.nan, np.nan],
                         [3e38, 3e38], [1e-40, 0.0], [-1e-45, 1e-45]])
    pts.append(specials)
    # denormal and near-overflow pairs: the ratio behind the phase guess must survive both
    pts.append(rng.standard_normal((200, 2)) * 1e-39)
    pts.append(rng.standard_normal((200, 2)) * 1e37)
    # on (fl32 of) each magnitude threshold along random directions
    if thr.size:
        ang = rng.uniform(-np.pi, np.pi, thr.size)
        pts.append(np.stack([thr * np.cos(ang), thr * np.sin(ang)], 1))
        pts.append(np.stack([thr.astype(np.float32).astype(np.float64), np.zeros(thr.size)], 1))
    # on (fl32 of) each phase-bin edge, and just either side of it
    k = np.arange(n_ph)
    e = (2 * k + 1) * np.pi / n_ph
    rad = rng.uniform(0.2, 3.0, n_ph)
    for d in (0.0, 1e-6, -1e-6):
        pts.append(np.stack([rad * np.cos(e + d), rad * np.sin(e + d)], 1))
    return np.concatenate(pts).astype(np.float32)


def test_polar_index_beyond_one_grid(q, orc):
    """More pairs than one launch covers (at most 2048 workgroups of 256 threads, then a grid
    stride): 2048 * 256 + 12345 Gaussian pairs, ba = 5, bp = 6."""
    _, thr = orc.rayleigh_lloyd_max(5)
    n = 2048 * 256 + 12345
    p = np.random.default_rng(77).standard_normal((n, 2)).astype(np.float32)
    log("polar index %d points" % n)
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    got = q.polar_index(t(p), 5, 6, t(thr.astype(np.float64)), status=st).cpu().numpy()
    ref = orc.polar_index(p, 5, 6, thr)
    assert int(st.item()) == 0
    flips = check_polar(got, ref, p, 5, 6, thr)
    log("  %d near-tie flips" % flips)


@pytest.mark.parametrize("ba,bp", [(1, 1), (1, 2), (2, 2), (3, 3), (4, 4), (5, 6), (8, 4), (3, 9), (1, 11)],
                         ids=lambda v: str(v))
def test_polar_index_matches_oracle(q, orc, ba, bp):
    _, thr = orc.rayleigh_lloyd_max(ba)
    p = _crafted_points(ba, bp, thr, 17 * ba + bp)
    log("polar index ba=%d bp=%d: %d points" % (ba, bp, len(p)))
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    got = q.polar_index(t(p), ba, bp, t(thr.astype(np.float64)), status=st).cpu().numpy()
    ref = orc.polar_index(p, ba, bp, thr)
    assert int(st.item()) == 0
    flips = check_polar(got, ref, p, ba, bp, thr)
    log("  %d near-tie flips" % flips)
    # the unambiguous points agree exactly: zero pairs, NaN, the axes
    na = 1 << ba
    for xy in ([0.0, 0.0], [-0.0, -0.0], [-0.0, 0.0], [np.nan, 1.0]):
        i = np.where((p[:, 0].view(np.uint32) == np.float32(xy[0]).view(np.uint32)) &
                     (p[:, 1].view(np.uint32) == np.float32(xy[1]).view(np.uint32)))[0]
        assert i.size and np.all(got[i] == 0), (xy, got[i])
    if bp >= 2:
        i = np.where((p[:, 0] == 0) & (p[:, 1] == 3.0))[0]
        assert np.all(got[i] // na == (1 << bp) // 4)


def _problem(seed, d_out, d_in, block, dtype="bf16"):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(5, size=(d_out, d_in)) * 0.015).astype(np.float32)
    w[:, rng.choice(d_in, size=max(1, d_in // 100), replace=False)] *= 10
    w[min(1, d_out - 1)] = 0                         # a zero row
    if d_out > 3:
        w[2] = 0
        w[2, 5] = 0.3                                # one non-zero: exact zeros in the other blocks
    if d_out > 4:
        w[3, block:] = 0                             # only the first block non-zero
    if dtype == "bf16":
        w = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    seed = int(rng.integers(0, 2**62))   # sign-mask seed
    return w, s, seed


ENCODE_CASES = {
    "4096_b128_5+6": (40, 4096, 128, 5, 6, "bf16", False, None),
    "768_b256_4+4_ragged": (33, 768, 256, 4, 4, "bf16", False, None),
    "1024_b1024_3+7": (12, 1024, 1024, 3, 7, "bf16", False, None),
    "512_b64_1+1": (17, 512, 64, 1, 1, "bf16", False, None),
    "256_b32_2+2_fp32": (20, 256, 32, 2, 2, "fp32", False, None),
    "2048_b512_8+4_given_sigma": (9, 2048, 512, 8, 4, "bf16", True, None),
    "1536_b512_6+5_padded_ld": (11, 1536, 512, 6, 5, "bf16", False, 1536 + 24),
    "256_b64_3+3_many_rows": (1300, 256, 64, 3, 3, "bf16", False, None),
    "13824_b512_5+6": (6, 13824, 512, 5, 6, "bf16", False, None),
}


def _encode_polar_case(q, orc, case):
    d_out, d_in, block, ba, bp, dtype, given, ld = ENCODE_CASES[case]
    w, s, seed = _problem(d_out * 13 + d_in + ba, d_out, d_in, block, dtype)
    sb = orc.sign_mask(seed, d_in)
    _, thr = orc.rayleigh_lloyd_max(ba)
    if given:
        sig = (np.abs(np.random.default_rng(d_in).standard_normal(d_in // 2)) * 0.05 + 0.01).astype(np.float32)
    else:
        sig, st_c = orc.calibrate(w[:1024], s, sb, block)
        assert st_c == 0
    ref = orc.encode_polar(w, s, sb, block, ba, bp, thr, sig, want_idx=True, want_p=True)
    log("encode_polar %s" % case)
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = q.encode_polar(w_tensor(w, ld), ba, bp, t(thr.astype(np.float64)), scale=t(s), sign_seed=seed,
                         block=block, sigma=t(sig) if given else None, status=st)
    torch.cuda.synchronize()
    codes = out["codes"].cpu().numpy()
    norm = out["norm"].cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(out["sigma"].cpu().numpy(), sig)
    np.testing.assert_array_equal(norm, ref["norm"])
    assert int(st.item()) == ref["status"] == 0
    gidx = unpack_rows(orc, codes, ba + bp, d_in)
    flips = check_polar(gidx, ref["idx"], ref["p"], ba, bp, thr)
    log("  %d near-tie flips" % flips)
    same = np.all(gidx == ref["idx"], axis=1)   # rows without a tie: the packed bytes agree too
    np.testing.assert_array_equal(codes[same], ref["codes"][same])
    return codes, norm, sig, s, seed, sb, ref, thr


@pytest.mark.parametrize("case", list(ENCODE_CASES), ids=list(ENCODE_CASES))
def test_encode_polar_matches_oracle(q, orc, case):
    _encode_polar_case(q, orc, case)


def test_polar_encode_decode_roundtrip(q, orc):
    """GPU polar codes decoded by qamw_decode with the GPU's table, against the oracle's decode
    of its own codes with its own table."""
    codes, norm, sig, s, seed, sb, ref, thr = _encode_polar_case(q, orc, "4096_b128_5+6")
    ba, bp, d_in, block = 5, 6, 4096, 128
    lv, _, tab = q.polar_codebook(ba, bp)
    lv_r, _ = orc.rayleigh_lloyd_max(ba)
    tab_r = orc.polar_table(ba, bp, lv_r)
    # both sides decode the GPU's codes (any near-tie flip of the encode is then irrelevant); the
    # tables may differ by two fp32 ulps of the radius (see check rules above), so the bar is the
    # fp32 one on the whole matrix
    dec_ref = orc.decode(codes, norm, d_in, sig, tab_r, ba + bp, s, sb, block)
    dec = gpu_decode(q, codes, norm, sig, tab.cpu().numpy(), ba + bp, s, seed, d_in, block)
    n = assert_bf16_within_1ulp(dec, dec_ref["bf16"])
    log("  decode: %d BF16 outputs differ by 1 ulp" % n)
    # the reconstruction error of the polar code is that of a 5.5 bpw quantizer: well below 20 %
    w = torch.from_numpy(_problem(40 * 13 + 4096 + 5, 40, 4096, 128)[0].view(np.int16)).view(torch.bfloat16)
    w = w.float().numpy()
    d = torch.from_numpy(dec.view(np.int16)).view(torch.bfloat16).float().numpy()
    rows = np.linalg.norm(w, axis=1) > 0
    err = np.linalg.norm(d[rows] - w[rows]) / np.linalg.norm(w[rows])
    log("  relative reconstruction error %.4f" % err)
    assert err < 0.2


def test_polar_bad_thresholds_flag(q, orc):
    _, thr = orc.rayleigh_lloyd_max(4)
    bad = thr[::-1].copy()          # decreasing
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    p = np.random.default_rng(3).standard_normal((1000, 2)).astype(np.float32)
    q.polar_index(t(p), 4, 4, t(bad), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == q.FLAG_BAD_THRESHOLDS
    w, s, seed = _problem(5, 8, 256, 64)
    st.zero_()
    q.encode_polar(w_tensor(w), 4, 4, t(bad), scale=t(s), sign_seed=seed, block=64, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == q.FLAG_BAD_THRESHOLDS


# ----------------------------------------------------------------------------- full size

FULL = {
    "attn4096_5+6": (1, 0, 5, 6, 48),
    "l13b_gate_13824x5120_4+4": (3, 4, 4, 4, 24),
}


@pytest.mark.parametrize("case", list(FULL), ids=list(FULL))
def test_fullsize_polar(q, orc, synth, case):
    """Whole matrices encoded on the GPU as the benchmark does; the oracle checks sigma over every
    pair and the codes and norms of a seeded sample of rows (first and last rows included)."""
    cfg_i, sel, ba, bp, n_rows = FULL[case]
    cfg = synth.config(cfg_i)
    spec, block = cfg.matrices[sel], cfg.block
    d_out, d_in = spec.d_out, spec.d_in
    log("fullsize polar %s: %dx%d block=%d" % (case, d_out, d_in, block))
    w = spec.weights()
    s = spec.channel_scale()
    sb = orc.sign_mask(q.DEFAULT_SIGN_SEED, d_in)
    _, thr = orc.rayleigh_lloyd_max(ba)
    w_dev = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(DEV)
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    enc = q.encode_polar(w_dev, ba, bp, t(thr.astype(np.float64)), scale=t(s), block=block, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    sig_ref, _ = orc.calibrate(w[: min(d_out, 1024)], s, sb, block)
    np.testing.assert_array_equal(enc["sigma"].cpu().numpy(), sig_ref)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, d_out - 2, d_out - 1], rng.choice(d_out, n_rows, replace=False)]))
    ridx = torch.from_numpy(rows).to(DEV)
    codes = enc["codes"].index_select(0, ridx).cpu().numpy()
    norm = enc["norm"].index_select(0, ridx).cpu().numpy().view(np.uint16)
    ref = orc.encode_polar(w[rows], s, sb, block, ba, bp, thr, sig_ref, want_idx=True, want_p=True)
    np.testing.assert_array_equal(norm, ref["norm"])
    gidx = unpack_rows(orc, codes, ba + bp, d_in)
    flips = check_polar(gidx, ref["idx"], ref["p"], ba, bp, thr)
    log("  %d rows, %d near-tie flips" % (rows.size, flips))
