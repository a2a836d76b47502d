"""GPU parity of the scalar (d = 1) ablation (paper section 2, reading R10) against the CPU oracle.

The GPU builds the normal Lloyd-Max levels and the product table (qamw_scalar_codebook) and codes
with the QAM-W search over that table (qamw_codebook_index + qamw_encode, bits = 2b); the oracle
codes each coordinate with its scalar rule.

Comparison rules:
  * levels and thresholds within 1e-10 relative (as for the polar levels: the oracle's Phi
    difference loses about 1e-13 in the sparse tails, carried along by the slow iteration);
  * table entries within one fp32 ulp;
  * indices: the rule of tests/helpers.py (equal, or a codeword whose fp32 distance to the oracle's
    pair exceeds the oracle's by at most 1e-6 relative; the 2D search and the scalar rule can part
    only where the fp32 distance rounds two levels together).
"""
import numpy as np
import pytest
import torch

from helpers import DEV, assert_bf16_within_1ulp, check_indices, gpu_decode, log, t, unpack_rows, w_tensor

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6])
def test_scalar_codebook_matches_oracle(q, orc, b):
    lv, thr, tab = q.scalar_codebook(b)
    torch.cuda.synchronize()
    lv, thr, tab = lv.cpu().numpy(), thr.cpu().numpy(), tab.cpu().numpy()
    lv_r, thr_r = orc.gauss_lloyd_max(b)
    rel = np.max(np.abs(lv - lv_r) / np.abs(lv_r))
    log("scalar codebook b=%d: max rel diff %.3g" % (b, rel))
    assert rel <= 1e-10
    np.testing.assert_allclose(thr, thr_r, rtol=1e-10, atol=1e-14)
    np.testing.assert_array_equal(thr, 0.5 * (lv[:-1] + lv[1:]))
    tab_r = orc.scalar_table(b, lv_r)
    ulp = np.abs(tab.view(np.int32).astype(np.int64) - tab_r.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1


def _problem(seed, d_out, d_in):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(5, size=(d_out, d_in)) * 0.015).astype(np.float32)
    w[min(1, d_out - 1)] = 0
    w = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    seed = int(rng.integers(0, 2**62))   # sign-mask seed
    return w, s, seed


@pytest.mark.parametrize("shape", [(40, 4096, 128, 4), (33, 768, 256, 3), (17, 512, 64, 6), (20, 1024, 32, 1)],
                         ids=lambda s: "%dx%d_b%d_%dbit" % s)
def test_scalar_encode_matches_oracle(q, orc, shape):
    d_out, d_in, block, b = shape
    w, s, seed = _problem(d_out + d_in + b, d_out, d_in)
    sb = orc.sign_mask(seed, d_in)
    sig, _ = orc.calibrate(w[:1024], s, sb, block)
    lv_r, thr_r = orc.gauss_lloyd_max(b)
    tab_r = orc.scalar_table(b, lv_r)
    ref = orc.encode_scalar(w, s, sb, block, b, thr_r, sig, want_idx=True, want_p=True)
    log("scalar encode %s" % (shape,))
    cb_dev = t(tab_r)
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = q.encode(w_tensor(w), cb_dev, 2 * b, q.codebook_index(cb_dev, 2 * b), scale=t(s), sign_seed=seed,
                   block=block, status=st)
    torch.cuda.synchronize()
    codes = out["codes"].cpu().numpy()
    np.testing.assert_array_equal(out["sigma"].cpu().numpy(), sig)
    np.testing.assert_array_equal(out["norm"].cpu().numpy().view(np.uint16), ref["norm"])
    assert int(st.item()) == 0
    gidx = unpack_rows(orc, codes, 2 * b, d_in)
    flips = check_indices(gidx, ref["idx"], ref["p"], tab_r)
    log("  %d near-tie flips" % flips)
    same = np.all(gidx == ref["idx"], axis=1)
    np.testing.assert_array_equal(codes[same], ref["codes"][same])
    # decode with the GPU's own table
    _, _, tab = q.scalar_codebook(b)
    dec = gpu_decode(q, codes, out["norm"].cpu().numpy().view(np.uint16), sig, tab.cpu().numpy(), 2 * b, s, seed, d_in,
                     block)
    dref = orc.decode(codes, ref["norm"], d_in, sig, tab_r, 2 * b, s, sb, block)
    n = assert_bf16_within_1ulp(dec, dref["bf16"])
    log("  decode: %d BF16 outputs differ by one ulp" % n)
