"""Pins for the oracle's product after dequantization (paper section 1): y = x W^T with W the
decoder's output before rounding.

The oracle decodes (pinned in test_oracle_pins.py) and sums x_j w_ij in fp64.  It is checked
against what the mathematics fixes without it: unit activations return the decoded columns
exactly; the same product computed the other way round, rotating the activation instead of the
weights (the block Hadamard matrix is symmetric), from scipy's Hadamard matrix, agrees to 1e-12;
the product is linear in x; a zero row gives zeros; and it stays within BF16 rounding of the
paper's pipeline, which rounds W to BF16 before the product.
"""
import numpy as np
import pytest
import scipy.linalg


def _problem(orc, seed, d_out=40, d_in=256, block=64, bits=8):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(5, size=(d_out, d_in)) * 0.015).astype(np.float32)
    w[3] = 0
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    sb = rng.integers(0, 2**32, size=(d_in + 31) // 32, dtype=np.uint64).astype(np.uint32)
    cb = rng.standard_normal((1 << bits, 2)).astype(np.float32)
    sig, _ = orc.calibrate(w, s, sb, block)
    e = orc.encode(w, s, sb, block, cb, bits, sig)
    return dict(codes=e["codes"], norm=e["norm"], d_in=d_in, sigma=sig, cb=cb, bits=bits, s=s, sign_bits=sb,
                block=block)


def _eps(sb, d_in):
    j = np.arange(d_in)
    return np.where((sb[j // 32] >> (j % 32)) & 1, -1.0, 1.0)


def test_unit_activations_return_the_decoded_columns(orc):
    pr = _problem(orc, 1)
    d_in = pr["d_in"]
    w64 = orc.decode(pr["codes"], pr["norm"], d_in, pr["sigma"], pr["cb"], pr["bits"], pr["s"], pr["sign_bits"],
                     pr["block"], want_f64=True)["f64"]
    y = orc.qgemm(np.eye(d_in, dtype=np.float32), **pr)
    np.testing.assert_array_equal(y, w64.T)


@pytest.mark.parametrize("block", [2, 64, 256])
def test_rotating_the_activation_gives_the_same_product(orc, block):
    """sum_j x_j w_ij = f16(norm_i) sum_k sigma_k (c[idx_ik] . u_k), u = blockdiag(H_b/sqrt b)(eps x / s)."""
    pr = _problem(orc, 2, block=block)
    d_in, n_pairs = pr["d_in"], pr["d_in"] // 2
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, d_in)).astype(np.float32)
    y = orc.qgemm(x, **pr)
    H = scipy.linalg.hadamard(block).astype(np.float64) / np.sqrt(block)
    v = x.astype(np.float64) * _eps(pr["sign_bits"], d_in) / pr["s"].astype(np.float64)
    u = (v.reshape(5, d_in // block, block) @ H).reshape(5, d_in)   # H is symmetric
    idx = np.stack([orc.unpack_row(pr["codes"][i], pr["bits"], d_in) for i in range(len(pr["norm"]))])
    c = pr["cb"].astype(np.float64)[idx]                              # d_out x n_pairs x 2
    sig = pr["sigma"].astype(np.float64)
    up = u.reshape(5, n_pairs, 2)
    t = np.einsum("ikc,mkc->mik", c * sig[None, :, None], up)       # per-pair terms
    rn = pr["norm"].astype(np.uint16).view(np.float16).astype(np.float64)
    want = rn[None, :] * t.sum(axis=2)
    scale = rn[None, :] * np.abs(t).sum(axis=2) + 1e-300
    assert np.max(np.abs(y - want) / scale) < 1e-12


def test_linear_in_the_activation(orc):
    pr = _problem(orc, 4)
    rng = np.random.default_rng(5)
    a = rng.standard_normal((3, pr["d_in"])).astype(np.float32)
    b = rng.standard_normal((3, pr["d_in"])).astype(np.float32)
    ya, yb = orc.qgemm(a, **pr), orc.qgemm(b, **pr)
    yab = orc.qgemm(np.concatenate([a, b]), **pr)
    np.testing.assert_array_equal(yab, np.concatenate([ya, yb]))
    y2 = orc.qgemm(2 * a, **pr)                      # exact: scaling by 2
    np.testing.assert_array_equal(y2, 2 * ya)
    assert np.all(ya[:, 3] == 0)                     # the zero row


def test_within_bf16_rounding_of_the_paper_pipeline(orc):
    """Section 1: the paper rounds W to BF16 before the product; the exact product differs from that
    by at most the BF16 rounding of each weight (2^-9 relative), summed over the row."""
    pr = _problem(orc, 6, d_out=24, d_in=512, block=128, bits=7)
    d_in = pr["d_in"]
    dec = orc.decode(pr["codes"], pr["norm"], d_in, pr["sigma"], pr["cb"], pr["bits"], pr["s"], pr["sign_bits"],
                     pr["block"], want_f64=True)
    wb = (dec["bf16"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = np.random.default_rng(7).standard_normal((2, d_in)).astype(np.float32)
    y = orc.qgemm(x, **pr)
    y_bf16 = x.astype(np.float64) @ wb.T
    bound = 2.0 ** -8 * (np.abs(x.astype(np.float64)) @ np.abs(dec["f64"]).T)
    assert np.all(np.abs(y - y_bf16) <= bound)
    assert np.any(y != y_bf16)
