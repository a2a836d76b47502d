"""GPU parity of the fused dequantize-and-multiply (paper section 1) against the CPU oracle.

y = x W^T with W the decoder's weights before rounding.  The oracle decodes in fp64 and sums in
fp64; the kernel rotates the activation instead (u in fp64, rounded to fp32 once) and sums
c[idx] . u on the matrix cores with each fp32 operand split into bf16 pieces: c = c1 + c2 + dc with
|dc| <= 2^-18 |c|, u = u1 + u2 (+ u3) + du with |du| <= 2^-18 |u| (du = 0 with three pieces).  The
piece products are exact in fp32, so a term carries a relative error of at most 2^-18 + 2^-18 +
2^-24 (u's rounding) + their products < 2^-16.9; the fp32 sum adds, per output, 2 x np x d_in
piece products (np <= 3), eight wavefront partials, np column pieces and the norm, each addition
rounded once.  So |y - y_ref| <= (2^-16.9 + (6 d_in + 16) 2^-24) E, where E is the sum of the
absolute values of the terms, f16(norm_i) sum_k |c[idx].x u_2k| + |c[idx].y u_2k+1| (computed here
in fp64 from scipy's Hadamard matrix).  A BF16 output is the round-to-nearest-even of some value
within that bound of the oracle's.

Cases: one chunk and many chunks per row (a ragged last chunk), rows beyond one 16-row tile and
ragged last tiles, M = 1..16 (the three column layouts: 3 pieces x M <= 5, 2 pieces x M <= 8, two
operand groups up to 16), every index width 1..12, block sizes 2..1024, fp32 and BF16 inputs and
outputs, padded leading dimensions, zero rows, and the benchmark's 4096 x 4096 matrix whole.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

from helpers import DEV, bf16_ordinal, log, t

pytestmark = pytest.mark.gpu


def _problem(orc, seed, d_out, d_in, block, bits):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(5, size=(d_out, d_in)) * 0.015).astype(np.float32)
    w[:, rng.choice(d_in, size=max(1, d_in // 100), replace=False)] *= 10
    w[min(2, d_out - 1)] = 0
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    sseed = int(rng.integers(0, 2**62))   # sign-mask seed
    sb = orc.sign_mask(sseed, d_in)
    cb = rng.standard_normal((1 << bits, 2)).astype(np.float32)
    sig, _ = orc.calibrate(w[:1024], s, sb, block)
    e = orc.encode(w, s, sb, block, cb, bits, sig)
    return dict(codes=e["codes"], norm=e["norm"], d_in=d_in, sigma=sig, cb=cb, bits=bits, s=s, sign_bits=sb,
                sign_seed=sseed, block=block)


def _abs_terms(orc, x, pr):
    """E[m][i]: the sum of the absolute values of the terms the kernel adds for y[m][i]."""
    d_in, block = pr["d_in"], pr["block"]
    n_pairs = d_in // 2
    j = np.arange(d_in)
    eps = np.where((pr["sign_bits"][j // 32] >> (j % 32)) & 1, -1.0, 1.0)
    H = scipy.linalg.hadamard(block).astype(np.float64) / np.sqrt(block)
    v = x.astype(np.float64) * eps / pr["s"].astype(np.float64)
    u = (v.reshape(len(x), d_in // block, block) @ H).reshape(len(x), n_pairs, 2) * pr["sigma"].astype(np.float64)[None, :, None]
    idx = np.stack([orc.unpack_row(pr["codes"][i], pr["bits"], d_in) for i in range(len(pr["norm"]))])
    c = np.abs(pr["cb"].astype(np.float64)[idx])                         # d_out x n_pairs x 2
    rn = pr["norm"].astype(np.uint16).view(np.float16).astype(np.float64)
    return rn[None, :] * np.einsum("ikc,mkc->mi", c, np.abs(u))


def _run(q, orc, pr, M, x_dtype="bf16", y_dtype=torch.float32, ld_x=None, ld_y=None, seed=0):
    d_in, d_out = pr["d_in"], len(pr["norm"])
    rng = np.random.default_rng(100 + seed)
    x = rng.standard_normal((M, d_in)).astype(np.float32)
    if x_dtype == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        x = xt.float().numpy()                     # the values the kernel sees
    else:
        xt = torch.from_numpy(x)
    if ld_x is not None:
        big = torch.zeros((M, ld_x), dtype=xt.dtype)
        big[:, :d_in] = xt
        xd = big.to(DEV)[:, :d_in]
    else:
        xd = xt.to(DEV)
    out = full = None
    if ld_y is not None:
        full = torch.full((M, ld_y), 7.0, dtype=y_dtype, device=DEV)
        out = full[:, :d_out]
    y = q.qgemm(xd, t(pr["codes"]), t(pr["norm"].view(np.int16)), t(pr["sigma"]), t(pr["cb"]), pr["bits"],
                scale=t(pr["s"]), sign_seed=pr["sign_seed"], block=pr["block"], out_dtype=y_dtype,
                out=out)
    torch.cuda.synchronize()
    if full is not None:
        assert torch.all(full[:, d_out:] == 7.0).item()   # padding untouched
    ref = orc.qgemm(x, pr["codes"], pr["norm"], d_in, pr["sigma"], pr["cb"], pr["bits"], pr["s"], pr["sign_bits"],
                    pr["block"])
    return x, y, ref


def _bound(pr):
    return 2.0 ** -16.9 + (6 * pr["d_in"] + 16) * 2.0 ** -24


def _check_f32(orc, x, y, ref, pr):
    bound = _bound(pr)
    E = _abs_terms(orc, x, pr)
    got = y.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    rel = float(np.max(err / np.maximum(E, 1e-30)))
    assert np.all(err <= bound * E + 1e-37), "max error %.3g of the absolute term sum (bound %.3g)" % (rel, bound)
    return rel


CASES = {
    # id: (d_out, d_in, block, bits, M, x dtype)
    "4096_b128_B11_M1": (64, 4096, 128, 11, 1, "bf16"),
    "4096_b128_B11_M4": (100, 4096, 128, 11, 4, "bf16"),
    "768_b256_B8_M3": (33, 768, 256, 8, 3, "bf16"),
    "13824_b512_B11_M16": (20, 13824, 512, 11, 16, "bf16"),
    "5120_b128_B7_M2": (40, 5120, 128, 7, 2, "fp32"),
    "11008_b256_B11_M1": (17, 11008, 256, 11, 1, "bf16"),
    "5120_b128_B11_M5": (23, 5120, 128, 11, 5, "fp32"),
    "256_b2_B1_M7": (9, 256, 2, 1, 7, "fp32"),
    "2048_b1024_B12_M9": (31, 2048, 1024, 12, 9, "bf16"),
    "512_b64_B3_M16": (70, 512, 64, 3, 16, "bf16"),
    "1000_b8_B9_M8_ragged_chunk": (19, 1000, 8, 9, 8, "bf16"),
    "200_b8_B11_M6_one_ragged_chunk": (35, 200, 8, 11, 6, "bf16"),
    "2_b2_B4_M3_one_pair": (5, 2, 2, 4, 3, "fp32"),
    "64_b64_B12_M16": (4097, 64, 64, 12, 16, "bf16"),
}


@pytest.mark.parametrize("case", list(CASES), ids=list(CASES))
def test_qgemm_matches_oracle(q, orc, case):
    d_out, d_in, block, bits, M, xdt = CASES[case]
    log("qgemm %s" % case)
    pr = _problem(orc, d_out + d_in + bits, d_out, d_in, block, bits)
    x, y, ref = _run(q, orc, pr, M, x_dtype=xdt)
    rel = _check_f32(orc, x, y, ref, pr)
    assert np.all(y.cpu().numpy()[:, min(2, d_out - 1)] == 0)   # the zero row
    log("  max error %.3g of the absolute term sum" % rel)


@pytest.mark.parametrize("M,d_out,d_in", [(2, 12, 4416), (12, 12, 4416), (12, 4100, 320)])
@pytest.mark.parametrize("bits", list(range(1, 13)))
def test_qgemm_every_index_width(q, orc, bits, M, d_out, d_in):
    """Every index width on the three kernel layouts: two activation rows (one operand group), twelve
    on 12 weight rows (two operand groups; 4416 columns: 2208 pairs, 17 chunks of 128 and a ragged
    18th of 32) and twelve on 4100 weight rows (32-row tiles; 320 columns: two chunks of 64 and a
    ragged third of 32)."""
    pr = _problem(orc, 500 + bits, d_out, d_in, 64, bits)
    x, y, ref = _run(q, orc, pr, M, seed=bits)
    _check_f32(orc, x, y, ref, pr)


@pytest.mark.parametrize("d_out,M", [(8229, 1), (8229, 3), (32851, 8), (5120, 3), (8229, 9), (13824, 16), (2000, 1)])
def test_qgemm_tall_matrices(q, orc, d_out, M):
    """Tall matrices: whole rounds of tiles over the 256 compute units, the rows left over in one
    round of shorter tiles.  16-row tiles: 8229 rows are 512 tiles, then 37 of one row; 32851 are
    2048, then 83 of one; 5120 are 256, then 256 of four; 2000 are 250 of eight.  32-row tiles
    (M > 8): 8229 rows are 256 tiles, then 37 of one; 13824 are 256, then 256 of 22."""
    log("qgemm tall %d rows M=%d" % (d_out, M))
    pr = _problem(orc, 900 + M, d_out, 256, 64, 6)
    x, y, ref = _run(q, orc, pr, M, seed=M)
    _check_f32(orc, x, y, ref, pr)


def test_qgemm_bf16_output_and_padded_strides(q, orc):
    pr = _problem(orc, 7, 50, 1024, 128, 10)
    x, y, ref = _run(q, orc, pr, 6, x_dtype="fp32", y_dtype=torch.bfloat16, ld_x=1024 + 40, ld_y=50 + 14)
    E = _abs_terms(orc, x, pr)
    r = _bound(pr) * E

    def bf16_of(v):
        return bf16_ordinal(torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
                            .view(np.uint16))
    lo, hi = bf16_of(ref - r), bf16_of(ref + r)   # rounding is monotone
    got = bf16_ordinal(y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all((got >= lo) & (got <= hi)), "BF16 output outside the rounding of the bound at %s" % (
        np.argwhere((got < lo) | (got > hi))[:3])
    n = int(np.sum(got != bf16_of(ref)))
    log("  bf16: %d of %d outputs differ from the rounded oracle value (within the bound)" % (n, got.size))


def test_qgemm_empty_and_limits(q, orc):
    pr = _problem(orc, 8, 8, 256, 64, 8)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    y = q.qgemm(x, t(pr["codes"]), t(pr["norm"].view(np.int16)), t(pr["sigma"]), t(pr["cb"]), 8,
                scale=t(pr["s"]), sign_seed=pr["sign_seed"], block=64)
    assert y.shape == (0, 8)
    x17 = torch.zeros((17, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QamwError) as ei:
        q.qgemm(x17, t(pr["codes"]), t(pr["norm"].view(np.int16)), t(pr["sigma"]), t(pr["cb"]), 8, block=64)
    assert ei.value.code == q.ERR_UNSUPPORTED


@pytest.mark.parametrize("M", [1, 16])
def test_qgemm_fullsize_attn4096(q, orc, synth, M):
    """The benchmark's whole 4096 x 4096 matrix and K = 2048 codebook, multiplied as the benchmark
    does; every output against the oracle's product (codes from the oracle's encoder)."""
    cfg = synth.config(1)
    m = cfg.matrices[0]
    d_out, d_in, block, bits = m.d_out, m.d_in, cfg.block, cfg.bits[0]
    log("qgemm fullsize 4096x4096 M=%d" % M)
    cb = np.ascontiguousarray(np.load("tests/golden/cb_cfg1_k2048.npz")["codebook"]).astype(np.float32)
    w = m.weights()
    s = m.channel_scale()
    sb = orc.sign_mask(q.DEFAULT_SIGN_SEED, d_in)
    sig, _ = orc.calibrate(w[:1024], s, sb, block)
    e = orc.encode(w, s, sb, block, cb, bits, sig, want_idx=False)
    pr = dict(codes=e["codes"], norm=e["norm"], d_in=d_in, sigma=sig, cb=cb, bits=bits, s=s, sign_bits=sb,
              sign_seed=q.DEFAULT_SIGN_SEED, block=block)
    x, y, ref = _run(q, orc, pr, M, seed=M)
    rel = _check_f32(orc, x, y, ref, pr)
    log("  max error %.3g of the absolute term sum" % rel)
