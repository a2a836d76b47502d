"""qamw_decode_many (section 3.2, the decoder, applied to the matrices of a model coded with one
codebook): every matrix of a grouped call comes out exactly as qamw_decode writes it, whatever the
mix of shapes, span widths, block sizes and matrix counts (launches of up to 48 matrices); one
matrix of each call is also held to the oracle's tolerances."""
import numpy as np
import pytest
import torch

from helpers import DEV, assert_bf16_within_1ulp, assert_rel_l2, log, t

pytestmark = pytest.mark.gpu


def _job(q, rng, d_out, d_in, bits, out_dtype=torch.bfloat16):
    """Random packed indices (any byte pattern is a valid code stream), f16 norms with one zero row,
    per-pair sigma, channel scale and sign seed."""
    codes = rng.integers(0, 256, size=(d_out, q.row_stride(d_in, bits)), dtype=np.uint8)
    norm = rng.uniform(0.25, 4.0, size=d_out).astype(np.float16)
    if d_out > 3:
        norm[3] = 0
    sigma = rng.uniform(0.5, 1.5, size=d_in // 2).astype(np.float32)
    scale = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    seed = int(rng.integers(0, 2**62))
    return {"codes": t(codes), "norm": t(norm.view(np.int16)), "sigma": t(sigma), "scale": t(scale), "d_in": d_in,
            "sign_seed": seed, "out": torch.full((d_out, d_in), 3.0, dtype=out_dtype, device=DEV),
            "np": (codes, norm.view(np.uint16), sigma, scale, seed)}


def _check_against_single(q, jobs, cb, bits, block, out_dtype):
    for k, j in enumerate(jobs):
        ref = q.decode(j["codes"], j["norm"], j["sigma"], cb, bits, j["d_in"], scale=j["scale"],
                       sign_seed=j["sign_seed"], block=block, out_dtype=out_dtype)
        torch.cuda.synchronize()
        got = j["out"]
        iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
        same = torch.equal(got.view(iv), ref.view(iv))
        assert same, "job %d (%d x %d): %d elements differ from qamw_decode" % (
            k, got.shape[0], got.shape[1], int((got.view(iv) != ref.view(iv)).sum()))


def _check_oracle(orc, j, cb_np, bits, block):
    codes, norm, sigma, scale, seed = j["np"]
    d_in = j["d_in"]
    ref = orc.decode(codes, norm, d_in, sigma, cb_np, bits, scale, orc.sign_mask(seed, d_in), block)
    got = j["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert_bf16_within_1ulp(got, ref["bf16"])


SHAPES = [(37, 512), (300, 384), (64, 256), (1, 5120), (129, 640), (0, 512), (260, 1024)]


@pytest.mark.parametrize("bits", [7, 8, 11])
def test_grouped_matches_single_block128(q, orc, bits):
    rng = np.random.default_rng(100 + bits)
    cb_np = rng.standard_normal((1 << bits, 2)).astype(np.float32)
    cb = t(cb_np)
    jobs = [_job(q, rng, d_out, d_in, bits) for d_out, d_in in SHAPES]
    log("decode_many bits %d: %s" % (bits, SHAPES))
    q.decode_many(jobs, cb, bits, block=128)
    torch.cuda.synchronize()
    _check_against_single(q, jobs, cb, bits, 128, torch.bfloat16)
    _check_oracle(orc, jobs[1], cb_np, bits, 128)


def test_grouped_default_blocks_and_fp32(q, orc):
    """block 0: 384 and 640 columns take block 128 and 256 columns block 256 (grouped launches of each
    block size), 512 and 1024 their own larger default (a launch each); fp32 output."""
    bits = 11
    rng = np.random.default_rng(7)
    cb_np = rng.standard_normal((1 << bits, 2)).astype(np.float32)
    cb = t(cb_np)
    jobs = [_job(q, rng, d_out, d_in, bits, torch.float32) for d_out, d_in in SHAPES]
    log("decode_many default blocks, fp32")
    q.decode_many(jobs, cb, bits, block=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_against_single(q, jobs, cb, bits, 0, torch.float32)
    codes, norm, sigma, scale, seed = jobs[1]["np"]
    ref = orc.decode(codes, norm, 384, sigma, cb_np, bits, scale, orc.sign_mask(seed, 384), 128)
    assert_rel_l2(jobs[1]["out"].cpu().numpy(), ref["f32"], 1e-5)


def test_grouped_more_than_one_launch(q):
    """110 matrices: three launches of at most 48, with span widths changing inside the list."""
    bits = 11
    rng = np.random.default_rng(9)
    cb = t(rng.standard_normal((1 << bits, 2)).astype(np.float32))
    shapes = [(int(rng.integers(1, 90)), 128 * int(rng.choice([1, 2, 3, 4, 8]))) for _ in range(110)]
    jobs = [_job(q, rng, d_out, d_in, bits) for d_out, d_in in shapes]
    log("decode_many 110 jobs")
    q.decode_many(jobs, cb, bits, block=128)
    torch.cuda.synchronize()
    _check_against_single(q, jobs, cb, bits, 128, torch.bfloat16)


def test_grouped_rejects_before_queueing(q):
    """A failing job leaves every output untouched: the checks run before anything is queued."""
    bits = 8
    rng = np.random.default_rng(11)
    cb = t(rng.standard_normal((1 << bits, 2)).astype(np.float32))
    good = _job(q, rng, 40, 512, bits)
    bad = _job(q, rng, 40, 512, bits)
    bad["d_in"] = 500   # codes no longer match: the binding or the library refuses the call
    with pytest.raises((ValueError, q.QamwError)):
        q.decode_many([good, bad], cb, bits, block=128)
    torch.cuda.synchronize()
    assert bool((good["out"] == 3.0).all())
