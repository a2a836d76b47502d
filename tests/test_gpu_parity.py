"""GPU parity: libqamw.so (HIP, gfx950) against the CPU oracle on seeded inputs.

Covers the search index (exact nearest codeword), decode cross-fed with oracle codes, encode
(calibration, norms, indices, packed bytes), the encode -> decode round trip, Lloyd training,
data-fault flags, and edge shapes: ragged row counts, partial wavefronts, every block size from
2 to 1024, index widths 1..12 bits, padded leading dimensions, zero rows, and the widest rows
accepted (16384 columns at b = 128 and 512, 32768 at b = 1024).
"""
import os

import numpy as np
import pytest
import torch

from helpers import (DEV, assert_bf16_within_1ulp, assert_rel_l2, check_indices, gpu_decode, gpu_encode, log, t,
                     unpack_rows, w_tensor)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_cb(name):
    z = np.load(os.path.join(GOLDEN, name + ".npz"))
    return z["codebook"], z["trace"], z["meta"]


def rand_problem(seed, d_out, d_in, dtype="bf16", heavy=True):
    rng = np.random.default_rng(seed)
    if heavy:
        w = rng.standard_t(5, size=(d_out, d_in)) * 0.015
        cols = rng.choice(d_in, size=max(1, d_in // 100), replace=False)
        w[:, cols] *= 10
    else:
        w = rng.standard_normal((d_out, d_in)) * 0.02
    w = w.astype(np.float32)
    if dtype == "bf16":
        w = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = (np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)
    sign_seed = int(rng.integers(0, 2**63, dtype=np.int64)) * 2 + 1   # any 64-bit seed
    return w, s, sign_seed


def rand_cb(seed, bits):
    rng = np.random.default_rng(1000 + seed)
    return rng.standard_normal((1 << bits, 2)).astype(np.float32)


# ----------------------------------------------------------------------------- search index

def _probes(cb, n, seed):
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal((n, 2)) * sc for sc in (0.5, 1.0, 2.0, 4.0)]
    ext = float(np.abs(cb).max())
    parts.append(rng.uniform(-1.5 * ext, 1.5 * ext, size=(n, 2)))
    parts.append(cb.astype(np.float64))
    # midpoints between each codeword and a close neighbour: near-exact ties
    j = np.arange(len(cb))
    k = (j * 7 + 1) % len(cb)
    d = ((cb[:, None, :].astype(np.float64) - cb[None, :, :]) ** 2).sum(-1) if len(cb) <= 4096 else None
    if d is not None:
        d[j, j] = np.inf
        k = d.argmin(1)
    parts.append((cb.astype(np.float64) + cb[k]) / 2)
    parts.append(np.array([[ext * 3, 0], [0, -ext * 5], [1e30, 1e30], [np.nan, 0], [np.inf, 1.0], [0, 0]]))
    return np.concatenate(parts).astype(np.float32)


@pytest.mark.parametrize("name", ["cfg0", "cfg1", "cfg3", "rand12", "rand1", "dup4", "grid8", "cfg0_beyond_grid"])
def test_nearest_matches_bruteforce(q, orc, name):
    if name in ("cfg0", "cfg0_beyond_grid"):
        cb, bits = golden_cb("cb_cfg0_k256")[0], 8
    elif name == "cfg1":
        cb, bits = golden_cb("cb_cfg1_k2048")[0], 11
    elif name == "cfg3":
        cb, bits = golden_cb("cb_cfg3_k128")[0], 7
    elif name == "rand12":
        cb, bits = rand_cb(12, 12), 12
    elif name == "rand1":
        cb, bits = rand_cb(1, 1), 1
    elif name == "dup4":  # repeated codewords: ties must go to the lowest index
        base = rand_cb(4, 2)
        cb, bits = np.concatenate([base, base, base[::-1], base]).astype(np.float32), 4
    else:  # lattice codebook: many exact ties on the cell boundaries
        g = np.arange(16) - 7.5
        cb, bits = np.stack(np.meshgrid(g, g), -1).reshape(-1, 2).astype(np.float32) * 0.25, 8
    # more probes than one launch covers (2048 workgroups of 256 threads, then a grid stride)
    n = 2048 * 256 + 5000 if name == "cfg0_beyond_grid" else (60000 if bits >= 11 else 200000)
    p = _probes(cb, n, bits)
    log("nearest %s: K=%d probes=%d" % (name, len(cb), len(p)))
    cbd = t(cb)
    idx = q.codebook_index(cbd, bits)
    got = q.nearest(t(p), cbd, bits, idx).cpu().numpy()
    ref, _ = orc.nearest(p, cb)
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------------------- decode (oracle codes)

SHAPES = [  # d_out, d_in, block, bits
    (64, 512, 64, 8), (37, 320, 64, 5), (17, 256, 2, 3), (9, 128, 16, 7), (33, 1024, 32, 11),
    (12, 2048, 256, 11), (8, 4096, 512, 12), (5, 2048, 1024, 1), (40, 4096, 128, 11),
    (3, 13824, 128, 11), (4, 11008, 256, 11), (6, 5120, 128, 7), (7, 192, 4, 9), (11, 96, 8, 6),
    # the widest rows the kernels take: 1024 lanes of 16 columns, 512 of 32, 512 of 64
    (2, 16384, 128, 11), (3, 16384, 512, 12), (2, 32768, 1024, 8),
    # b = 1024 with 11- and 12-bit indices on wide rows (the decoder's LDS limit; block 0 picks 1024
    # for 5120 columns)
    (8, 5120, 0, 11), (4, 16384, 1024, 12), (2, 28672, 1024, 11),
    # the 128-column decoder: ragged 16-row tiles, one and three column blocks, every supported width
    (17, 128, 128, 11), (33, 384, 128, 8), (100, 1280, 128, 7), (47, 2560, 128, 11),
    # ... and its 256-column form (two 128-column halves per block): spans of 2 and 4 halves
    (33, 512, 256, 8), (70, 768, 256, 11), (17, 1024, 256, 7), (9, 11008, 256, 11),
]


def _shape_id(s):
    return "x".join(map(str, s))


@pytest.mark.parametrize("shape", SHAPES, ids=_shape_id)
def test_decode_crossfed(q, orc, shape):
    d_out, d_in, block, bits = shape
    w, s, seed = rand_problem(d_out * 31 + d_in, d_out, d_in)
    sb = orc.sign_mask(seed, d_in)
    w[min(2, d_out - 1)] = 0
    cb = rand_cb(bits, bits)
    ob = block or orc.default_block(d_in)   # block 0: the library applies the section 3.3 rule
    sigma, _ = orc.calibrate(w, s, sb, ob)
    enc = orc.encode(w, s, sb, ob, cb, bits, sigma, want_idx=False)
    ref = orc.decode(enc["codes"], enc["norm"], d_in, sigma, cb, bits, s, sb, ob)
    log("decode %s" % (shape,))
    got16 = gpu_decode(q, enc["codes"], enc["norm"], sigma, cb, bits, s, seed, d_in, block)
    n_diff = assert_bf16_within_1ulp(got16, ref["bf16"])
    got32 = gpu_decode(q, enc["codes"], enc["norm"], sigma, cb, bits, s, seed, d_in, block, out_dtype=torch.float32)
    assert_rel_l2(got32, ref["f32"], 1e-5)
    # every output is within one BF16 ulp (checked above); the 128-column decoder holds eps_j / s_j
    # in fp32, which moves about 5e-5 of the outputs across a BF16 rounding boundary
    assert n_diff <= max(4, got16.size // 2000)
    assert not got16[min(2, d_out - 1)].any()


def test_decode_padded_output_and_defaults(q, orc):
    d_out, d_in, block, bits = 21, 640, 128, 8
    w, _, _ = rand_problem(5, d_out, d_in)
    cb = rand_cb(8, bits)
    ones = np.ones(d_in, np.float32)
    plus = orc.sign_mask(q.DEFAULT_SIGN_SEED, d_in)   # the mask of the default seed
    sigma, _ = orc.calibrate(w, ones, plus, block)
    enc = orc.encode(w, ones, plus, block, cb, bits, sigma, want_idx=False)
    ref = orc.decode(enc["codes"], enc["norm"], d_in, sigma, cb, bits, ones, plus, block)
    got = gpu_decode(q, enc["codes"], enc["norm"], sigma, cb, bits, None, None, d_in, block, ld=d_in + 64)
    assert_bf16_within_1ulp(got, ref["bf16"])


# ----------------------------------------------------------------------------- encode

def _encode_case(q, orc, shape, dtype="bf16", given_sigma=False, ld=None, seed=0):
    d_out, d_in, block, bits = shape
    w, s, sseed = rand_problem(seed + d_out * 7 + d_in, d_out, d_in, dtype=dtype)
    sb = orc.sign_mask(sseed, d_in)
    w[min(1, d_out - 1)] = 0
    cb = rand_cb(bits + 50, bits)
    ob = block or orc.default_block(d_in)   # block 0: the library applies the section 3.3 rule
    sig_ref, st_ref = orc.calibrate(w[:1024], s, sb, ob)
    sigma_in = None
    if given_sigma:
        sig_ref = (np.abs(np.random.default_rng(seed).standard_normal(d_in // 2)) * 0.05 + 0.01).astype(np.float32)
        sigma_in = sig_ref
    ref = orc.encode(w, s, sb, ob, cb, bits, sig_ref, want_p=True)
    log("encode %s %s sigma=%s ld=%s" % (shape, dtype, "given" if given_sigma else "calibrated", ld))
    got = gpu_encode(q, w, s, sseed, block, cb, bits, sigma=sigma_in, ld=ld)
    np.testing.assert_array_equal(got["sigma"], sig_ref)
    np.testing.assert_array_equal(got["norm"], ref["norm"])
    assert got["status"] == ref["status"] == 0
    gidx = unpack_rows(orc, got["codes"], bits, d_in)
    flips = check_indices(gidx, ref["idx"], ref["p"], cb)
    # packed bytes, padding included, of every row without a near-tie flip
    same = (gidx == ref["idx"]).all(axis=1)
    np.testing.assert_array_equal(got["codes"][same], ref["codes"][same])
    if flips:
        log("  %d near-tie index flips in %d rows" % (flips, int((~same).sum())))
    return got, ref, cb, sig_ref, s, sseed, sb


@pytest.mark.parametrize("shape", SHAPES, ids=_shape_id)
def test_encode_matches_oracle(q, orc, shape):
    _encode_case(q, orc, shape)


@pytest.mark.parametrize("variant", ["fp32", "given_sigma", "padded_ld", "many_rows"])
def test_encode_variants(q, orc, variant):
    if variant == "fp32":
        _encode_case(q, orc, (50, 512, 64, 8), dtype="fp32")
    elif variant == "given_sigma":
        _encode_case(q, orc, (30, 1024, 128, 11), given_sigma=True)
    elif variant == "padded_ld":
        _encode_case(q, orc, (25, 768, 256, 10), ld=768 + 40)
    else:  # more rows than the calibration window and than the grid
        _encode_case(q, orc, (1300, 256, 64, 6))


@pytest.mark.parametrize("shape", [(48, 2048, 128, 11), (300, 4096, 128, 11), (64, 11008, 256, 11),
                                   (40, 13824, 128, 7), (33, 1024, 32, 8)], ids=_shape_id)
def test_roundtrip_gpu_encode_gpu_decode(q, orc, shape):
    """GPU encode then GPU decode, against the oracle decoding the same (GPU) codes: unconditional,
    whatever near-tie flips the encode had."""
    d_out, d_in, block, bits = shape
    got, ref, cb, sigma, s, sseed, sb = _encode_case(q, orc, shape, seed=3)
    dec_ref = orc.decode(got["codes"], got["norm"], d_in, sigma, cb, bits, s, sb, block or orc.default_block(d_in))
    dec = gpu_decode(q, got["codes"], got["norm"], got["sigma"], cb, bits, s, sseed, d_in, block)
    assert_bf16_within_1ulp(dec, dec_ref["bf16"])
    dec32 = gpu_decode(q, got["codes"], got["norm"], got["sigma"], cb, bits, s, sseed, d_in, block,
                       out_dtype=torch.float32)
    assert_rel_l2(dec32, dec_ref["f32"], 1e-5)


@pytest.mark.parametrize("seed", [0, 1, 1234567, 0x51414D57, 2**64 - 1])
def test_sign_mask_matches_oracle(q, orc, seed):
    for d_in in (1, 31, 32, 33, 4096, 13824, 32768):
        got = q.sign_mask(d_in, seed).cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got, orc.sign_mask(seed, d_in))


def test_sign_seed_changes_the_code(q, orc):
    """Two seeds give two rotations: the codes differ, and each decodes only with its own seed."""
    w, s, _ = rand_problem(77, 16, 1024)
    cb = rand_cb(8, 8)
    a = gpu_encode(q, w, s, 11, 128, cb, 8)
    b = gpu_encode(q, w, s, 12, 128, cb, 8)
    assert not np.array_equal(a["codes"], b["codes"])
    ok = gpu_decode(q, a["codes"], a["norm"], a["sigma"], cb, 8, s, 11, 1024, 128, out_dtype=torch.float32)
    bad = gpu_decode(q, a["codes"], a["norm"], a["sigma"], cb, 8, s, 12, 1024, 128, out_dtype=torch.float32)
    wf = w_tensor(w).float().cpu().numpy()
    assert np.linalg.norm(ok - wf) < 0.5 * np.linalg.norm(bad - wf)


def test_side_stream_matches_default_stream(q):
    """Every call runs on the caller's current stream: encode (with calibration), decode and the
    fused product issued on a second stream give the bytes they give on the default stream."""
    w, s, seed = rand_problem(41, 300, 2048)
    cb = t(rand_cb(11, 11))
    wd, sd = w_tensor(w), t(s)
    idx = q.codebook_index(cb, 11)
    x = torch.from_numpy(np.random.default_rng(5).standard_normal((8, 2048)).astype(np.float32)).to(DEV)

    def run():
        e = q.encode(wd, cb, 11, idx, scale=sd, sign_seed=seed, block=128)
        dec = q.decode(e["codes"], e["norm"], e["sigma"], cb, 11, 2048, scale=sd, sign_seed=seed, block=128)
        y = q.qgemm(x, e["codes"], e["norm"], e["sigma"], cb, 11, scale=sd, sign_seed=seed, block=128)
        return [e["codes"], e["norm"], e["sigma"], dec.view(torch.int16), y]

    ref = [v.cpu() for v in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run()
    side.synchronize()
    got = [v.cpu() for v in got]
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_encode_is_deterministic(q):
    w, s, seed = rand_problem(99, 300, 4096)
    cb = rand_cb(11, 11)
    a = gpu_encode(q, w, s, seed, 128, cb, 11)
    b = gpu_encode(q, w, s, seed, 128, cb, 11)
    for k in ("codes", "norm", "sigma"):
        np.testing.assert_array_equal(a[k], b[k])


def test_empty_matrix(q, orc):
    d_in = 256
    w = np.zeros((0, d_in), np.uint16)
    cb = rand_cb(3, 6)
    got = gpu_encode(q, w, None, None, 64, cb, 6)
    assert got["codes"].shape == (0, q.row_stride(d_in, 6))
    np.testing.assert_array_equal(got["sigma"], np.float32(1 / np.sqrt(d_in)))


# ----------------------------------------------------------------------------- data-fault flags

def test_status_flags(q):
    d_out, d_in = 6, 256
    w, s, sb = rand_problem(7, d_out, d_in, dtype="fp32")   # sb: the sign-mask seed
    cb = rand_cb(5, 6)
    sig = np.full(d_in // 2, 0.05, np.float32)
    assert gpu_encode(q, w, s, sb, 64, cb, 6, sigma=sig)["status"] == 0
    w2 = w.copy()
    w2[3, 17] = np.nan
    assert gpu_encode(q, w2, s, sb, 64, cb, 6, sigma=sig)["status"] & 1
    s2 = s.copy()
    s2[9] = -1.0
    assert gpu_encode(q, w, s2, sb, 64, cb, 6, sigma=sig)["status"] & 2
    w3 = w.copy()
    w3[2] *= 1e6
    assert gpu_encode(q, w3, s, sb, 64, cb, 6, sigma=sig)["status"] == 4


# ----------------------------------------------------------------------------- Lloyd

def test_lloyd_bit_identical_small(q, orc, synth):
    pts = synth.points(synth.CONFIG_SEED_BASE + 9, 4, 20000)
    for bits, iters in ((1, 5), (4, 9), (8, 6), (10, 3)):
        ref_cb, ref_tr, _ = orc.lloyd(pts, bits, iters)
        cb, tr = q.codebook_train(t(pts), bits, iters)
        np.testing.assert_array_equal(cb.cpu().numpy(), ref_cb)
        np.testing.assert_array_equal(tr.cpu().numpy(), ref_tr)


@pytest.mark.parametrize("name", ["cb_cfg0_k256", "cb_cfg3_k128", "cb_cfg1_k2048", "cb_cfg2_k2048"])
def test_lloyd_matches_golden(q, synth, name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip("golden codebook %s not generated" % name)
    cb_ref, tr_ref, meta = golden_cb(name)
    cfg_i, sid, n, bits, iters = [int(x) for x in meta]
    pts = synth.points(synth.config(cfg_i).seed, sid, n)
    log("lloyd %s: n=%d K=%d iters=%d" % (name, n, 1 << bits, iters))
    cb, tr = q.codebook_train(t(pts), bits, iters)
    np.testing.assert_array_equal(cb.cpu().numpy(), cb_ref)
    np.testing.assert_array_equal(tr.cpu().numpy(), tr_ref)


def test_lloyd_resume_and_init(q, orc, synth):
    pts = synth.points(synth.CONFIG_SEED_BASE + 11, 4, 30000)
    full, trf = q.codebook_train(t(pts), 7, 8)
    a, tra = q.codebook_train(t(pts), 7, 3)
    b, trb = q.codebook_train(t(pts), 7, 5, init=a.clone())
    np.testing.assert_array_equal(b.cpu().numpy(), full.cpu().numpy())
    np.testing.assert_array_equal(torch.cat([tra, trb]).cpu().numpy(), trf.cpu().numpy())
    ref, _, _ = orc.lloyd(pts, 7, 5, init=a.cpu().numpy())
    np.testing.assert_array_equal(b.cpu().numpy(), ref)


def test_lloyd_point_range_flag(q):
    pts = np.random.default_rng(3).standard_normal((5000, 2)).astype(np.float32)
    pts[17, 0] = 1e5
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    q.codebook_train(t(pts), 4, 2, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 8


def test_index_of_another_codebook_size_is_rejected_on_the_device(q):
    """An index built for K = 2^10 used with a K = 2^11 codebook: nearest answers -1 and encode flags
    QAMW_FLAG_BAD_INDEX and writes nothing (the LDS image it would load has another size)."""
    cb10, cb11 = t(rand_cb(10, 10)), t(rand_cb(11, 11))
    idx10 = q.codebook_index(cb10, 10)
    pad = torch.zeros((q.index_bytes(11),), dtype=torch.uint8, device=DEV)
    pad[: idx10.numel()] = idx10
    pts = t(np.random.default_rng(2).standard_normal((1000, 2)).astype(np.float32))
    assert (q.nearest(pts, cb11, 11, pad).cpu().numpy() == -1).all()
    w, s, seed = rand_problem(3, 8, 256)
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    codes = torch.full((8, q.row_stride(256, 11)), 0xAB, dtype=torch.uint8, device=DEV)
    q.encode(w_tensor(w), cb11, 11, pad, scale=t(s), sign_seed=seed, block=64, status=st, out={"codes": codes})
    torch.cuda.synchronize()
    assert int(st.item()) & q.FLAG_BAD_INDEX
    assert (codes.cpu().numpy() == 0xAB).all()
