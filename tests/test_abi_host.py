"""The C ABI without a GPU: libqamw.so loads, exports every function include/qamw.h declares,
and its host-side helpers and argument checks behave as documented.  Every call below is
rejected by host code before any HIP call is made."""
import ctypes
import os
import subprocess

import pytest

import weight_quantization_codec_amd as q

ARG, UNSUP, WS = q.ERR_ARG, q.ERR_UNSUPPORTED, q.ERR_WORKSPACE


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.LIB_PATH):
        from weight_quantization_codec_amd import _build
        _build.build()
    return q.load()


def test_exports_every_declared_symbol(lib):
    names = q.header_symbols()
    assert len(names) == 22
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_header_is_plain_c():
    import re
    text = re.sub(r"/\*.*?\*/", "", open(q.HEADER_PATH).read(), flags=re.S)
    for bad in ("hip_runtime", "torch", "hipStream_t", "namespace", "template"):
        assert bad not in text
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-x", "c", q.HEADER_PATH], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_row_stride_and_block_rule(lib, orc):
    for d_in in (2, 6, 64, 512, 4096, 5120, 11008, 13824):
        for bits in range(1, 17):
            assert lib.qamw_row_stride(d_in, bits) == orc.row_stride(d_in, bits)
        assert lib.qamw_default_block(d_in) == orc.default_block(d_in)
    assert lib.qamw_row_stride(4096, 11) == 2816 and lib.qamw_row_stride(5120, 7) == 2240
    assert lib.qamw_row_stride(0, 8) == 0 and lib.qamw_row_stride(7, 8) == 0 and lib.qamw_row_stride(8, 0) == 0
    assert lib.qamw_default_block(0) == 0


def test_sizes(lib):
    assert lib.qamw_index_bytes(11) > 0 and lib.qamw_index_bytes(13) == 0 and lib.qamw_index_bytes(0) == 0
    assert lib.qamw_index_bytes(11) >= lib.qamw_index_bytes(7)
    assert lib.qamw_encode_workspace(4096, 4096, 11) >= 128 * 2048 * 8
    assert lib.qamw_encode_workspace(4096, 4095, 11) == 0
    assert lib.qamw_train_workspace(1 << 20, 11) >= 3 * 2048 * 8


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _enc(lib, **kw):
    a = dict(w=FAKE, dt=q.BF16, d_out=16, d_in=256, ld=256, scale=None, seed=q.DEFAULT_SIGN_SEED, block=64, cb=FAKE,
             bits=8, index=FAKE, sig_in=FAKE, sig_out=None, norm=FAKE, codes=FAKE, status=None, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.qamw_encode(a["w"], a["dt"], a["d_out"], a["d_in"], a["ld"], a["scale"], a["block"], a["seed"],
                           a["cb"], a["bits"], a["index"], a["sig_in"], a["sig_out"], a["norm"], a["codes"],
                           a["status"], a["ws"], a["ws_bytes"], None)


def _dec(lib, **kw):
    a = dict(codes=FAKE, norm=FAKE, sigma=FAKE, cb=FAKE, bits=8, scale=None, seed=q.DEFAULT_SIGN_SEED, d_out=16,
             d_in=256, block=64, out=FAKE, dt=q.BF16, ld=256)
    a.update(kw)
    return lib.qamw_decode(a["codes"], a["norm"], a["sigma"], a["cb"], a["bits"], a["scale"], a["d_out"], a["d_in"],
                           a["block"], a["seed"], a["out"], a["dt"], a["ld"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d_in=255, ld=255), ARG), (dict(d_in=0), ARG), (dict(d_out=-1), ARG), (dict(dt=7), ARG),
    (dict(block=3), ARG), (dict(block=48), ARG), (dict(block=2048), ARG), (dict(block=512), ARG),
    (dict(ld=128), ARG), (dict(bits=0), ARG), (dict(bits=17), ARG), (dict(bits=13), UNSUP),
    (dict(sig_in=None, sig_out=None), ARG), (dict(w=None), ARG), (dict(codes=None), ARG),
    (dict(index=None), ARG), (dict(codes=FAKE + 2), ARG), (dict(cb=FAKE + 4), ARG), (dict(w=FAKE + 1), ARG),
    (dict(sig_in=None, sig_out=FAKE, ws=None), WS), (dict(sig_in=None, sig_out=FAKE, ws=FAKE, ws_bytes=64), WS),
    (dict(d_in=16384 + 256, ld=16384 + 256, block=64), UNSUP), (dict(d_in=16384 + 256, ld=16640, block=256), UNSUP),
    (dict(d_in=24, ld=24, block=8), UNSUP), (dict(d_in=8, ld=8, block=8), UNSUP),
    (dict(d_out=1 << 30), UNSUP), (dict(d_out=2**31 - 1), UNSUP),
    # rows the decoder's LDS cannot hold at b = 1024 and K >= 2048: rejected by encode as well
    (dict(d_in=32768, ld=32768, block=1024, bits=11), UNSUP), (dict(d_in=29696, ld=29696, block=1024, bits=12), UNSUP),
])
def test_encode_rejects(lib, kw, code):
    assert _enc(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(d_in=255), ARG), (dict(block=12), ARG), (dict(ld=255), ARG), (dict(ld=128), ARG), (dict(dt=3), ARG),
    (dict(bits=14), UNSUP), (dict(bits=0), ARG), (dict(codes=None), ARG), (dict(out=FAKE + 2), ARG),
    (dict(out=FAKE + 4, dt=q.F32), ARG), (dict(sigma=None), ARG), (dict(d_out=-3), ARG),
    (dict(d_in=40, ld=40, block=8), UNSUP), (dict(d_out=1 << 30), UNSUP),
    (dict(d_in=32768, ld=32768, block=1024, bits=11), UNSUP),
])
def test_decode_rejects(lib, kw, code):
    assert _dec(lib, **kw) == code


def test_empty_decode_is_a_noop(lib):
    assert _dec(lib, d_out=0, codes=None, norm=None, sigma=None, cb=None, out=None) == q.OK


def _job(**kw):
    a = dict(d_codes=FAKE, d_norm_f16=FAKE, d_sigma=FAKE, d_scale=None, d_out=16, d_in=256,
             sign_seed=q.DEFAULT_SIGN_SEED, d_out_w=FAKE, ld_out=256)
    a.update(kw)
    return q.DecodeJob(**a)


def _many(lib, jobs, bits=8, block=128, dt=q.BF16, cb=FAKE):
    arr = (q.DecodeJob * max(1, len(jobs)))(*jobs)
    return lib.qamw_decode_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), cb, bits, block, dt, None)


def test_decode_many_checks_every_job_before_queueing(lib):
    assert ctypes.sizeof(q.DecodeJob) == 64
    assert lib.qamw_decode_many(None, 0, FAKE, 8, 128, q.BF16, None) == q.OK
    assert lib.qamw_decode_many(None, 2, FAKE, 8, 128, q.BF16, None) == ARG
    assert lib.qamw_decode_many(None, -1, FAKE, 8, 128, q.BF16, None) == ARG
    # the first job would launch if it were alone: the later failing job returns its error first
    # (a launch with these placeholder pointers would fail as a HIP error on a machine without a GPU)
    assert _many(lib, [_job(), _job(d_in=255)]) == ARG
    assert _many(lib, [_job(), _job(ld_out=128)]) == ARG
    assert _many(lib, [_job(), _job(d_codes=FAKE + 2)]) == ARG
    assert _many(lib, [_job(), _job(d_out=1 << 30)]) == UNSUP
    assert _many(lib, [_job(), _job()], bits=13) == UNSUP
    assert _many(lib, [_job(), _job()], dt=5) == ARG
    assert _many(lib, [_job(), _job()], cb=None) == ARG
    assert _many(lib, [_job(d_out=0, d_codes=None, d_norm_f16=None, d_sigma=None, d_out_w=None)]) == q.OK


def test_train_and_index_reject(lib):
    assert lib.qamw_codebook_train(FAKE, 100, 8, 5, None, FAKE, None, None, FAKE, 1 << 20, None) == ARG  # n < K
    assert lib.qamw_codebook_train(FAKE, 1000, 8, -1, None, FAKE, None, None, FAKE, 1 << 20, None) == ARG
    assert lib.qamw_codebook_train(FAKE, 1000, 13, 5, None, FAKE, None, None, FAKE, 1 << 20, None) == UNSUP
    assert lib.qamw_codebook_train(FAKE, 1000, 8, 5, None, FAKE, None, None, FAKE, 16, None) == WS
    assert lib.qamw_codebook_train(FAKE + 4, 1000, 8, 5, None, FAKE, None, None, FAKE, 1 << 20, None) == ARG
    assert lib.qamw_codebook_index(FAKE, 11, FAKE, 100, None) == WS
    assert lib.qamw_codebook_index(FAKE, 11, FAKE + 8, 1 << 24, None) == WS
    assert lib.qamw_codebook_index(None, 11, FAKE, 1 << 24, None) == ARG
    assert lib.qamw_nearest(FAKE, -1, FAKE, 8, FAKE, FAKE, None) == ARG
    assert lib.qamw_nearest(None, 0, None, 8, None, None, None) == q.OK


def test_status_strings(lib):
    for c in (0, -1, -2, -3, -4, 99):
        assert isinstance(q.status_string(c), str) and q.status_string(c)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        q.load(str(tmp_path / "missing.so"))


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.dirname(q.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in text.lower(), f


def _encp(lib, **kw):
    a = dict(w=FAKE, dt=q.BF16, d_out=16, d_in=256, ld=256, scale=None, seed=q.DEFAULT_SIGN_SEED, block=64, ba=5,
             bp=6, thr=FAKE, sig_in=FAKE, sig_out=None, norm=FAKE, codes=FAKE, status=None, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.qamw_encode_polar(a["w"], a["dt"], a["d_out"], a["d_in"], a["ld"], a["scale"], a["block"], a["seed"],
                                 a["ba"], a["bp"], a["thr"], a["sig_in"], a["sig_out"], a["norm"], a["codes"],
                                 a["status"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ba=0), ARG), (dict(bp=0), ARG), (dict(ba=9, bp=1), UNSUP), (dict(ba=6, bp=7), UNSUP),
    (dict(ba=8, bp=9), ARG), (dict(thr=None), ARG), (dict(thr=FAKE + 4), ARG), (dict(d_in=255, ld=255), ARG),
    (dict(w=None), ARG), (dict(codes=FAKE + 2), ARG), (dict(sig_in=None, sig_out=FAKE, ws=None), WS),
    (dict(d_in=24, ld=24, block=8), UNSUP), (dict(d_out=1 << 30), UNSUP),
])
def test_encode_polar_rejects(lib, kw, code):
    assert _encp(lib, **kw) == code


def test_polar_codebook_and_index_reject(lib):
    assert lib.qamw_polar_codebook(0, 4, FAKE, FAKE, FAKE, None) == ARG
    assert lib.qamw_polar_codebook(9, 1, FAKE, FAKE, FAKE, None) == UNSUP
    assert lib.qamw_polar_codebook(4, 9, FAKE, FAKE, FAKE, None) == UNSUP
    assert lib.qamw_polar_codebook(4, 4, None, FAKE, FAKE, None) == ARG
    assert lib.qamw_polar_codebook(4, 4, FAKE, FAKE + 4, FAKE, None) == ARG
    assert lib.qamw_polar_index(FAKE, -1, 4, 4, FAKE, FAKE, None, None) == ARG
    assert lib.qamw_polar_index(FAKE, 10, 4, 4, None, FAKE, None, None) == ARG
    assert lib.qamw_polar_index(FAKE + 4, 10, 4, 4, FAKE, FAKE, None, None) == ARG
    assert lib.qamw_polar_index(None, 0, 4, 4, None, None, None, None) == q.OK


def _qg(lib, **kw):
    a = dict(x=FAKE, xt=q.BF16, M=4, ld_x=256, codes=FAKE, norm=FAKE, sigma=FAKE, cb=FAKE, bits=8, scale=None,
             seed=q.DEFAULT_SIGN_SEED, d_out=16, d_in=256, block=64, y=FAKE, yt=q.F32, ld_y=16, ws=FAKE,
             ws_bytes=1 << 20)
    a.update(kw)
    return lib.qamw_qgemm(a["x"], a["xt"], a["M"], a["ld_x"], a["codes"], a["norm"], a["sigma"], a["cb"], a["bits"],
                          a["scale"], a["d_out"], a["d_in"], a["block"], a["seed"], a["y"], a["yt"], a["ld_y"],
                          a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), ARG), (dict(xt=5), ARG), (dict(yt=5), ARG), (dict(d_in=255, ld_x=255), ARG), (dict(block=48), ARG),
    (dict(block=2048), ARG), (dict(bits=0), ARG), (dict(bits=13), UNSUP), (dict(M=17), UNSUP), (dict(ld_x=128), ARG),
    (dict(ld_y=8), ARG), (dict(x=None), ARG), (dict(codes=None), ARG), (dict(y=FAKE + 2), ARG),
    (dict(x=FAKE + 1), ARG), (dict(ws=None), WS), (dict(ws=FAKE + 16), WS), (dict(ws_bytes=64), WS),
    (dict(d_out=1 << 30, ld_y=1 << 30), UNSUP),
])
def test_qgemm_rejects(lib, kw, code):
    assert _qg(lib, **kw) == code


def test_qgemm_noops_and_workspace(lib):
    assert _qg(lib, M=0, x=None, y=None, ws=None) == q.OK
    assert _qg(lib, d_out=0, codes=None, norm=None, ws=None) == q.OK
    assert lib.qamw_qgemm_workspace(0, 16, 256) >= 0
    # the B operands: 8 KiB per chunk of 128 pairs and operand group (one group up to 8 rows, two
    # above)
    assert lib.qamw_qgemm_workspace(1, 4096, 4096) == 16 * 8192
    assert lib.qamw_qgemm_workspace(16, 5120, 13824) == 54 * 2 * 8192
    assert lib.qamw_qgemm_workspace(8, 5120, 1000) == 4 * 8192
    assert lib.qamw_qgemm_workspace(1, 16, 255) == 0


def test_qgemm_column_limit(lib):
    """Rows wider than QAMW_QGEMM_MAX_COLS (2^24) are refused before any HIP call: the product's
    buffer offsets are 32-bit."""
    big = (1 << 24) + 64
    assert _qg(lib, d_in=big, ld_x=big) == UNSUP
    assert _qg(lib, d_in=(1 << 24), ld_x=(1 << 24), ws=None) == WS


def test_qgemm_noalloc_checks_and_size_limit(lib):
    """The static-workspace product checks its arguments as qamw_qgemm does and refuses shapes
    whose workspace exceeds the library's array, before any HIP call."""
    assert q.QGEMM_NOALLOC_BYTES == 4 << 20
    base = dict(x=FAKE, xd=q.BF16, M=4, ldx=4096, codes=FAKE, norm=FAKE, sigma=FAKE, cb=FAKE, bits=11, scale=None,
                d_out=4096, d_in=4096, block=128, seed=q.DEFAULT_SIGN_SEED, y=FAKE, yd=q.F32, ldy=4096)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.qamw_qgemm_noalloc(a["x"], a["xd"], a["M"], a["ldx"], a["codes"], a["norm"], a["sigma"], a["cb"],
                                      a["bits"], a["scale"], a["d_out"], a["d_in"], a["block"], a["seed"], a["y"],
                                      a["yd"], a["ldy"], None)
    assert call(M=17) == UNSUP and call(bits=13) == UNSUP and call(block=3) == ARG and call(codes=None) == ARG
    assert call(M=0) == q.OK and call(d_out=0) == q.OK
    big = 131072   # 16 x 131072 activations need 8 MiB of B operands
    assert lib.qamw_qgemm_workspace(16, 64, big) > q.QGEMM_NOALLOC_BYTES
    assert call(M=16, d_in=big, ldx=big, d_out=64, ldy=64, block=1024) == WS
    assert lib.qamw_qgemm_workspace(16, 28672, 65536) == q.QGEMM_NOALLOC_BYTES


def test_scalar_codebook_rejects(lib):
    assert lib.qamw_scalar_codebook(0, FAKE, FAKE, FAKE, None) == ARG
    assert lib.qamw_scalar_codebook(9, FAKE, FAKE, FAKE, None) == ARG
    assert lib.qamw_scalar_codebook(7, FAKE, FAKE, FAKE, None) == UNSUP
    assert lib.qamw_scalar_codebook(4, None, FAKE, FAKE, None) == ARG
    assert lib.qamw_scalar_codebook(4, FAKE, FAKE, FAKE + 4, None) == ARG


def test_act_scale_rejects(lib):
    import math
    ok = dict(x=FAKE, dt=q.BF16, T=16, d=64, ld=64, a=0.3, s=FAKE, r=None, ws=FAKE, wsb=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.qamw_act_scale(a["x"], a["dt"], a["T"], a["d"], a["ld"], a["a"], a["s"], a["r"], a["ws"], a["wsb"], None)
    assert call(T=0) == ARG and call(d=0) == ARG and call(ld=32) == ARG and call(dt=9) == ARG
    assert call(a=math.inf) == ARG and call(a=math.nan) == ARG and call(x=None) == ARG and call(s=FAKE + 2) == ARG
    assert call(x=FAKE + 1) == ARG and call(r=FAKE + 4) == ARG
    assert call(ws=None) == WS and call(wsb=8) == WS
    assert lib.qamw_act_scale_workspace(2048, 4096) >= 4096 * 8 and lib.qamw_act_scale_workspace(0, 8) == 0


def test_sign_mask_rejects(lib):
    assert lib.qamw_sign_mask(1, -1, FAKE, None) == ARG
    assert lib.qamw_sign_mask(1, 64, None, None) == ARG
    assert lib.qamw_sign_mask(1, 64, FAKE + 2, None) == ARG
    assert lib.qamw_sign_mask(1, 0, None, None) == q.OK


def test_header_default_seed_matches_binding():
    import re
    text = open(q.HEADER_PATH).read()
    m = re.search(r"#define QAMW_DEFAULT_SIGN_SEED (0x[0-9A-Fa-f]+)ull", text)
    assert m and int(m.group(1), 16) == q.DEFAULT_SIGN_SEED
    m = re.search(r"#define QAMW_QGEMM_NOALLOC_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == q.QGEMM_NOALLOC_BYTES


# ----------------------------------------------------------------------------- binding argument checks
# The library trusts the sizes it is given, so the binding checks every tensor against the shape the
# call implies before a pointer is passed.  These calls use host tensors: each must be rejected by a
# size or dtype check (a ValueError naming the argument), before the device check.

import torch  # noqa: E402


def _bad(fn, match, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_binding_rejects_short_or_mistyped_buffers(lib):
    d_out, d_in, bits = 8, 256, 8
    stride = q.row_stride(d_in, bits)
    codes = torch.zeros((d_out, stride), dtype=torch.uint8)
    norm = torch.zeros((d_out,), dtype=torch.int16)
    sigma = torch.zeros((d_in // 2,), dtype=torch.float32)
    cb = torch.zeros((1 << bits, 2), dtype=torch.float32)
    # decode
    _bad(q.decode, "codes", codes[:, :-16], norm, sigma, cb, bits, d_in)
    _bad(q.decode, "codes", codes[:-1], norm, sigma, cb, bits, d_in)
    _bad(q.decode, "sigma", codes, norm, sigma[:-1], cb, bits, d_in)
    _bad(q.decode, "sigma", codes, norm, sigma.double(), cb, bits, d_in)
    _bad(q.decode, "codebook", codes, norm, sigma, cb[:-1], bits, d_in)
    _bad(q.decode, "codes", codes, norm, sigma, cb, bits + 1, d_in)   # the stride of 9-bit codes
    _bad(q.decode, "norm", codes, norm.float(), sigma, cb, bits, d_in)
    _bad(q.decode, "scale", codes, norm, sigma, cb, bits, d_in, scale=torch.ones(d_in - 1))
    _bad(q.decode, "out", codes, norm, sigma, cb, bits, d_in, out=torch.zeros((d_out, d_in - 2), dtype=torch.bfloat16))
    _bad(q.decode, "device", codes, norm, sigma, cb, bits, d_in)   # all sizes right: the device check
    # encode
    w = torch.zeros((d_out, d_in), dtype=torch.bfloat16)
    index = torch.zeros((q.index_bytes(bits),), dtype=torch.uint8)
    _bad(q.encode, "index", w, cb, bits, index[:-1])
    _bad(q.encode, "codebook", w, cb[:3], bits, index)
    _bad(q.encode, "w", w.to(torch.float16), cb, bits, index)
    _bad(q.encode, "scale", w, cb, bits, index, scale=torch.ones(d_in // 2))
    _bad(q.encode, "sigma", w, cb, bits, index, sigma=torch.ones(d_in // 4))
    _bad(q.encode, "status", w, cb, bits, index, status=torch.zeros(1, dtype=torch.int64))
    _bad(q.encode, "codes", w, cb, bits, index, out={"codes": torch.zeros((d_out, stride - 16), dtype=torch.uint8)})
    # fused product, polar, nearest, training
    _bad(q.qgemm, "codes", torch.zeros((2, d_in + 2)), codes, norm, sigma, cb, bits)   # x's width sets d_in
    _bad(q.qgemm, "x", torch.zeros((2, d_in), dtype=torch.float16), codes, norm, sigma, cb, bits)
    _bad(q.qgemm, "out", torch.zeros((2, d_in)), codes, norm, sigma, cb, bits, out=torch.zeros((2, d_out + 1)))
    _bad(q.encode_polar, "thresholds", w, 4, 4, torch.zeros(14, dtype=torch.float64))
    _bad(q.polar_index, "thresholds", torch.zeros((4, 2)), 4, 4, torch.zeros(15, dtype=torch.float32))
    _bad(q.nearest, "index", torch.zeros((4, 2)), cb, bits, index[:10])
    _bad(q.nearest, "pairs", torch.zeros((5,)), cb, bits, index)
    _bad(q.codebook_train, "init", torch.zeros((1024, 2)), bits, 3, init=cb[:10])


def test_encode_and_decode_accept_the_same_wide_rows(lib):
    """Every (d_in, block, bits) the encoder accepts, the decoder accepts (checked on the host
    rules alone, with d_out = 0 so nothing is launched)."""
    for block in (128, 256, 512, 1024):
        for bits in (7, 8, 11, 12):
            for d_in in range(block, 32768 + 1, block if block >= 1024 else 4 * block):
                e = _enc(lib, d_out=0, d_in=d_in, ld=d_in, block=block, bits=bits, w=None, codes=None, norm=None)
                d = _dec(lib, d_out=0, d_in=d_in, ld=d_in, block=block, bits=bits)
                assert (e == q.OK) == (d == q.OK), (d_in, block, bits, e, d)
