"""qamw_qgemm_noalloc, the fused product for callers that cannot allocate: through the C ABI, its
output equals qamw_qgemm's (same kernels, workspace in the library's static array instead of the
caller's) bit for bit, on two calls in a row, the second on a smaller input, so that the second
call runs over what the first left in the array."""
import ctypes

import numpy as np
import pytest
import torch

import weight_quantization_codec_amd as q
from helpers import DEV, log

pytestmark = pytest.mark.gpu


def _inputs(rng, M, d_out, d_in, bits, x_dtype):
    codes = rng.integers(0, 256, size=(d_out, q.row_stride(d_in, bits)), dtype=np.uint8)
    norm = rng.uniform(0.25, 4.0, size=d_out).astype(np.float16)
    norm[min(3, d_out - 1)] = 0
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return dict(
        x=dev(rng.standard_normal((M, d_in)).astype(np.float32)).to(x_dtype),
        codes=dev(codes), norm=dev(norm.view(np.int16)),
        sigma=dev(rng.uniform(0.5, 1.5, size=d_in // 2).astype(np.float32)),
        cb=dev(rng.standard_normal((1 << bits, 2)).astype(np.float32)),
        scale=dev((np.abs(rng.standard_normal(d_in)) ** 0.5 + 0.1).astype(np.float32)),
        seed=int(rng.integers(0, 2**62)), M=M, d_out=d_out, d_in=d_in, bits=bits)


def _dt(t):
    return q.BF16 if t.dtype == torch.bfloat16 else q.F32


def _both(lib, a, block, y_dtype):
    """(y from qamw_qgemm with a caller workspace, y from qamw_qgemm_noalloc)."""
    M, d_out, d_in = a["M"], a["d_out"], a["d_in"]
    st = torch.cuda.current_stream().cuda_stream
    ws = torch.empty((lib.qamw_qgemm_workspace(M, d_out, d_in),), dtype=torch.uint8, device=DEV)
    y_ref = torch.full((M, d_out), 5.0, dtype=y_dtype, device=DEV)
    y_new = torch.full((M, d_out), 7.0, dtype=y_dtype, device=DEV)
    common = (a["x"].data_ptr(), _dt(a["x"]), M, d_in, a["codes"].data_ptr(), a["norm"].data_ptr(),
              a["sigma"].data_ptr(), a["cb"].data_ptr(), a["bits"], a["scale"].data_ptr(), d_out, d_in, block,
              a["seed"])
    rc = lib.qamw_qgemm(*common, y_ref.data_ptr(), _dt(y_ref), d_out, ws.data_ptr(), ws.numel(), st)
    assert rc == q.OK, q.status_string(rc)
    rc = lib.qamw_qgemm_noalloc(*common, y_new.data_ptr(), _dt(y_new), d_out, st)
    assert rc == q.OK, q.status_string(rc)
    torch.cuda.synchronize()
    return y_ref, y_new


def _same(y_ref, y_new):
    iv = torch.int16 if y_ref.dtype == torch.bfloat16 else torch.int32
    return int((y_ref.view(iv) != y_new.view(iv)).sum())


def test_noalloc_equals_workspace_call_twice():
    lib = q.load()
    rng = np.random.default_rng(2024)
    # first call: 16 activation rows on a 13B down-projection (the matrix-core path, 864 KiB of
    # rotated fragments in the array)
    a = _inputs(rng, 16, 5120, 13824, 11, torch.bfloat16)
    log("qgemm_noalloc call 1: M=16 5120 x 13824 bits 11")
    y_ref, y_new = _both(lib, a, 128, torch.float32)
    assert _same(y_ref, y_new) == 0
    assert torch.isfinite(y_new).all()
    # second call, smaller: 3 rows (the vector-unit path), 300 x 1024, 8-bit indices, BF16 out
    b = _inputs(rng, 3, 300, 1024, 8, torch.float32)
    log("qgemm_noalloc call 2: M=3 300 x 1024 bits 8")
    y_ref, y_new = _both(lib, b, 0, torch.bfloat16)
    assert _same(y_ref, y_new) == 0
    assert not bool((y_new.float() == 7.0).all())


def test_noalloc_refuses_oversized_shapes_and_leaves_output():
    lib = q.load()
    big = 131072
    assert lib.qamw_qgemm_workspace(16, 64, big) > q.QGEMM_NOALLOC_BYTES
    y = torch.full((16, 64), 7.0, dtype=torch.float32, device=DEV)
    x = torch.zeros((16, big), dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros((64, q.row_stride(big, 8)), dtype=torch.uint8, device=DEV)
    norm = torch.zeros((64,), dtype=torch.int16, device=DEV)
    sigma = torch.ones((big // 2,), dtype=torch.float32, device=DEV)
    cb = torch.zeros((256, 2), dtype=torch.float32, device=DEV)
    rc = lib.qamw_qgemm_noalloc(x.data_ptr(), q.BF16, 16, big, codes.data_ptr(), norm.data_ptr(), sigma.data_ptr(),
                                cb.data_ptr(), 8, None, 64, big, 1024, q.DEFAULT_SIGN_SEED, y.data_ptr(), q.F32, 64,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == q.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
