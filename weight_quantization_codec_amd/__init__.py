"""MI355X-native QAM-W weight codec: a thin ctypes binding over libqamw.so.

The binding only marshals arguments: it allocates outputs with torch on the current HIP
device, passes raw device pointers and the current stream to the C ABI (include/qamw.h), and
raises on a non-zero return code.  Every step of encode, decode and codebook training runs in
the library's HIP kernels; there is no CPU path.  If libqamw.so has not been built, importing
works but every call raises.

QAM-W is defined in "QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
Rotation and Activation-Aware Scaling" (Sharma and Dobek), section 3.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libqamw.so")
HEADER_PATH = os.path.join(ROOT, "include", "qamw.h")

F32, BF16 = 0, 1
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
FLAG_NONFINITE, FLAG_BAD_SCALE, FLAG_NORM_RANGE, FLAG_POINT_RANGE, FLAG_BAD_THRESHOLDS = 1, 2, 4, 8, 16


class QamwError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, status_string(code), code))


_lib = None


def load(path: Optional[str] = None):
    """Load libqamw.so (raises if it is missing: build it with __graft_entry__.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libqamw.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "qamw_row_stride": ([i32, i32], sz),
        "qamw_default_block": ([i32], i32),
        "qamw_index_bytes": ([i32], sz),
        "qamw_encode_workspace": ([i32, i32, i32], sz),
        "qamw_train_workspace": ([i64, i32], sz),
        "qamw_codebook_train": ([vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "qamw_codebook_index": ([vp, i32, vp, sz, vp], ctypes.c_int),
        "qamw_nearest": ([vp, i64, vp, i32, vp, vp, vp], ctypes.c_int),
        "qamw_encode": ([vp, ctypes.c_int, i32, i32, i64, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
                        ctypes.c_int),
        "qamw_decode": ([vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, vp, ctypes.c_int, i64, vp], ctypes.c_int),
        "qamw_qgemm_workspace": ([i32, i32, i32], sz),
        "qamw_qgemm": ([vp, ctypes.c_int, i32, i64, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, vp, ctypes.c_int, i64,
                        vp, sz, vp], ctypes.c_int),
        "qamw_polar_codebook": ([i32, i32, vp, vp, vp, vp], ctypes.c_int),
        "qamw_polar_index": ([vp, i64, i32, i32, vp, vp, vp, vp], ctypes.c_int),
        "qamw_scalar_codebook": ([i32, vp, vp, vp, vp], ctypes.c_int),
        "qamw_act_scale_workspace": ([i64, i32], sz),
        "qamw_act_scale": ([vp, ctypes.c_int, i64, i32, i64, ctypes.c_double, vp, vp, vp, sz, vp], ctypes.c_int),
        "qamw_encode_polar": ([vp, ctypes.c_int, i32, i32, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz,
                               vp], ctypes.c_int),
        "qamw_status_string": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def header_symbols() -> list:
    """Names of the functions declared in include/qamw.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qamw_[a-z0-9_]+)\s*\(", text)))


# ----------------------------------------------------------------------------- helpers

def status_string(code: int) -> str:
    return load().qamw_status_string(code).decode()


def row_stride(d_in: int, bits: int) -> int:
    return load().qamw_row_stride(d_in, bits)


def default_block(d_in: int) -> int:
    return load().qamw_default_block(d_in)


def index_bytes(bits: int) -> int:
    return load().qamw_index_bytes(bits)


def encode_workspace(d_out: int, d_in: int, bits: int) -> int:
    return load().qamw_encode_workspace(d_out, d_in, bits)


def train_workspace(n_points: int, bits: int) -> int:
    return load().qamw_train_workspace(n_points, bits)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(rc: int, where: str):
    if rc != OK:
        raise QamwError(rc, where)


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty((max(int(nbytes), 16),), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- entry points

def codebook_train(points: torch.Tensor, bits: int, iters: int, init: Optional[torch.Tensor] = None,
                   status: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Lloyd codebook (section 3.6 eq. 2).  Returns (codebook K x 2 fp32, trace int64[iters])."""
    _dev(points, torch.float32, "points")
    n = points.numel() // 2
    dev = points.device
    cb = torch.empty((1 << bits, 2), dtype=torch.float32, device=dev)
    trace = torch.zeros((max(iters, 1),), dtype=torch.int64, device=dev)
    if init is not None:
        _dev(init, torch.float32, "init")
    nb = train_workspace(n, bits)
    ws = workspace if workspace is not None else _ws(nb, dev)
    rc = load().qamw_codebook_train(_ptr(points), n, bits, iters, _ptr(init), _ptr(cb), _ptr(trace), _ptr(status),
                                    _ptr(ws), ws.numel(), _stream())
    _check(rc, "qamw_codebook_train")
    return cb, trace[:iters]


def codebook_index(codebook: torch.Tensor, bits: int) -> torch.Tensor:
    """Nearest-codeword search index of a codebook (device byte buffer)."""
    _dev(codebook, torch.float32, "codebook")
    idx = torch.empty((index_bytes(bits),), dtype=torch.uint8, device=codebook.device)
    rc = load().qamw_codebook_index(_ptr(codebook), bits, _ptr(idx), idx.numel(), _stream())
    _check(rc, "qamw_codebook_index")
    return idx


def nearest(points: torch.Tensor, codebook: torch.Tensor, bits: int, index: torch.Tensor) -> torch.Tensor:
    _dev(points, torch.float32, "points")
    n = points.numel() // 2
    out = torch.empty((n,), dtype=torch.int32, device=points.device)
    rc = load().qamw_nearest(_ptr(points), n, _ptr(codebook), bits, _ptr(index), _ptr(out), _stream())
    _check(rc, "qamw_nearest")
    return out


def _encode_buffers(w, bits, scale, sign_bits, sigma, workspace, out):
    if w.dtype not in (torch.bfloat16, torch.float32) or not w.is_cuda or w.dim() != 2:
        raise ValueError("w must be a 2-D bf16 or fp32 device tensor")
    d_out, d_in = w.shape
    if d_out > 0 and w.stride(1) != 1:
        raise ValueError("w rows must be contiguous")
    ld = w.stride(0) if d_out > 0 else d_in
    dev = w.device
    stride = row_stride(d_in, bits)
    if out is None:
        out = {}
    codes = out.get("codes")
    if codes is None:
        codes = torch.empty((d_out, stride), dtype=torch.uint8, device=dev)
    norm = out.get("norm")
    if norm is None:
        norm = torch.empty((d_out,), dtype=torch.int16, device=dev)
    sig_out = out.get("sigma")
    if sig_out is None and sigma is None:
        sig_out = torch.empty((d_in // 2,), dtype=torch.float32, device=dev)
    if sigma is not None:
        sig_out = None   # the given sigma is used as is; nothing is copied
    if scale is not None:
        _dev(scale, torch.float32, "scale")
    if sign_bits is not None:
        _dev(sign_bits, torch.int32, "sign_bits")
    if sigma is not None:
        _dev(sigma, torch.float32, "sigma")
    ws = workspace
    if ws is None and sigma is None:
        ws = _ws(encode_workspace(d_out, d_in, bits), dev)
    return d_out, d_in, ld, codes, norm, sig_out, ws


def encode(w: torch.Tensor, codebook: torch.Tensor, bits: int, index: torch.Tensor,
           scale: Optional[torch.Tensor] = None, sign_bits: Optional[torch.Tensor] = None, block: int = 0,
           sigma: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None
           ) -> Dict[str, torch.Tensor]:
    """Encode W (d_out x d_in, bf16 or fp32) -> {codes, norm (int16 bit patterns of f16), sigma}."""
    d_out, d_in, ld, codes, norm, sig_out, ws = _encode_buffers(w, bits, scale, sign_bits, sigma, workspace, out)
    rc = load().qamw_encode(_ptr(w), BF16 if w.dtype == torch.bfloat16 else F32, d_out, d_in, ld,
                            _ptr(scale), _ptr(sign_bits), block, _ptr(codebook), bits, _ptr(index), _ptr(sigma),
                            _ptr(sig_out), _ptr(norm), _ptr(codes), _ptr(status), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream())
    _check(rc, "qamw_encode")
    return {"codes": codes, "norm": norm, "sigma": sigma if sigma is not None else sig_out}


def qgemm_workspace(M: int, d_out: int, d_in: int) -> int:
    return load().qamw_qgemm_workspace(M, d_out, d_in)


def qgemm(x: torch.Tensor, codes: torch.Tensor, norm: torch.Tensor, sigma: torch.Tensor, codebook: torch.Tensor,
          bits: int, scale: Optional[torch.Tensor] = None, sign_bits: Optional[torch.Tensor] = None, block: int = 0,
          out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W^T (section 1) with W the decoder's weights, W never formed.  x: M x d_in (bf16/fp32)."""
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dtype not in (torch.bfloat16, torch.float32) or not x.is_cuda or x.dim() != 2:
        raise ValueError("x must be an M x d_in bf16 or fp32 device tensor")
    M, d_in = x.shape
    if M > 0 and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    _dev(codes, torch.uint8, "codes")
    d_out = norm.numel()
    if out is None:
        out = torch.empty((M, d_out), dtype=out_dtype, device=x.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or (M > 0 and out.stride(1) != 1):
        raise ValueError("out must be a bf16 or fp32 tensor with contiguous rows")
    ws = workspace
    if ws is None:
        ws = _ws(qgemm_workspace(M, d_out, d_in), x.device)
    rc = load().qamw_qgemm(_ptr(x), BF16 if x.dtype == torch.bfloat16 else F32, M, x.stride(0) if M > 0 else d_in,
                           _ptr(codes), _ptr(norm), _ptr(sigma), _ptr(codebook), bits, _ptr(scale),
                           _ptr(sign_bits), d_out, d_in, block, _ptr(out),
                           BF16 if out.dtype == torch.bfloat16 else F32, out.stride(0) if M > 0 else d_out,
                           _ptr(ws), ws.numel(), _stream())
    _check(rc, "qamw_qgemm")
    return out


def polar_codebook(ba: int, bp: int, device=None):
    """Polar baseline (section 3.5): (levels float64[2^ba], thresholds float64[2^ba - 1],
    table float32[2^(ba+bp), 2]) on the current (or given) device."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    na = 1 << ba
    levels = torch.empty((na,), dtype=torch.float64, device=dev)
    thr = torch.empty((max(na - 1, 1),), dtype=torch.float64, device=dev)
    table = torch.empty((na << bp, 2), dtype=torch.float32, device=dev)
    rc = load().qamw_polar_codebook(ba, bp, _ptr(levels), _ptr(thr), _ptr(table), _stream())
    _check(rc, "qamw_polar_codebook")
    return levels, thr[: na - 1], table


def act_scale(x: torch.Tensor, alpha: float = 0.3, want_rms: bool = False, workspace: Optional[torch.Tensor] = None):
    """Activation-aware channel scale s_j = r_j^alpha from T x d_in calibration activations (bf16/fp32).
    Returns s (fp32[d_in]), or (s, r fp64[d_in]) with want_rms."""
    if x.dtype not in (torch.bfloat16, torch.float32) or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a T x d_in bf16 or fp32 device tensor with contiguous rows")
    T, d_in = x.shape
    s = torch.empty((d_in,), dtype=torch.float32, device=x.device)
    r = torch.empty((d_in,), dtype=torch.float64, device=x.device) if want_rms else None
    ws = workspace if workspace is not None else _ws(load().qamw_act_scale_workspace(T, d_in), x.device)
    rc = load().qamw_act_scale(_ptr(x), BF16 if x.dtype == torch.bfloat16 else F32, T, d_in, x.stride(0), float(alpha),
                               _ptr(s), _ptr(r), _ptr(ws), ws.numel(), _stream())
    _check(rc, "qamw_act_scale")
    return (s, r) if want_rms else s


def scalar_codebook(b: int, device=None):
    """Scalar (d = 1) ablation (section 2): (levels float64[2^b], thresholds float64[2^b - 1],
    product table float32[2^(2b), 2]) for qamw_codebook_index / encode / decode with bits = 2b."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    L = 1 << b
    levels = torch.empty((L,), dtype=torch.float64, device=dev)
    thr = torch.empty((L - 1,), dtype=torch.float64, device=dev)
    table = torch.empty((L * L, 2), dtype=torch.float32, device=dev)
    rc = load().qamw_scalar_codebook(b, _ptr(levels), _ptr(thr), _ptr(table), _stream())
    _check(rc, "qamw_scalar_codebook")
    return levels, thr, table


def polar_index(points: torch.Tensor, ba: int, bp: int, thresholds: torch.Tensor,
                status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Polar indices (section 3.5) of n fp32 pairs (n x 2)."""
    _dev(points, torch.float32, "points")
    _dev(thresholds, torch.float64, "thresholds")
    n = points.numel() // 2
    out = torch.empty((n,), dtype=torch.int32, device=points.device)
    rc = load().qamw_polar_index(_ptr(points), n, ba, bp, _ptr(thresholds), _ptr(out), _ptr(status), _stream())
    _check(rc, "qamw_polar_index")
    return out


def encode_polar(w: torch.Tensor, ba: int, bp: int, thresholds: torch.Tensor,
                 scale: Optional[torch.Tensor] = None, sign_bits: Optional[torch.Tensor] = None, block: int = 0,
                 sigma: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None
                 ) -> Dict[str, torch.Tensor]:
    """Polar-baseline encode (section 3.5); decode with `decode(..., table, ba + bp, ...)`."""
    _dev(thresholds, torch.float64, "thresholds")
    bits = ba + bp
    d_out, d_in, ld, codes, norm, sig_out, ws = _encode_buffers(w, bits, scale, sign_bits, sigma, workspace, out)
    rc = load().qamw_encode_polar(_ptr(w), BF16 if w.dtype == torch.bfloat16 else F32, d_out, d_in, ld,
                                  _ptr(scale), _ptr(sign_bits), block, ba, bp, _ptr(thresholds), _ptr(sigma),
                                  _ptr(sig_out), _ptr(norm), _ptr(codes), _ptr(status), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream())
    _check(rc, "qamw_encode_polar")
    return {"codes": codes, "norm": norm, "sigma": sigma if sigma is not None else sig_out}


def decode(codes: torch.Tensor, norm: torch.Tensor, sigma: torch.Tensor, codebook: torch.Tensor, bits: int,
           d_in: int, scale: Optional[torch.Tensor] = None, sign_bits: Optional[torch.Tensor] = None,
           block: int = 0, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode to a d_out x d_in bf16 (default) or fp32 tensor."""
    _dev(codes, torch.uint8, "codes")
    d_out = norm.numel()
    if out is None:
        out = torch.empty((d_out, d_in), dtype=out_dtype, device=codes.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or (d_out > 0 and out.stride(1) != 1):
        raise ValueError("out must be a bf16 or fp32 tensor with contiguous rows")
    ld_out = out.stride(0) if d_out > 0 else d_in
    rc = load().qamw_decode(_ptr(codes), _ptr(norm), _ptr(sigma), _ptr(codebook), bits, _ptr(scale),
                            _ptr(sign_bits), d_out, d_in, block, _ptr(out),
                            BF16 if out.dtype == torch.bfloat16 else F32, ld_out, _stream())
    _check(rc, "qamw_decode")
    return out
