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
FLAG_NONFINITE, FLAG_BAD_SCALE, FLAG_NORM_RANGE, FLAG_POINT_RANGE, FLAG_BAD_THRESHOLDS, FLAG_BAD_INDEX = (
    1, 2, 4, 8, 16, 32)
# seed of the rotation's sign mask when the caller gives none (QAMW_DEFAULT_SIGN_SEED of qamw.h)
DEFAULT_SIGN_SEED = 0x51414D57
# bytes of the static workspace of qamw_qgemm_noalloc (QAMW_QGEMM_NOALLOC_BYTES of qamw.h)
QGEMM_NOALLOC_BYTES = 4 << 20


class QamwError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, status_string(code), code))


_lib = None


def load(path: Optional[str] = None):
    """Load libqamw.so (raises if it is missing: build it with __graft_entry__.build()).

    Without a path this is the binding's library, loaded once.  With a path the file is loaded and
    returned but not installed: the functions of this module keep calling the binding's library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libqamw.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    vp, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    sig = {
        "qamw_row_stride": ([i32, i32], sz),
        "qamw_default_block": ([i32], i32),
        "qamw_index_bytes": ([i32], sz),
        "qamw_encode_workspace": ([i32, i32, i32], sz),
        "qamw_train_workspace": ([i64, i32], sz),
        "qamw_codebook_train": ([vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "qamw_codebook_index": ([vp, i32, vp, sz, vp], ctypes.c_int),
        "qamw_nearest": ([vp, i64, vp, i32, vp, vp, vp], ctypes.c_int),
        "qamw_encode": ([vp, ctypes.c_int, i32, i32, i64, vp, i32, u64, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
                        ctypes.c_int),
        "qamw_decode": ([vp, vp, vp, vp, i32, vp, i32, i32, i32, u64, vp, ctypes.c_int, i64, vp], ctypes.c_int),
        "qamw_decode_many": ([vp, i32, vp, i32, i32, ctypes.c_int, vp], ctypes.c_int),
        "qamw_sign_mask": ([u64, i32, vp, vp], ctypes.c_int),
        "qamw_qgemm_workspace": ([i32, i32, i32], sz),
        "qamw_qgemm": ([vp, ctypes.c_int, i32, i64, vp, vp, vp, vp, i32, vp, i32, i32, i32, u64, vp, ctypes.c_int, i64,
                        vp, sz, vp], ctypes.c_int),
        "qamw_qgemm_noalloc": ([vp, ctypes.c_int, i32, i64, vp, vp, vp, vp, i32, vp, i32, i32, i32, u64, vp,
                                ctypes.c_int, i64, vp], ctypes.c_int),
        "qamw_polar_codebook": ([i32, i32, vp, vp, vp, vp], ctypes.c_int),
        "qamw_polar_index": ([vp, i64, i32, i32, vp, vp, vp, vp], ctypes.c_int),
        "qamw_scalar_codebook": ([i32, vp, vp, vp, vp], ctypes.c_int),
        "qamw_act_scale_workspace": ([i64, i32], sz),
        "qamw_act_scale": ([vp, ctypes.c_int, i64, i32, i64, ctypes.c_double, vp, vp, vp, sz, vp], ctypes.c_int),
        "qamw_encode_polar": ([vp, ctypes.c_int, i32, i32, i64, vp, i32, u64, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz,
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


def _arg(t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None,
         shape: Optional[tuple] = None, optional: bool = False) -> Optional[torch.Tensor]:
    """Checks a tensor argument before its pointer reaches the library: dtype, size (at least
    `numel` elements, or exactly `shape`) and contiguity.  The library trusts the sizes it is
    given, so a short buffer here would be read or written past its end.  `_on_device` checks the
    device once every argument of a call has passed these checks."""
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s needs at least %d elements, got %d" % (name, numel, t.numel()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _on_device(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)


def _matrix(t: torch.Tensor, name: str, rows: Optional[int] = None, cols: Optional[int] = None,
            dtypes=(torch.bfloat16, torch.float32)) -> int:
    """A 2-D bf16/fp32 matrix with contiguous rows (any row pitch); returns its leading dimension."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.dtype not in dtypes:
        raise ValueError("%s must be a 2-D tensor of %s" % (name, dtypes))
    if (rows is not None and t.shape[0] != rows) or (cols is not None and t.shape[1] != cols):
        raise ValueError("%s must be %s x %s, got %s" % (name, rows, cols, tuple(t.shape)))
    if t.shape[0] > 0 and t.shape[1] > 0 and t.stride(1) != 1:
        raise ValueError("%s rows must be contiguous" % name)
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    if ld < t.shape[1]:
        raise ValueError("%s rows overlap" % name)
    return ld


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty((max(int(nbytes), 16),), dtype=torch.uint8, device=device)


def _dt(t: torch.Tensor) -> int:
    return BF16 if t.dtype == torch.bfloat16 else F32


# ----------------------------------------------------------------------------- entry points

def codebook_train(points: torch.Tensor, bits: int, iters: int, init: Optional[torch.Tensor] = None,
                   status: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Lloyd codebook (section 3.6 eq. 2).  Returns (codebook K x 2 fp32, trace int64[iters])."""
    _arg(points, "points", torch.float32)
    if points.numel() % 2:
        raise ValueError("points must hold (x, y) pairs")
    n = points.numel() // 2
    K = 1 << bits
    _arg(init, "init", torch.float32, numel=2 * K, optional=True)
    _arg(status, "status", torch.int32, numel=1, optional=True)
    dev = points.device
    cb = torch.empty((K, 2), dtype=torch.float32, device=dev)
    trace = torch.zeros((max(iters, 1),), dtype=torch.int64, device=dev)
    nb = train_workspace(n, bits)
    _arg(workspace, "workspace", torch.uint8, numel=nb, optional=True)
    _on_device(points=points, init=init, status=status, workspace=workspace)
    ws = workspace if workspace is not None else _ws(nb, dev)
    rc = load().qamw_codebook_train(_ptr(points), n, bits, iters, _ptr(init), _ptr(cb), _ptr(trace), _ptr(status),
                                    _ptr(ws), ws.numel(), _stream())
    _check(rc, "qamw_codebook_train")
    return cb, trace[:iters]


def codebook_index(codebook: torch.Tensor, bits: int) -> torch.Tensor:
    """Nearest-codeword search index of a codebook (device byte buffer)."""
    _arg(codebook, "codebook", torch.float32, numel=2 << bits)
    _on_device(codebook=codebook)
    idx = torch.empty((max(index_bytes(bits), 16),), dtype=torch.uint8, device=codebook.device)
    rc = load().qamw_codebook_index(_ptr(codebook), bits, _ptr(idx), idx.numel(), _stream())
    _check(rc, "qamw_codebook_index")
    return idx


def nearest(points: torch.Tensor, codebook: torch.Tensor, bits: int, index: torch.Tensor) -> torch.Tensor:
    _arg(points, "points", torch.float32)
    if points.numel() % 2:
        raise ValueError("points must hold (x, y) pairs")
    _arg(codebook, "codebook", torch.float32, numel=2 << bits)
    _arg(index, "index", torch.uint8, numel=index_bytes(bits))
    _on_device(points=points, codebook=codebook, index=index)
    n = points.numel() // 2
    out = torch.empty((n,), dtype=torch.int32, device=points.device)
    rc = load().qamw_nearest(_ptr(points), n, _ptr(codebook), bits, _ptr(index), _ptr(out), _stream())
    _check(rc, "qamw_nearest")
    return out


def sign_mask(d_in: int, sign_seed: int = DEFAULT_SIGN_SEED, device=None) -> torch.Tensor:
    """The rotation's sign mask of a seed (section 3.3) as int32 words: bit j % 32 of word j / 32 is
    set when eps_j = -1."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    out = torch.zeros((max((d_in + 31) // 32, 1),), dtype=torch.int32, device=dev)
    rc = load().qamw_sign_mask(sign_seed, d_in, _ptr(out), _stream())
    _check(rc, "qamw_sign_mask")
    return out[: (d_in + 31) // 32]


def _side_args(d_out, d_in, bits, scale, sigma, status):
    _arg(scale, "scale", torch.float32, numel=d_in, optional=True)
    _arg(sigma, "sigma", torch.float32, numel=d_in // 2, optional=True)
    _arg(status, "status", torch.int32, numel=1, optional=True)


def _encode_buffers(w, bits, scale, sigma, status, workspace, out):
    ld = _matrix(w, "w")
    d_out, d_in = w.shape
    if d_in % 2:
        raise ValueError("d_in must be even")
    _side_args(d_out, d_in, bits, scale, sigma, status)
    dev = w.device
    stride = row_stride(d_in, bits)
    if out is None:
        out = {}
    codes = out.get("codes")
    if codes is None:
        codes = torch.empty((d_out, stride), dtype=torch.uint8, device=dev)
    _arg(codes, "codes", torch.uint8, shape=(d_out, stride))
    norm = out.get("norm")
    if norm is None:
        norm = torch.empty((d_out,), dtype=torch.int16, device=dev)
    _arg(norm, "norm", torch.int16, numel=d_out)
    sig_out = out.get("sigma")
    if sig_out is None and sigma is None:
        sig_out = torch.empty((d_in // 2,), dtype=torch.float32, device=dev)
    if sigma is not None:
        sig_out = None   # the given sigma is used as is; nothing is copied
    _arg(sig_out, "out['sigma']", torch.float32, numel=d_in // 2, optional=True)
    need = encode_workspace(d_out, d_in, bits)
    _arg(workspace, "workspace", torch.uint8, numel=need if sigma is None else None, optional=True)
    _on_device(w=w, scale=scale, sigma=sigma, status=status, codes=codes, norm=norm, sig_out=sig_out,
               workspace=workspace)
    ws = workspace
    if ws is None and sigma is None:
        ws = _ws(need, dev)
    return d_out, d_in, ld, codes, norm, sig_out, ws


def encode(w: torch.Tensor, codebook: torch.Tensor, bits: int, index: torch.Tensor,
           scale: Optional[torch.Tensor] = None, sign_seed: int = DEFAULT_SIGN_SEED, block: int = 0,
           sigma: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None
           ) -> Dict[str, torch.Tensor]:
    """Encode W (d_out x d_in, bf16 or fp32) -> {codes, norm (int16 bit patterns of f16), sigma}."""
    _arg(codebook, "codebook", torch.float32, numel=2 << bits)
    _arg(index, "index", torch.uint8, numel=index_bytes(bits))
    d_out, d_in, ld, codes, norm, sig_out, ws = _encode_buffers(w, bits, scale, sigma, status, workspace, out)
    _on_device(codebook=codebook, index=index)
    rc = load().qamw_encode(_ptr(w), _dt(w), d_out, d_in, ld, _ptr(scale), block, sign_seed, _ptr(codebook), bits,
                            _ptr(index), _ptr(sigma), _ptr(sig_out), _ptr(norm), _ptr(codes), _ptr(status), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream())
    _check(rc, "qamw_encode")
    return {"codes": codes, "norm": norm, "sigma": sigma if sigma is not None else sig_out}


def _decode_inputs(codes, norm, sigma, codebook, bits, d_in, scale):
    _arg(norm, "norm", torch.int16)
    d_out = norm.numel()
    _arg(codes, "codes", torch.uint8, shape=(d_out, row_stride(d_in, bits)))
    _arg(sigma, "sigma", torch.float32, numel=d_in // 2)
    _arg(codebook, "codebook", torch.float32, numel=2 << bits)
    _arg(scale, "scale", torch.float32, numel=d_in, optional=True)
    return d_out


class DecodeJob(ctypes.Structure):
    """qamw_decode_job of include/qamw.h."""
    _fields_ = [("d_codes", ctypes.c_void_p), ("d_norm_f16", ctypes.c_void_p), ("d_sigma", ctypes.c_void_p),
                ("d_scale", ctypes.c_void_p), ("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("sign_seed", ctypes.c_uint64), ("d_out_w", ctypes.c_void_p), ("ld_out", ctypes.c_int64)]


class DecodeManyPlan:
    """A checked qamw_decode_many call, launched by calling it: the job table is built once, so
    repeated launches (a model's weights decoded again and again) cost no per-job Python work.
    jobs: sequence of dicts with codes, norm, sigma, d_in and optionally scale, sign_seed and out
    (allocated when absent).  The tensors are held until the plan is dropped."""

    def __init__(self, jobs, codebook: torch.Tensor, bits: int, block: int = 0, out_dtype=torch.bfloat16):
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be bfloat16 or float32")
        self.outs, self._keep = [], [codebook]
        self._arr = (DecodeJob * max(1, len(jobs)))()
        for k, j in enumerate(jobs):
            codes, norm, sigma, d_in = j["codes"], j["norm"], j["sigma"], j["d_in"]
            scale = j.get("scale")
            d_out = _decode_inputs(codes, norm, sigma, codebook, bits, d_in, scale)
            out = j.get("out")
            if out is None:
                out = torch.empty((d_out, d_in), dtype=out_dtype, device=codes.device)
            if out.dtype != out_dtype:
                raise ValueError("job %d: out must be %s" % (k, out_dtype))
            ld_out = _matrix(out, "out", rows=d_out, cols=d_in)
            _on_device(codes=codes, norm=norm, sigma=sigma, codebook=codebook, scale=scale, out=out)
            self._arr[k] = DecodeJob(_ptr(codes), _ptr(norm), _ptr(sigma), _ptr(scale), d_out, d_in,
                                     j.get("sign_seed", DEFAULT_SIGN_SEED), _ptr(out), ld_out)
            self._keep += [codes, norm, sigma, scale]
            self.outs.append(out)
        self._n, self._cb, self._bits, self._block = len(jobs), _ptr(codebook), bits, block
        self._dt = BF16 if out_dtype == torch.bfloat16 else F32
        self._lib = load()

    def __call__(self, stream=None) -> list:
        rc = self._lib.qamw_decode_many(ctypes.addressof(self._arr), self._n, self._cb, self._bits, self._block,
                                        self._dt, _stream(stream))
        _check(rc, "qamw_decode_many")
        return self.outs


def decode_many(jobs, codebook: torch.Tensor, bits: int, block: int = 0, out_dtype=torch.bfloat16) -> list:
    """Decode several matrices coded with one codebook (qamw_decode_many); returns the outputs in
    job order.  See DecodeManyPlan for the job fields."""
    return DecodeManyPlan(jobs, codebook, bits, block, out_dtype)()


def qgemm_workspace(M: int, d_out: int, d_in: int) -> int:
    return load().qamw_qgemm_workspace(M, d_out, d_in)


class QgemmPlan:
    """A checked qamw_qgemm call with its inputs, output and workspace fixed, launched by calling it:
    the argument checks run once, so a loop over the same buffers (a serving step) costs only the
    library call per launch.  Arguments as qgemm; the tensors are held until the plan is dropped."""

    def __init__(self, x: torch.Tensor, codes: torch.Tensor, norm: torch.Tensor, sigma: torch.Tensor,
                 codebook: torch.Tensor, bits: int, scale: Optional[torch.Tensor] = None,
                 sign_seed: int = DEFAULT_SIGN_SEED, block: int = 0, out_dtype=torch.float32,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
        if isinstance(x, torch.Tensor) and x.dim() == 1:
            x = x.unsqueeze(0)
        ld_x = _matrix(x, "x")
        M, d_in = x.shape
        d_out = _decode_inputs(codes, norm, sigma, codebook, bits, d_in, scale)
        if out is None:
            out = torch.empty((M, d_out), dtype=out_dtype, device=x.device)
        ld_y = _matrix(out, "out", rows=M, cols=d_out)
        need = qgemm_workspace(M, d_out, d_in)
        _arg(workspace, "workspace", torch.uint8, numel=need, optional=True)
        _on_device(x=x, codes=codes, norm=norm, sigma=sigma, codebook=codebook, scale=scale, out=out,
                   workspace=workspace)
        ws = workspace if workspace is not None else _ws(need, x.device)
        self.out = out
        self._keep = (x, codes, norm, sigma, codebook, scale, ws)
        self._fn = load().qamw_qgemm
        self._args = (_ptr(x), _dt(x), M, ld_x, _ptr(codes), _ptr(norm), _ptr(sigma), _ptr(codebook), bits,
                      _ptr(scale), d_out, d_in, block, sign_seed, _ptr(out), _dt(out), ld_y, _ptr(ws), ws.numel())

    def __call__(self, stream=None) -> torch.Tensor:
        rc = self._fn(*self._args, _stream(stream))
        _check(rc, "qamw_qgemm")
        return self.out


def qgemm(x: torch.Tensor, codes: torch.Tensor, norm: torch.Tensor, sigma: torch.Tensor, codebook: torch.Tensor,
          bits: int, scale: Optional[torch.Tensor] = None, sign_seed: int = DEFAULT_SIGN_SEED, block: int = 0,
          out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W^T (section 1) with W the decoder's weights, W never formed.  x: M x d_in (bf16/fp32)."""
    return QgemmPlan(x, codes, norm, sigma, codebook, bits, scale, sign_seed, block, out_dtype, out, workspace)()


def qgemm_noalloc(x: torch.Tensor, codes: torch.Tensor, norm: torch.Tensor, sigma: torch.Tensor,
                  codebook: torch.Tensor, bits: int, scale: Optional[torch.Tensor] = None,
                  sign_seed: int = DEFAULT_SIGN_SEED, block: int = 0, out: Optional[torch.Tensor] = None,
                  out_dtype=torch.float32) -> torch.Tensor:
    """qgemm with the library's static workspace (qamw_qgemm_noalloc): no workspace argument, and
    no allocation when `out` is given."""
    if isinstance(x, torch.Tensor) and x.dim() == 1:
        x = x.unsqueeze(0)
    ld_x = _matrix(x, "x")
    M, d_in = x.shape
    d_out = _decode_inputs(codes, norm, sigma, codebook, bits, d_in, scale)
    if out is None:
        out = torch.empty((M, d_out), dtype=out_dtype, device=x.device)
    ld_y = _matrix(out, "out", rows=M, cols=d_out)
    _on_device(x=x, codes=codes, norm=norm, sigma=sigma, codebook=codebook, scale=scale, out=out)
    rc = load().qamw_qgemm_noalloc(_ptr(x), _dt(x), M, ld_x, _ptr(codes), _ptr(norm), _ptr(sigma), _ptr(codebook),
                                   bits, _ptr(scale), d_out, d_in, block, sign_seed, _ptr(out), _dt(out), ld_y,
                                   _stream())
    _check(rc, "qamw_qgemm_noalloc")
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
    ld = _matrix(x, "x")
    T, d_in = x.shape
    s = torch.empty((d_in,), dtype=torch.float32, device=x.device)
    r = torch.empty((d_in,), dtype=torch.float64, device=x.device) if want_rms else None
    need = load().qamw_act_scale_workspace(T, d_in)
    _arg(workspace, "workspace", torch.uint8, numel=need, optional=True)
    _on_device(x=x, workspace=workspace)
    ws = workspace if workspace is not None else _ws(need, x.device)
    rc = load().qamw_act_scale(_ptr(x), _dt(x), T, d_in, ld, float(alpha), _ptr(s), _ptr(r), _ptr(ws), ws.numel(),
                               _stream())
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
    _arg(points, "points", torch.float32)
    if points.numel() % 2:
        raise ValueError("points must hold (x, y) pairs")
    _arg(thresholds, "thresholds", torch.float64, numel=(1 << ba) - 1)
    _arg(status, "status", torch.int32, numel=1, optional=True)
    _on_device(points=points, thresholds=thresholds, status=status)
    n = points.numel() // 2
    out = torch.empty((n,), dtype=torch.int32, device=points.device)
    rc = load().qamw_polar_index(_ptr(points), n, ba, bp, _ptr(thresholds), _ptr(out), _ptr(status), _stream())
    _check(rc, "qamw_polar_index")
    return out


def encode_polar(w: torch.Tensor, ba: int, bp: int, thresholds: torch.Tensor,
                 scale: Optional[torch.Tensor] = None, sign_seed: int = DEFAULT_SIGN_SEED, block: int = 0,
                 sigma: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None
                 ) -> Dict[str, torch.Tensor]:
    """Polar-baseline encode (section 3.5); decode with `decode(..., table, ba + bp, ...)`."""
    _arg(thresholds, "thresholds", torch.float64, numel=(1 << ba) - 1)
    bits = ba + bp
    d_out, d_in, ld, codes, norm, sig_out, ws = _encode_buffers(w, bits, scale, sigma, status, workspace, out)
    _on_device(thresholds=thresholds)
    rc = load().qamw_encode_polar(_ptr(w), _dt(w), d_out, d_in, ld, _ptr(scale), block, sign_seed, ba, bp,
                                  _ptr(thresholds), _ptr(sigma), _ptr(sig_out), _ptr(norm), _ptr(codes),
                                  _ptr(status), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check(rc, "qamw_encode_polar")
    return {"codes": codes, "norm": norm, "sigma": sigma if sigma is not None else sig_out}


def decode(codes: torch.Tensor, norm: torch.Tensor, sigma: torch.Tensor, codebook: torch.Tensor, bits: int,
           d_in: int, scale: Optional[torch.Tensor] = None, sign_seed: int = DEFAULT_SIGN_SEED,
           block: int = 0, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode to a d_out x d_in bf16 (default) or fp32 tensor."""
    d_out = _decode_inputs(codes, norm, sigma, codebook, bits, d_in, scale)
    if out is None:
        out = torch.empty((d_out, d_in), dtype=out_dtype, device=codes.device)
    ld_out = _matrix(out, "out", rows=d_out, cols=d_in)
    _on_device(codes=codes, norm=norm, sigma=sigma, codebook=codebook, scale=scale, out=out)
    rc = load().qamw_decode(_ptr(codes), _ptr(norm), _ptr(sigma), _ptr(codebook), bits, _ptr(scale), d_out, d_in,
                            block, sign_seed, _ptr(out), _dt(out), ld_out, _stream())
    _check(rc, "qamw_decode")
    return out
