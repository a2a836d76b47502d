"""Python access to the CPU oracle (``qamw_oracle.c``) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this module.  The GPU library and its binding never do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qamw_oracle.c")
_HDR = os.path.join(_HERE, "qamw_oracle.h")
_LIB = os.path.join(_HERE, "libqamw_oracle.so")

FLAG_NONFINITE, FLAG_BAD_SCALE, FLAG_NORM_RANGE, FLAG_POINT_RANGE = 1, 2, 4, 8

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def compile_to(src: str, out: str, extra=()) -> None:
    """Compile an oracle source file (the given one or a variant) into a shared library."""
    cmd = ["gcc"] + GCC_FLAGS + ["-I", _HERE] + list(extra) + [src, "-o", out, "-lm"]
    subprocess.check_call(cmd)


def build(force: bool = False) -> str:
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp%d" % os.getpid()
        compile_to(_SRC, tmp)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    vp, i32, i64, dbl, f32, u16 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_float, ctypes.c_uint16)
    sig = {
        "oracle_f16_from_f32": ([f32], u16),
        "oracle_f32_from_f16": ([u16], f32),
        "oracle_bf16_from_f32": ([f32], u16),
        "oracle_splitmix64": ([ctypes.c_uint64, i64, vp], None),
        "oracle_sign_mask": ([ctypes.c_uint64, i32, vp], None),
        "oracle_hadamard": ([i32, vp], None),
        "oracle_default_block": ([i32], i32),
        "oracle_bpw": ([i32, i32], dbl),
        "oracle_row_stride": ([i32, i32], ctypes.c_size_t),
        "oracle_front_end": ([vp, i32, i64, i32, i64, vp, vp, i32, vp, vp, vp], ctypes.c_int),
        "oracle_calibrate": ([vp, i32, i64, i32, i64, vp, vp, i32, vp, vp], ctypes.c_int),
        "oracle_nearest": ([f32, f32, vp, i32, vp], i32),
        "oracle_nearest_many": ([vp, i64, vp, i32, vp, vp], None),
        "oracle_pack_row": ([vp, i32, i32, vp, ctypes.c_size_t], None),
        "oracle_unpack_row": ([vp, i32, i32, vp], None),
        "oracle_encode": ([vp, i32, i64, i32, i64, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp],
                          ctypes.c_int),
        "oracle_decode": ([vp, vp, i64, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp], ctypes.c_int),
        "oracle_lloyd": ([vp, i64, i32, i32, vp, vp, vp, vp], ctypes.c_int),
        "oracle_qgemm": ([vp, i32, i64, vp, vp, i64, i32, vp, vp, i32, vp, vp, i32, vp], ctypes.c_int),
        "oracle_rayleigh_lloyd_max": ([i32, vp, vp], ctypes.c_int),
        "oracle_gauss_lloyd_max": ([i32, vp, vp], ctypes.c_int),
        "oracle_act_scale": ([vp, i64, i32, i64, dbl, vp, vp], ctypes.c_int),
        "oracle_scalar_index": ([f32, i32, vp], i32),
        "oracle_scalar_table": ([i32, vp, vp], None),
        "oracle_encode_scalar": ([vp, i32, i64, i32, i64, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp],
                                 ctypes.c_int),
        "oracle_polar_index": ([f32, f32, i32, i32, vp], i32),
        "oracle_polar_table": ([i32, i32, vp, vp], None),
        "oracle_encode_polar": ([vp, i32, i64, i32, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp],
                                ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


class Oracle:
    """numpy front-end to one compiled oracle library (the default build or a variant)."""

    def __init__(self, path: Optional[str] = None):
        if path is None:
            path = _LIB if os.path.exists(_LIB) else build()
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _p(a: Optional[np.ndarray]):
        return None if a is None else a.ctypes.data

    @staticmethod
    def _w(w: np.ndarray) -> Tuple[np.ndarray, int]:
        w = np.ascontiguousarray(w)
        if w.dtype == np.uint16:
            return w, 1
        if w.dtype == np.float32:
            return w, 0
        raise TypeError("weights must be float32 or uint16 (bf16 bits)")

    # -- scalars -------------------------------------------------------------
    def f16_from_f32(self, x: float) -> int:
        return self.lib.oracle_f16_from_f32(x)

    def f32_from_f16(self, h: int) -> float:
        return self.lib.oracle_f32_from_f16(h)

    def bf16_from_f32(self, x: float) -> int:
        return self.lib.oracle_bf16_from_f32(x)

    def default_block(self, d_in: int) -> int:
        return self.lib.oracle_default_block(d_in)

    def bpw(self, d_in: int, bits: int) -> float:
        return self.lib.oracle_bpw(d_in, bits)

    def row_stride(self, d_in: int, bits: int) -> int:
        return self.lib.oracle_row_stride(d_in, bits)

    # -- arrays --------------------------------------------------------------
    def splitmix64(self, seed: int, n: int) -> np.ndarray:
        """The first n outputs of splitmix64 started at `seed` (uint64)."""
        out = np.empty((max(n, 1),), dtype=np.uint64)
        self.lib.oracle_splitmix64(seed, n, self._p(out))
        return out[:n]

    def sign_mask(self, seed: int, d_in: int) -> np.ndarray:
        """Sign-mask bits of a seed (section 3.3): bit j % 32 of word j / 32 set when eps_j = -1."""
        out = np.zeros((max((d_in + 31) // 32, 1),), dtype=np.uint32)
        self.lib.oracle_sign_mask(seed, d_in, self._p(out))
        return out[: (d_in + 31) // 32]

    @staticmethod
    def signs(bits: np.ndarray, d_in: int) -> np.ndarray:
        """+1 / -1 (float64) of mask bits."""
        j = np.arange(d_in)
        return np.where((bits[j >> 5] >> (j & 31).astype(np.uint32)) & 1, -1.0, 1.0)

    def hadamard(self, b: int) -> np.ndarray:
        H = np.empty((b, b), dtype=np.float64)
        self.lib.oracle_hadamard(b, self._p(H))
        return H

    def front_end(self, w, s, sign_bits, block):
        w, bf = self._w(w)
        n, d_in = w.shape
        y = np.empty((n, d_in), dtype=np.float64)
        r = np.empty((n,), dtype=np.float64)
        st = np.zeros((1,), dtype=np.int32)
        rc = self.lib.oracle_front_end(self._p(w), bf, n, d_in, d_in, self._p(s), self._p(sign_bits),
                                       block, self._p(y), self._p(r), self._p(st))
        assert rc == 0
        return y, r, int(st[0])

    def calibrate(self, w, s, sign_bits, block):
        w, bf = self._w(w)
        n, d_in = w.shape
        sigma = np.empty((d_in // 2,), dtype=np.float32)
        st = np.zeros((1,), dtype=np.int32)
        rc = self.lib.oracle_calibrate(self._p(w), bf, n, d_in, d_in, self._p(s), self._p(sign_bits),
                                       block, self._p(sigma), self._p(st))
        assert rc == 0
        return sigma, int(st[0])

    def nearest(self, p: np.ndarray, cb: np.ndarray):
        p = np.ascontiguousarray(p, dtype=np.float32).reshape(-1, 2)
        cb = np.ascontiguousarray(cb, dtype=np.float32).reshape(-1, 2)
        idx = np.empty((p.shape[0],), dtype=np.int32)
        d = np.empty((p.shape[0],), dtype=np.float32)
        self.lib.oracle_nearest_many(self._p(p), p.shape[0], self._p(cb), cb.shape[0], self._p(idx), self._p(d))
        return idx, d

    def pack_row(self, idx: np.ndarray, bits: int, d_in: int) -> np.ndarray:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        stride = self.row_stride(d_in, bits)
        out = np.empty((stride,), dtype=np.uint8)
        self.lib.oracle_pack_row(self._p(idx), d_in // 2, bits, self._p(out), stride)
        return out

    def unpack_row(self, row: np.ndarray, bits: int, d_in: int) -> np.ndarray:
        row = np.ascontiguousarray(row, dtype=np.uint8)
        idx = np.empty((d_in // 2,), dtype=np.int32)
        self.lib.oracle_unpack_row(self._p(row), d_in // 2, bits, self._p(idx))
        return idx

    def encode(self, w, s, sign_bits, block, cb, bits, sigma, want_idx=True, want_p=False):
        w, bf = self._w(w)
        n, d_in = w.shape
        stride = self.row_stride(d_in, bits)
        norm = np.empty((n,), dtype=np.uint16)
        codes = np.empty((n, stride), dtype=np.uint8)
        idx = np.empty((n, d_in // 2), dtype=np.int32) if want_idx else None
        p = np.empty((n, d_in), dtype=np.float32) if want_p else None
        st = np.zeros((1,), dtype=np.int32)
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        sigma = np.ascontiguousarray(sigma, dtype=np.float32)
        rc = self.lib.oracle_encode(self._p(w), bf, n, d_in, d_in, self._p(s), self._p(sign_bits), block,
                                    self._p(cb), bits, self._p(sigma), self._p(norm), self._p(codes),
                                    self._p(idx), self._p(p), self._p(st))
        assert rc == 0
        return {"norm": norm, "codes": codes, "idx": idx, "p": p, "status": int(st[0])}

    def decode(self, codes, norm, d_in, sigma, cb, bits, s, sign_bits, block, want_f64=False):
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        norm = np.ascontiguousarray(norm, dtype=np.uint16)
        n = norm.shape[0]
        f32 = np.empty((n, d_in), dtype=np.float32)
        b16 = np.empty((n, d_in), dtype=np.uint16)
        f64 = np.empty((n, d_in), dtype=np.float64) if want_f64 else None
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        rc = self.lib.oracle_decode(self._p(codes), self._p(norm), n, d_in, self._p(sigma), self._p(cb), bits,
                                    self._p(s), self._p(sign_bits), block, self._p(f32), self._p(b16),
                                    self._p(f64))
        assert rc == 0
        return {"f32": f32, "bf16": b16, "f64": f64}

    def qgemm(self, x, codes, norm, d_in, sigma, cb, bits, s, sign_bits, block):
        """y = x W^T (M x d_out, fp64) with W the decoder's output before rounding (section 1)."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        norm = np.ascontiguousarray(norm, dtype=np.uint16)
        n = norm.shape[0]
        y = np.empty((x.shape[0], n), dtype=np.float64)
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        rc = self.lib.oracle_qgemm(self._p(x), x.shape[0], x.shape[1], self._p(codes), self._p(norm), n, d_in,
                                   self._p(sigma), self._p(cb), bits, self._p(s), self._p(sign_bits), block,
                                   self._p(y))
        assert rc == 0
        return y

    def lloyd(self, pts, bits, iters, init=None):
        pts = np.ascontiguousarray(pts, dtype=np.float32).reshape(-1, 2)
        K = 1 << bits
        cb = np.empty((K, 2), dtype=np.float32)
        e = np.empty((max(iters, 1),), dtype=np.int64)
        st = np.zeros((1,), dtype=np.int32)
        init_a = None if init is None else np.ascontiguousarray(init, dtype=np.float32)
        rc = self.lib.oracle_lloyd(self._p(pts), pts.shape[0], bits, iters, self._p(init_a), self._p(cb),
                                   self._p(e), self._p(st))
        assert rc == 0
        return cb, e[:iters], int(st[0])


    # -- polar baseline (section 3.5) -----------------------------------------
    def rayleigh_lloyd_max(self, ba):
        na = 1 << ba
        levels = np.empty((na,), dtype=np.float64)
        thr = np.zeros((max(na - 1, 1),), dtype=np.float64)
        rc = self.lib.oracle_rayleigh_lloyd_max(ba, self._p(levels), self._p(thr))
        assert rc == 0
        return levels, thr[: na - 1]

    def polar_index(self, p, ba, bp, thresholds):
        p = np.ascontiguousarray(p, dtype=np.float32).reshape(-1, 2)
        thr = np.ascontiguousarray(thresholds, dtype=np.float64)
        if thr.size == 0:
            thr = np.zeros((1,), dtype=np.float64)
        return np.array([self.lib.oracle_polar_index(float(x), float(y), ba, bp, self._p(thr)) for x, y in p],
                        dtype=np.int32)

    def polar_table(self, ba, bp, levels):
        cb = np.empty((1 << (ba + bp), 2), dtype=np.float32)
        levels = np.ascontiguousarray(levels, dtype=np.float64)
        self.lib.oracle_polar_table(ba, bp, self._p(levels), self._p(cb))
        return cb

    def encode_polar(self, w, s, sign_bits, block, ba, bp, thresholds, sigma, want_idx=True, want_p=False):
        w, bf = self._w(w)
        n, d_in = w.shape
        bits = ba + bp
        stride = self.row_stride(d_in, bits)
        norm = np.empty((n,), dtype=np.uint16)
        codes = np.empty((n, stride), dtype=np.uint8)
        idx = np.empty((n, d_in // 2), dtype=np.int32) if want_idx else None
        p = np.empty((n, d_in), dtype=np.float32) if want_p else None
        st = np.zeros((1,), dtype=np.int32)
        thr = np.ascontiguousarray(thresholds, dtype=np.float64)
        if thr.size == 0:
            thr = np.zeros((1,), dtype=np.float64)
        sigma = np.ascontiguousarray(sigma, dtype=np.float32)
        rc = self.lib.oracle_encode_polar(self._p(w), bf, n, d_in, d_in, self._p(s), self._p(sign_bits), block, ba,
                                          bp, self._p(thr), self._p(sigma), self._p(norm), self._p(codes),
                                          self._p(idx), self._p(p), self._p(st))
        assert rc == 0
        return {"norm": norm, "codes": codes, "idx": idx, "p": p, "status": int(st[0])}

    def act_scale(self, x, alpha):
        """Activation-aware channel scale (reading R11): (s fp32[d_in], r fp64[d_in])."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        T, d_in = x.shape
        s = np.empty((d_in,), dtype=np.float32)
        r = np.empty((d_in,), dtype=np.float64)
        rc = self.lib.oracle_act_scale(self._p(x), T, d_in, d_in, float(alpha), self._p(s), self._p(r))
        assert rc == 0
        return s, r

    # ---- the scalar (d = 1) ablation, reading R10
    def gauss_lloyd_max(self, b):
        L = 1 << b
        levels = np.empty((L,), dtype=np.float64)
        thr = np.zeros((L - 1,), dtype=np.float64)
        rc = self.lib.oracle_gauss_lloyd_max(b, self._p(levels), self._p(thr))
        assert rc == 0
        return levels, thr

    def scalar_index(self, p, b, thresholds):
        thr = np.ascontiguousarray(thresholds, dtype=np.float64)
        return np.array([self.lib.oracle_scalar_index(float(v), b, self._p(thr)) for v in np.ravel(p)],
                        dtype=np.int32)

    def scalar_table(self, b, levels):
        cb = np.empty((1 << (2 * b), 2), dtype=np.float32)
        self.lib.oracle_scalar_table(b, self._p(np.ascontiguousarray(levels, dtype=np.float64)), self._p(cb))
        return cb

    def encode_scalar(self, w, s, sign_bits, block, b, thresholds, sigma, want_idx=True, want_p=False):
        w, bf = self._w(w)
        n, d_in = w.shape
        stride = self.row_stride(d_in, 2 * b)
        norm = np.empty((n,), dtype=np.uint16)
        codes = np.empty((n, stride), dtype=np.uint8)
        idx = np.empty((n, d_in // 2), dtype=np.int32) if want_idx else None
        p = np.empty((n, d_in), dtype=np.float32) if want_p else None
        st = np.zeros((1,), dtype=np.int32)
        thr = np.ascontiguousarray(thresholds, dtype=np.float64)
        sigma = np.ascontiguousarray(sigma, dtype=np.float32)
        rc = self.lib.oracle_encode_scalar(self._p(w), bf, n, d_in, d_in, self._p(s), self._p(sign_bits), block, b,
                                           self._p(thr), self._p(sigma), self._p(norm), self._p(codes), self._p(idx),
                                           self._p(p), self._p(st))
        assert rc == 0
        return {"norm": norm, "codes": codes, "idx": idx, "p": p, "status": int(st[0])}


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
