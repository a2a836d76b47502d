"""Seeded synthetic inputs for the QAM-W codec (test and benchmark data only).

The QAM-W pages measure on real LLM checkpoints (TinyLlama-1.1B ... 13B) that are
not available here; these generators stand in for them with matrices of the
same shapes and heavy-tailed, outlier-column statistics.  Everything is a pure
function of (seed, stream id, counter), produced by ``synth.c``.  This module
contains none of the codec's arithmetic (the rotation's sign mask is drawn from
its seed by the library and by the oracle, each on its own); the CPU oracle and
the GPU library both read the bytes it produces.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_SRC_GPU = os.path.join(_HERE, "synth_gpu.hip")
_LIB_GPU = os.path.join(_HERE, "libsynth_gpu.so")

CONFIG_SEED_BASE = 0x51414D5700000000
SID_POINTS = 4
SID_POINTS_K128 = 5

_lib = None


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so with gcc (IEEE semantics, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def build_gpu(force: bool = False) -> str:
    """Compile synth_gpu.hip (the device form of synth_weights) for gfx950 into libsynth_gpu.so."""
    if force or not os.path.exists(_LIB_GPU) or os.path.getmtime(_LIB_GPU) < os.path.getmtime(_SRC_GPU):
        tmp = _LIB_GPU + ".tmp%d" % os.getpid()
        cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3", "-std=c++17",
               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", "-fPIC", "-shared", _SRC_GPU, "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_GPU)
    return _LIB_GPU


_lib_gpu = None


def _load_gpu():
    global _lib_gpu
    if _lib_gpu is None:
        if not os.path.exists(_LIB_GPU):
            raise RuntimeError("libsynth_gpu.so is not built (%s); run __graft_entry__.build()" % _LIB_GPU)
        lib = ctypes.CDLL(_LIB_GPU)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p)
        lib.synth_weights_device.argtypes = [u64, u64, i64, i64, i32, i32, i32, dbl, vp, dbl, i32, vp, vp]
        lib.synth_weights_device.restype = ctypes.c_int
        _lib_gpu = lib
    return _lib_gpu


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_u64.argtypes = [u64, u64]
        lib.synth_u64.restype = u64
        lib.synth_uniform.argtypes = [u64, u64]
        lib.synth_uniform.restype = dbl
        lib.synth_gauss.argtypes = [u64, u64]
        lib.synth_gauss.restype = dbl
        lib.synth_weights.argtypes = [u64, u64, i64, i64, i32, i32, i32, dbl, vp, dbl, i32, vp]
        lib.synth_weights.restype = None
        lib.synth_outlier_columns.argtypes = [u64, u64, i32, i32, vp]
        lib.synth_outlier_columns.restype = None
        lib.synth_channel_scale.argtypes = [u64, u64, i32, vp]
        lib.synth_channel_scale.restype = None
        lib.synth_points.argtypes = [u64, u64, i64, vp]
        lib.synth_points.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ----------------------------------------------------------------------------- primitives

def gauss(seed: int, sid: int, q: np.ndarray) -> np.ndarray:
    lib = _load()
    key = lib.synth_key(seed, sid)
    return np.array([lib.synth_gauss(key, int(x)) for x in np.asarray(q).ravel()], dtype=np.float64)


def uniform(seed: int, sid: int, i: np.ndarray) -> np.ndarray:
    lib = _load()
    key = lib.synth_key(seed, sid)
    return np.array([lib.synth_uniform(key, int(x)) for x in np.asarray(i).ravel()], dtype=np.float64)


def points(seed: int, sid: int, n: int) -> np.ndarray:
    """n x 2 float32 samples of the unit circular Gaussian."""
    out = np.empty((n, 2), dtype=np.float32)
    _load().synth_points(seed, sid, n, _ptr(out))
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- matrix specs

@dataclass
class MatrixSpec:
    name: str
    d_out: int
    d_in: int
    bf16: bool
    dist: int            # 0 gaussian, 1 student-t
    nu: int
    scale: float
    outlier_frac: float  # fraction of input columns
    n_outlier: int
    outlier_factor: float
    seed: int
    sid_w: int

    @property
    def sid_outlier(self) -> int:
        return self.sid_w + 0x10000

    @property
    def sid_scale(self) -> int:
        return self.sid_w + 0x20000

    def outlier_columns(self) -> np.ndarray:
        if self.n_outlier == 0:
            return np.zeros((0,), dtype=np.int32)
        buf = np.empty((self.d_in,), dtype=np.int32)
        _load().synth_outlier_columns(self.seed, self.sid_outlier, self.d_in, self.n_outlier, _ptr(buf))
        return np.sort(buf[: self.n_outlier])

    def outlier_mask(self) -> np.ndarray:
        m = np.zeros((self.d_in,), dtype=np.uint8)
        m[self.outlier_columns()] = 1
        return m

    def weights(self, row0: int = 0, nrows: Optional[int] = None) -> np.ndarray:
        """Rows [row0, row0+nrows): float32, or uint16 bf16 bit patterns when bf16."""
        if nrows is None:
            nrows = self.d_out - row0
        mask = self.outlier_mask()
        out = np.empty((nrows, self.d_in), dtype=np.uint16 if self.bf16 else np.float32)
        _load().synth_weights(self.seed, self.sid_w, row0, nrows, self.d_in, self.dist, self.nu,
                              self.scale, _ptr(mask), self.outlier_factor, 1 if self.bf16 else 0,
                              _ptr(out))
        return out

    def weights_device(self, device, row0: int = 0, nrows: Optional[int] = None, out=None):
        """The same rows as weights(), drawn on the GPU (synth_gpu.hip) into a torch tensor:
        bfloat16 or float32, nrows x d_in, on `device`; generated on torch's current stream."""
        import torch
        if nrows is None:
            nrows = self.d_out - row0
        dt = torch.bfloat16 if self.bf16 else torch.float32
        if out is None:
            out = torch.empty((nrows, self.d_in), dtype=dt, device=device)
        if out.dtype != dt or tuple(out.shape) != (nrows, self.d_in) or not out.is_contiguous():
            raise ValueError("out must be a contiguous %d x %d %s tensor" % (nrows, self.d_in, dt))
        mask = None
        if self.n_outlier:
            mask = torch.from_numpy(self.outlier_mask()).to(out.device)
        rc = _load_gpu().synth_weights_device(self.seed, self.sid_w, row0, nrows, self.d_in, self.dist, self.nu,
                                              self.scale, None if mask is None else mask.data_ptr(),
                                              self.outlier_factor, 1 if self.bf16 else 0, out.data_ptr(),
                                              torch.cuda.current_stream(out.device).cuda_stream)
        if rc != 0:
            raise RuntimeError("synth_weights_device failed")
        if mask is not None:
            torch.cuda.current_stream(out.device).synchronize()   # the mask tensor is freed here
        return out

    def channel_scale(self) -> np.ndarray:
        out = np.empty((self.d_in,), dtype=np.float32)
        _load().synth_channel_scale(self.seed, self.sid_scale, self.d_in, _ptr(out))
        return out


def _spec(name, d_out, d_in, bf16, dist, nu, scale, frac, factor, seed, sid_w) -> MatrixSpec:
    n_out = int(round(frac * d_in)) if frac > 0 else 0
    return MatrixSpec(name, d_out, d_in, bf16, dist, nu, scale, frac, n_out, factor, seed, sid_w)


def sid_matrix(layer: int, m: int) -> int:
    return 0x100 + 16 * layer + m


LAYER13B_SHAPES = [("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
                   ("gate", 13824, 5120), ("up", 13824, 5120), ("down", 5120, 13824)]


@dataclass
class Config:
    index: int
    name: str
    block: int
    bits: List[int]
    matrices: List[MatrixSpec]
    n_points: int
    lloyd_iters: int
    points_sid: int = SID_POINTS
    fixed_sigma: Optional[float] = None
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return CONFIG_SEED_BASE + self.index


def _layer13b(seed: int, layer: int) -> List[MatrixSpec]:
    return [_spec("L%d.%s" % (layer, nm), do, di, True, 1, 4, 0.015, 0.0, 1.0, seed, sid_matrix(layer, m))
            for m, (nm, do, di) in enumerate(LAYER13B_SHAPES)]


def config(index: int, n_layers: int = 40) -> Config:
    """The five workloads (0-based): shapes, value distributions and codebook sizes."""
    seed = CONFIG_SEED_BASE + index
    if index == 0:
        ms = [_spec("W", 256, 512, False, 0, 0, 0.02, 4.0 / 512.0, 20.0, seed, sid_matrix(0, 0))]
        return Config(0, "small-256x512", 64, [8], ms, 1 << 16, 20, fixed_sigma=0.125)
    if index == 1:
        ms = [_spec("W", 4096, 4096, True, 1, 5, 0.015, 0.01, 10.0, seed, sid_matrix(0, 0))]
        return Config(1, "attn-4096x4096", 128, [11], ms, 1 << 20, 20)
    if index == 2:
        ms = [_spec("up", 11008, 4096, True, 0, 0, 0.02, 0.005, 15.0, seed, sid_matrix(0, 0)),
              _spec("down", 4096, 11008, True, 0, 0, 0.02, 0.005, 15.0, seed, sid_matrix(0, 1))]
        return Config(2, "mlp7b-11008x4096", 256, [11], ms, 1 << 22, 50)
    if index == 3:
        return Config(3, "layer13b", 128, [11, 7], _layer13b(seed, 0), 1 << 20, 20,
                      extra={"k128_points": 1 << 20, "k128_sid": SID_POINTS_K128})
    if index == 4:
        ms: List[MatrixSpec] = []
        for layer in range(n_layers):
            ms.extend(_layer13b(seed, layer))
        return Config(4, "stack13b-40L", 128, [11], ms, 1 << 20, 20)
    raise ValueError("config index must be 0..4")
