"""Seeded synthetic inputs shared by the GPU library's tests and the CPU oracle.

The generator itself is C (``synth.c``, built into ``libsynth.so`` next to this
file); this wrapper only marshals numpy arrays.  It contains no arithmetic of
the quantizer.  See ``synth.c`` for the exact definition of every stream.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")
_SO_DEV = os.path.join(_HERE, "libsynth_gpu.so")
_SRC_DEV = os.path.join(_HERE, "synth_gpu.hip")

NORMAL, ACT_NORMAL, ACT_T4, GRAD_LOGNORMAL, INT, ACT_T4_DRIFT = 0, 1, 2, 3, 4, 5
_DT = {"f64": (0, np.float64), "f32": (1, np.float32), "bf16": (2, np.uint16)}

_lib = None


def build(force: bool = False, device: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP) and, with `device`, its device
    copy libsynth_gpu.so with hipcc for gfx950; returns the host library path."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    if device and (force or not os.path.exists(_SO_DEV)
                   or os.path.getmtime(_SO_DEV) < os.path.getmtime(_SRC_DEV)):
        tmp = _SO_DEV + ".tmp%d" % os.getpid()
        hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
        r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
                            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", _SRC_DEV, "-o", tmp],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("building %s failed:\n%s" % (_SRC_DEV, r.stderr))
        os.replace(tmp, _SO_DEV)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        i64, u64, vp, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        lib.synth_matrix.argtypes = [ctypes.c_int, u64, i64, i64, i64, i64, i64, i64, dbl, vp, i64,
                                     dbl, ctypes.c_int, vp, i64]
        lib.synth_matrix.restype = ctypes.c_int
        lib.synth_outlier_channels.argtypes = [u64, i64, i64, vp]
        lib.synth_outlier_channels.restype = ctypes.c_int
        lib.synth_signs.argtypes = [u64, i64, vp]
        lib.synth_signs.restype = ctypes.c_int
        lib.synth_mix64.argtypes = [u64]
        lib.synth_mix64.restype = u64
        lib.synth_col_factors.argtypes = [ctypes.c_int, u64, i64, i64, dbl, vp, i64, dbl, vp]
        lib.synth_col_factors.restype = ctypes.c_int
        _lib = lib
    return _lib


_lib_dev = None


def _load_dev():
    global _lib_dev
    if _lib_dev is None:
        if not os.path.exists(_SO_DEV):
            raise OSError("libsynth_gpu.so not built: run synth.build()")
        lib = ctypes.CDLL(_SO_DEV)
        i64, u64, vp, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        lib.synth_matrix_dev.argtypes = [ctypes.c_int, u64, i64, i64, dbl, vp, ctypes.c_int, vp, i64, vp]
        lib.synth_matrix_dev.restype = ctypes.c_int
        _lib_dev = lib
    return _lib_dev


def mix64(z: int) -> int:
    return int(_load().synth_mix64(z & 0xFFFFFFFFFFFFFFFF))


def outlier_channels(seed: int, n: int, k: int) -> np.ndarray:
    out = np.zeros(max(k, 1), dtype=np.int64)
    rc = _load().synth_outlier_channels(seed, n, k, out.ctypes.data)
    if rc:
        raise ValueError("synth_outlier_channels failed (%d)" % rc)
    return out[:k].copy()


def signs(seed: int, n: int) -> np.ndarray:
    """+-1.0 float32 vector (stream 5 of `seed`)."""
    out = np.zeros(max(n, 1), dtype=np.float32)
    rc = _load().synth_signs(seed, n, out.ctypes.data)
    if rc:
        raise ValueError("synth_signs failed (%d)" % rc)
    return out[:n].copy()


def matrix(kind: int, seed: int, rows: int, cols: int, *, r0: int = 0, nr: int | None = None,
           c0: int = 0, nc: int | None = None, p1: float = 1.0, outliers=None,
           out_factor: float = 1.0, dtype: str = "f64", out: np.ndarray | None = None) -> np.ndarray:
    """Block [r0:r0+nr, c0:c0+nc] of the logical rows x cols matrix of `kind`.

    dtype "bf16" returns the raw bf16 bit patterns as uint16.
    """
    nr = rows - r0 if nr is None else nr
    nc = cols - c0 if nc is None else nc
    code, npdt = _DT[dtype]
    if out is None:
        out = np.empty((nr, nc), dtype=npdt)
    assert out.dtype == npdt and out.shape == (nr, nc) and out.flags["C_CONTIGUOUS"]
    if outliers is None or len(outliers) == 0:
        optr, nout = None, 0
    else:
        outliers = np.ascontiguousarray(outliers, dtype=np.int64)
        optr, nout = outliers.ctypes.data, len(outliers)
    rc = _load().synth_matrix(kind, seed, rows, cols, r0, nr, c0, nc, float(p1), optr, nout,
                              float(out_factor), code, out.ctypes.data if out.size else None,
                              max(nc, 1))
    if rc:
        raise ValueError("synth_matrix failed (%d)" % rc)
    return out


def col_factors(kind: int, seed: int, cols: int, *, p1: float = 1.0, outliers=None,
                out_factor: float = 1.0) -> np.ndarray:
    """The per-column factors `matrix` applies (float64[cols])."""
    colf = np.empty(max(cols, 1), dtype=np.float64)
    if outliers is None or len(outliers) == 0:
        optr, nout = None, 0
    else:
        outliers = np.ascontiguousarray(outliers, dtype=np.int64)
        optr, nout = outliers.ctypes.data, len(outliers)
    rc = _load().synth_col_factors(kind, seed, 0, cols, float(p1), optr, nout, float(out_factor),
                                   colf.ctypes.data)
    if rc:
        raise ValueError("synth_col_factors failed (%d)" % rc)
    return colf[:cols]


def matrix_dev(kind: int, seed: int, rows: int, cols: int, *, p1: float = 1.0, outliers=None,
               out_factor: float = 1.0, dtype: str = "bf16", device="cuda:0", stream=None):
    """The whole rows x cols matrix of `kind` generated in device memory by the
    device copy of the generator; returns a torch tensor (bf16 for "bf16")."""
    import torch
    colf = torch.from_numpy(col_factors(kind, seed, cols, p1=p1, outliers=outliers,
                                        out_factor=out_factor)).to(device)
    tdt = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    out = torch.empty((rows, cols), dtype=tdt, device=device)
    st = torch.cuda.current_stream(device) if stream is None else stream
    rc = _load_dev().synth_matrix_dev(kind, seed, rows, cols, float(p1), colf.data_ptr(), _DT[dtype][0],
                                      out.data_ptr(), cols, st.cuda_stream)
    if rc:
        raise ValueError("synth_matrix_dev failed (%d)" % rc)
    torch.cuda.current_stream(device).synchronize()
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bit patterns (uint16) to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)
