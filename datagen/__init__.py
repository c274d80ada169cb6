"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check.  Holds no codec arithmetic: it only draws numbers (``librcgen.so``)
and narrows them to the storage dtype with library casts (torch for bfloat16,
numpy for float16, both round-to-nearest-even).

Workloads (names say what they are):

* ``fp16_normal_64x2048``      -- 64 x 2048 fp16 ~ N(0,1), seeds 0 and 1
* ``bf16_act_256x8192_outl``   -- 256 x 8192 bf16 ~ N(0,1), each element x20
                                  with probability 0.001 (separate draw), seed 2
* ``fp32_normal_4m_x8``        -- 8 streams of 4,194,304 fp32 ~ N(0, sd 0.5),
                                  seeds 300+k
* ``bf16_weight_4096x4096``    -- 0.02 * N(0,1) * d_row, d_row ~ U[0.5, 2]
                                  per row; z seed 41, drift seed 40
* ``bf16_student4``            -- Student-t (nu = 4) bf16 messages of any size,
                                  seeds 500+k
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librcgen.so")

NORMAL, STUDENT4, NORMAL_OUTLIER, ROWDRIFT, UNIFORM = 0, 1, 2, 3, 4

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            subprocess.run(["make", "-C", _HERE], check=True, capture_output=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.rcg_fill.restype = ctypes.c_int
        lib.rcg_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64,
                                 ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int]
        lib.rcg_draw64.restype = ctypes.c_uint64
        lib.rcg_draw64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint]
        lib.rcg_mix64.restype = ctypes.c_uint64
        lib.rcg_mix64.argtypes = [ctypes.c_uint64]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def fill(kind: int, seed: int, n: int, p0=0.0, p1=1.0, p2=0.0, seed2: int = 0, cols: int = 1,
         start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().rcg_fill(kind, seed, seed2, p0, p1, p2, cols, start, n, out.ctypes.data, _threads())
    return out


def normal(seed: int, n: int, mean: float = 0.0, std: float = 1.0, start: int = 0) -> np.ndarray:
    return fill(NORMAL, seed, n, mean, std, start=start)


def student_t4(seed: int, n: int, scale: float = 1.0, start: int = 0) -> np.ndarray:
    return fill(STUDENT4, seed, n, 0.0, scale, start=start)


def normal_outliers(seed: int, n: int, factor: float = 20.0, prob: float = 0.001,
                    std: float = 1.0, start: int = 0) -> np.ndarray:
    return fill(NORMAL_OUTLIER, seed, n, factor, std, prob, start=start)


def rowdrift(seed_z: int, seed_d: int, rows: int, cols: int, std: float = 0.02,
             lo: float = 0.5, hi: float = 2.0) -> np.ndarray:
    return fill(ROWDRIFT, seed_z, rows * cols, lo, std, hi, seed2=seed_d, cols=cols)


def uniform(seed: int, n: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    return fill(UNIFORM, seed, n, lo, hi)


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage dtype by a library cast (RNE).  bf16 comes back as
    uint16 bit patterns, fp16 as numpy float16, fp32 unchanged."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)
    raise ValueError(dtype)


# ---- the five workloads --------------------------------------------------

def fp16_normal_64x2048(stream: int = 0) -> np.ndarray:
    """INT4 round trip: 64 tiles of 2048 fp16 ~ N(0,1); stream 0 seed 0, stream 1 seed 1."""
    return narrow(normal(stream, 64 * 2048), "fp16")


def bf16_act_256x8192_outl() -> np.ndarray:
    """INT3 activation message: 256 tokens x 8192 hidden bf16, N(0,1) with 0.1% outliers x20."""
    return narrow(normal_outliers(2, 256 * 8192, 20.0, 0.001), "bf16")


def fp32_normal_4m(stream: int) -> np.ndarray:
    """FP8 reduce: one of 8 fp32 streams of 4M elements ~ N(0, sd 0.5), seed 300+k."""
    return normal(300 + stream, 4 * 1024 * 1024, 0.0, 0.5)


def bf16_weight_4096x4096() -> np.ndarray:
    """MXFP4 direct cast: bf16 4096x4096, 0.02*N(0,1)*U[0.5,2] per-row drift."""
    return narrow(rowdrift(41, 40, 4096, 4096, 0.02, 0.5, 2.0), "bf16")


def bf16_student4(nbytes: int, stream: int = 0) -> np.ndarray:
    """Size sweep: a bf16 message of nbytes bytes, Student-t nu=4, seed 500+k."""
    return narrow(student_t4(500 + stream, nbytes // 2), "bf16")
