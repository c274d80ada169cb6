"""Python view of the plain CPU oracle (``librcodec_oracle.so``).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the product path
(``reduction_codec_amd``) never does, and the oracle shares no code with it.

Arrays are numpy; bf16 data travels as its uint16 bit patterns.  Every call
is synchronous and single-threaded (``*_parallel`` helpers split tile ranges
over threads only to bound wall time; results are identical).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RC_ORACLE_LIB names another build of rcodec_oracle.c (the mutation tests load
# deliberately broken copies this way); unset, the library built beside this file.
_LIB_PATH = os.environ.get("RC_ORACLE_LIB") or os.path.join(_HERE, "librcodec_oracle.so")

TILE = 2048
BLOCK = 32
MAX_STREAMS = 16

FMT_INT4, FMT_INT3, FMT_FP8_E4M3, FMT_MXFP4, FMT_FP8_E5M2 = 1, 2, 3, 4, 5
SCALE_FP16, SCALE_FP32, SCALE_E8M0 = 1, 2, 3
DT_FP32, DT_FP16, DT_BF16 = 1, 2, 3
OK, ERR_NULL, ERR_UNSUPPORTED, ERR_ALIGN, ERR_RANGE, ERR_HIP = 0, 1, 2, 3, 4, 5

INT4 = (FMT_INT4, SCALE_FP16, BLOCK)
INT3 = (FMT_INT3, SCALE_FP16, BLOCK)
FP8 = (FMT_FP8_E4M3, SCALE_FP32, BLOCK)
MXFP4 = (FMT_MXFP4, SCALE_E8M0, BLOCK)
CODECS = {"int4": INT4, "int3": INT3, "fp8": FP8, "mxfp4": MXFP4}

# Every supported codec, named "<element>_<scale>_b<block>": INT4/INT3 with
# FP16 or E8M0 scales, E4M3/E5M2 with FP32, FP16 or E8M0 scales, E2M1 with
# E8M0 scales, blocks of 16, 32 and 64.
_ELEMS = {"int4": FMT_INT4, "int3": FMT_INT3, "e4m3": FMT_FP8_E4M3, "e5m2": FMT_FP8_E5M2,
          "e2m1": FMT_MXFP4}
_SCALES = {"f16": SCALE_FP16, "f32": SCALE_FP32, "e8m0": SCALE_E8M0}
_SUPPORTED = {"int4": ("f16", "e8m0"), "int3": ("f16", "e8m0"), "e4m3": ("f32", "f16", "e8m0"),
              "e5m2": ("f32", "f16", "e8m0"), "e2m1": ("e8m0",)}
ALL_CODECS = {f"{el}_{sc}_b{b}": (_ELEMS[el], _SCALES[sc], b)
              for el, scs in _SUPPORTED.items() for sc in scs for b in (16, 32, 64)}


class Codec(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("scale", ctypes.c_int32), ("block", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) and not os.environ.get("RC_ORACLE_LIB"):
        subprocess.run(["make", "-C", _HERE], check=True, capture_output=True)
    lib = ctypes.CDLL(_LIB_PATH)
    C, vp, sz, i32 = Codec, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sig = {
        "rco_tile_bytes": (sz, [C]),
        "rco_packed_bytes": (sz, [C, sz]),
        "rco_quantize_pack": (i32, [C, i32, vp, sz, vp]),
        "rco_quantize_pack_tiles": (i32, [C, i32, vp, sz, vp, sz, sz]),
        "rco_unpack_dequant": (i32, [C, vp, sz, i32, vp]),
        "rco_dequant_reduce_requant": (i32, [C, ctypes.POINTER(vp), i32, sz, vp, vp]),
        "rco_dequant_reduce_requant_tiles": (i32, [C, ctypes.POINTER(vp), i32, sz, vp, vp, sz, sz]),
        "rco_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "rco_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "rco_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "rco_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "rco_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "rco_e2m1_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "rco_e8m0_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "rco_e4m3_mag_of_quotient": (i32, [ctypes.c_double, ctypes.c_double]),
        "rco_e2m1_mag_of": (i32, [ctypes.c_double]),
        "rco_int_mag": (i32, [ctypes.c_float, ctypes.c_float, i32]),
        "rco_int_scale_bits": (ctypes.c_uint16, [ctypes.c_float, i32]),
        "rco_fp8_scale": (ctypes.c_float, [ctypes.c_float]),
        "rco_mx_exponent": (i32, [ctypes.c_float]),
        "rco_e5m2_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "rco_e5m2_mag_of_quotient": (i32, [ctypes.c_double, ctypes.c_double]),
        "rco_elem_emax": (i32, [i32]),
        "rco_e8m0_exponent": (i32, [ctypes.c_float, i32]),
        "rco_fp8_scale_f32": (ctypes.c_float, [ctypes.c_float, i32]),
        "rco_fp8_scale_f16_bits": (ctypes.c_uint16, [ctypes.c_float, i32]),
    }
    for name in ("rco_map_f32_to_f16", "rco_map_f32_to_bf16", "rco_map_f16_to_f32",
                 "rco_map_bf16_to_f32", "rco_map_e4m3_mag", "rco_map_e2m1_mag",
                 "rco_map_fp8_scale", "rco_map_mx_exponent"):
        sig[name] = (None, [vp, vp, sz] if "e4m3" not in name else [vp, vp, vp, sz])
    sig["rco_map_int_mag"] = (None, [vp, vp, i32, vp, sz])
    sig["rco_map_int_scale_bits"] = (None, [vp, i32, vp, sz])
    sig["rco_map_e5m2_mag"] = (None, [vp, vp, vp, sz])
    sig["rco_map_e8m0_exponent"] = (None, [vp, i32, vp, sz])
    sig["rco_map_fp8_scale_f16_bits"] = (None, [vp, i32, vp, sz])
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def lib():
    return _load()


def _codec(c) -> Codec:
    return c if isinstance(c, Codec) else Codec(*c)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray, dtype: int | None) -> int:
    if dtype is not None:
        return dtype
    if a.dtype == np.float32:
        return DT_FP32
    if a.dtype == np.float16:
        return DT_FP16
    raise ValueError("pass dtype=DT_BF16 for uint16 bf16 bit patterns")


def tile_bytes(c) -> int:
    return _load().rco_tile_bytes(_codec(c))


def packed_bytes(c, n: int) -> int:
    return _load().rco_packed_bytes(_codec(c), n)


def _check(st: int):
    if st != OK:
        raise RuntimeError(f"oracle status {st}")


def quantize_pack(c, x: np.ndarray, dtype: int | None = None, tiles: tuple[int, int] | None = None,
                  out: np.ndarray | None = None) -> np.ndarray:
    """Pack x (float32 / float16 / uint16 bf16 bits) into tiles.  With
    ``tiles=(t0, t1)`` only those tiles of ``out`` are written."""
    x = np.ascontiguousarray(x)
    n = x.size
    if out is None:
        out = np.zeros(packed_bytes(c, n), dtype=np.uint8)
    dt = _dtype_code(x, dtype)
    if tiles is None:
        _check(_load().rco_quantize_pack(_codec(c), dt, _ptr(x), n, _ptr(out)))
    else:
        _check(_load().rco_quantize_pack_tiles(_codec(c), dt, _ptr(x), n, _ptr(out), tiles[0], tiles[1]))
    return out


def unpack_dequant(c, packed: np.ndarray, n: int, out_dtype: int = DT_FP32) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size < packed_bytes(c, n):
        raise ValueError("packed must hold packed_bytes(codec, n) bytes")
    out = np.empty(n, dtype=np.float32 if out_dtype == DT_FP32 else np.uint16)
    _check(_load().rco_unpack_dequant(_codec(c), _ptr(packed), n, out_dtype, _ptr(out)))
    if out_dtype == DT_FP16:
        return out.view(np.float16)
    return out


def dequant_reduce_requant(c, streams, n: int, want_sum: bool = False,
                           tiles: tuple[int, int] | None = None,
                           out: np.ndarray | None = None, sum_out: np.ndarray | None = None):
    """Reduce K packed streams; returns (packed, sums or None)."""
    streams = [np.ascontiguousarray(s, dtype=np.uint8) for s in streams]
    k = len(streams)
    if any(s.size < packed_bytes(c, n) for s in streams):
        raise ValueError("every stream must hold packed_bytes(codec, n) bytes")
    arr = (ctypes.c_void_p * max(k, 1))(*[s.ctypes.data for s in streams])
    if out is None:
        out = np.zeros(packed_bytes(c, n), dtype=np.uint8)
    if want_sum and sum_out is None:
        sum_out = np.zeros(n, dtype=np.float32)
    sp = _ptr(sum_out) if sum_out is not None else None
    if tiles is None:
        st = _load().rco_dequant_reduce_requant(_codec(c), arr, k, n, _ptr(out), sp)
    else:
        st = _load().rco_dequant_reduce_requant_tiles(_codec(c), arr, k, n, _ptr(out), sp,
                                                      tiles[0], tiles[1])
    _check(st)
    return out, sum_out


def _tile_ranges(tiles: int, parts: int):
    step = (tiles + parts - 1) // parts
    return [(a, min(a + step, tiles)) for a in range(0, tiles, step)]


def quantize_pack_parallel(c, x: np.ndarray, dtype: int | None = None, threads: int = 8):
    """Same bytes as quantize_pack, tile ranges spread over threads (ctypes
    releases the GIL during the call)."""
    x = np.ascontiguousarray(x)
    out = np.zeros(packed_bytes(c, x.size), dtype=np.uint8)
    tiles = (x.size + TILE - 1) // TILE
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda r: quantize_pack(c, x, dtype, tiles=r, out=out), _tile_ranges(tiles, threads)))
    return out


def dequant_reduce_requant_parallel(c, streams, n: int, want_sum: bool = False, threads: int = 8):
    out = np.zeros(packed_bytes(c, n), dtype=np.uint8)
    sum_out = np.zeros(n, dtype=np.float32) if want_sum else None
    tiles = (n + TILE - 1) // TILE
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda r: dequant_reduce_requant(c, streams, n, want_sum, tiles=r, out=out,
                                                     sum_out=sum_out), _tile_ranges(tiles, threads)))
    return out, sum_out


# ---- element-wise scalar rules (vectorised through the C loops) ----------

def _map(name, out_dtype, *arrays, extra=None):
    arrays = [np.ascontiguousarray(a) for a in arrays]
    n = arrays[0].size
    out = np.empty(n, dtype=out_dtype)
    args = [_ptr(a) for a in arrays]
    if extra is not None:
        args.append(extra)
    getattr(_load(), name)(*args, _ptr(out), n)
    return out


def f32_to_f16_bits(x):
    return _map("rco_map_f32_to_f16", np.uint16, np.asarray(x, dtype=np.float32))


def f32_to_bf16_bits(x):
    return _map("rco_map_f32_to_bf16", np.uint16, np.asarray(x, dtype=np.float32))


def f16_bits_to_f32(h):
    return _map("rco_map_f16_to_f32", np.float32, np.asarray(h, dtype=np.uint16))


def bf16_bits_to_f32(h):
    return _map("rco_map_bf16_to_f32", np.float32, np.asarray(h, dtype=np.uint16))


def widen_to_f32(x: np.ndarray, dtype: int | None = None) -> np.ndarray:
    """x (float32, float16, or uint16 bf16 bits with dtype=DT_BF16) widened
    exactly to float32."""
    x = np.ascontiguousarray(x)
    dt = _dtype_code(x, dtype)
    if dt == DT_FP32:
        return x.astype(np.float32)
    if dt == DT_FP16:
        return f16_bits_to_f32(x.view(np.uint16))
    return bf16_bits_to_f32(x.view(np.uint16))


def e4m3_mag_of_quotient(num, den):
    num = np.asarray(num, dtype=np.float64)
    den = np.broadcast_to(np.asarray(den, dtype=np.float64), num.shape)
    return _map("rco_map_e4m3_mag", np.int32, num, den)


def e2m1_mag_of(v):
    return _map("rco_map_e2m1_mag", np.int32, np.asarray(v, dtype=np.float64))


def int_mag(v_abs, s, qmax):
    """min(round-half-even(|v| / s), qmax) of the exact quotient, element-wise
    (float32 |v|, fp16-valued float32 s > 0)."""
    v_abs = np.ascontiguousarray(v_abs, dtype=np.float32)
    s = np.ascontiguousarray(np.broadcast_to(np.asarray(s, dtype=np.float32), v_abs.shape))
    out = np.empty(v_abs.size, dtype=np.int32)
    _load().rco_map_int_mag(_ptr(v_abs), _ptr(s), qmax, _ptr(out), v_abs.size)
    return out


def int_scale_bits(amax, qmax):
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(amax.size, dtype=np.uint16)
    _load().rco_map_int_scale_bits(_ptr(amax), qmax, _ptr(out), amax.size)
    return out


def fp8_scale(amax):
    return _map("rco_map_fp8_scale", np.float32, np.asarray(amax, dtype=np.float32))


def mx_exponent(amax):
    return _map("rco_map_mx_exponent", np.int32, np.asarray(amax, dtype=np.float32))


def e4m3_decode(code: int) -> float:
    return _load().rco_e4m3_decode(code)


def e2m1_decode(nib: int) -> float:
    return _load().rco_e2m1_decode(nib)


def e8m0_decode(b: int) -> float:
    return _load().rco_e8m0_decode(b)


def e5m2_decode(code: int) -> float:
    return _load().rco_e5m2_decode(code)


def e5m2_mag_of_quotient(num, den):
    num = np.asarray(num, dtype=np.float64)
    den = np.broadcast_to(np.asarray(den, dtype=np.float64), num.shape)
    return _map("rco_map_e5m2_mag", np.int32, num, den)


def elem_emax(fmt: int) -> int:
    return _load().rco_elem_emax(fmt)


def e8m0_exponent(amax, emax: int):
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(amax.size, dtype=np.int32)
    _load().rco_map_e8m0_exponent(_ptr(amax), emax, _ptr(out), amax.size)
    return out


def fp8_scale_f32(amax: float, fmt: int) -> float:
    return _load().rco_fp8_scale_f32(amax, fmt)


def fp8_scale_f16_bits(amax, fmt: int):
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(amax.size, dtype=np.uint16)
    _load().rco_map_fp8_scale_f16_bits(_ptr(amax), fmt, _ptr(out), amax.size)
    return out


def allreduce_emulate(c, msgs, dtype: int, two_shot: bool = True):
    """What a quantized all-reduce of the messages (one per rank) delivers,
    composed from the operations above: quantize every message, reduce the
    packed streams (FP32 sums in message order), then either unpack the
    requantized sum (two-shot) or round the sums to the messages' dtype
    (one-shot).  Returns (out, packed requantized sum)."""
    n = msgs[0].size
    streams = [quantize_pack(c, m, dtype=dtype) for m in msgs]
    packed, sums = dequant_reduce_requant(c, streams, n, want_sum=True)
    if two_shot:
        return unpack_dequant(c, packed, n, dtype), packed
    if dtype == DT_FP32:
        return sums, packed
    if dtype == DT_FP16:
        return f32_to_f16_bits(sums).view(np.float16), packed
    return f32_to_bf16_bits(sums), packed


def mxfp4_gemv(w_packed: np.ndarray, rows: int, cols: int, x: np.ndarray, x_dtype: int | None = None):
    """y = W x on an MXFP4-packed row-major matrix (row r = tiles r*cols/2048
    ...), by its definition: the dot product of each row's decoded weights
    with x, summed exactly.  Weights decode exactly to binary32 (E2M1 value
    times 2^e, unpack_dequant), x widens exactly, and each product is exact in
    binary64 (at most 2 + 24 significant bits, exponents within range);
    math.fsum adds them exactly and rounds once to binary64.  Returns
    (y, mag): the float64 sums and the float64 sums of |W_ij x_j|, the scale
    of the rounding bound an implementation is held to.  The pages fix no
    summation order ("ML-SpecQD: Multi-Level Speculative Decoding with
    Quantized Drafts", abstract: MXFP4 weights direct-cast from BF16)."""
    if cols <= 0 or cols % TILE:
        raise ValueError("cols must be a positive multiple of 2048")
    w_packed = np.ascontiguousarray(w_packed, dtype=np.uint8)
    if w_packed.size < packed_bytes(MXFP4, rows * cols) or np.asarray(x).size < cols:
        raise ValueError("w_packed or x too small")
    wd = unpack_dequant(MXFP4, w_packed, rows * cols, DT_FP32).reshape(rows, cols).astype(np.float64)
    xd = widen_to_f32(np.asarray(x)[:cols], x_dtype).astype(np.float64)
    prod = wd * xd
    y = np.array([math.fsum(r) for r in prod], dtype=np.float64)
    mag = np.array([math.fsum(r) for r in np.abs(prod)], dtype=np.float64)
    return y, mag
