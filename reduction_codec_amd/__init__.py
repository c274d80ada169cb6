"""Python binding of the MI355X codec library ``librcodec.so``.

Argument marshalling only: every step of the codec runs in the HIP kernels
behind the C ABI declared in ``include/rcodec.h``.  PyTorch provides device
memory and the current stream; nothing here computes on the CPU, and there is
no fallback: if the library is not built, every call raises.

Entry points (same names as the C ABI, minus the ``rc_`` prefix):

* ``quantize_pack(x, codec)``             -> packed uint8 tensor
* ``unpack_dequant(packed, codec, n, dtype)`` -> tensor of n values
* ``dequant_reduce_requant(streams, codec, n, sum_out=False)``
                                           -> (packed, fp32 sums or None)
* ``tile_bytes(codec)``, ``packed_bytes(codec, n)``, ``copy(dst, src)``
"""
from __future__ import annotations

import ctypes
import os

import torch  # must load before librcodec.so: both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librcodec.so")

TILE = 2048
BLOCK = 32
MAX_STREAMS = 16

FMT_INT4, FMT_INT3, FMT_FP8_E4M3, FMT_MXFP4, FMT_FP8_E5M2 = 1, 2, 3, 4, 5
SCALE_FP16, SCALE_FP32, SCALE_E8M0 = 1, 2, 3
DT_FP32, DT_FP16, DT_BF16 = 1, 2, 3
OK, ERR_NULL, ERR_UNSUPPORTED, ERR_ALIGN, ERR_RANGE, ERR_HIP = 0, 1, 2, 3, 4, 5


class Codec(ctypes.Structure):
    """rc_codec: element format, scale type, block size (passed by value)."""
    _fields_ = [("format", ctypes.c_int32), ("scale", ctypes.c_int32), ("block", ctypes.c_int32)]

    def __repr__(self):
        return f"Codec({self.format}, {self.scale}, {self.block})"


INT4 = Codec(FMT_INT4, SCALE_FP16, BLOCK)
INT3 = Codec(FMT_INT3, SCALE_FP16, BLOCK)
FP8 = Codec(FMT_FP8_E4M3, SCALE_FP32, BLOCK)
MXFP4 = Codec(FMT_MXFP4, SCALE_E8M0, BLOCK)
CODECS = {"int4": INT4, "int3": INT3, "fp8": FP8, "mxfp4": MXFP4}


def _all_codecs():
    """Every codec the library supports, by name "<element>_<scale>_b<block>"
    (also accepted wherever a codec is expected)."""
    elems = {"int4": FMT_INT4, "int3": FMT_INT3, "e4m3": FMT_FP8_E4M3, "e5m2": FMT_FP8_E5M2, "e2m1": FMT_MXFP4}
    scales = {"f16": SCALE_FP16, "f32": SCALE_FP32, "e8m0": SCALE_E8M0}
    allowed = {"int4": ("f16", "e8m0"), "int3": ("f16", "e8m0"), "e4m3": ("f32", "f16", "e8m0"),
               "e5m2": ("f32", "f16", "e8m0"), "e2m1": ("e8m0",)}
    return {f"{e}_{sc}_b{b}": Codec(elems[e], scales[sc], b)
            for e, scs in allowed.items() for sc in scs for b in (16, 32, 64)}


ALL_CODECS = _all_codecs()

ABI_VERSION = 3                       # RC_ABI_VERSION of include/rcodec.h
_DTYPES = {torch.float32: DT_FP32, torch.float16: DT_FP16, torch.bfloat16: DT_BF16}
_lib = None


class CodecError(RuntimeError):
    """A non-zero rc_status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().rc_status_str(status).decode()} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded librcodec.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                           "(the codec has no CPU fallback)")
    l = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    l.rc_tile_bytes.restype, l.rc_tile_bytes.argtypes = sz, [Codec]
    l.rc_packed_bytes.restype, l.rc_packed_bytes.argtypes = sz, [Codec, sz]
    l.rc_quantize_pack.restype, l.rc_quantize_pack.argtypes = i32, [Codec, i32, vp, sz, vp, vp]
    l.rc_unpack_dequant.restype, l.rc_unpack_dequant.argtypes = i32, [Codec, vp, sz, i32, vp, vp]
    l.rc_dequant_reduce_requant.restype = i32
    l.rc_dequant_reduce_requant.argtypes = [Codec, ctypes.POINTER(vp), i32, sz, vp, vp, vp]
    l.rc_copy.restype, l.rc_copy.argtypes = i32, [vp, vp, sz, vp]
    l.rc_mxfp4_gemv.restype = i32
    l.rc_mxfp4_gemv.argtypes = [vp, sz, sz, i32, vp, i32, vp, vp]
    l.rc_allreduce_emulate.restype = i32
    l.rc_allreduce_emulate.argtypes = [Codec, i32, ctypes.POINTER(vp), i32, sz, i32, vp, vp, vp]
    l.rc_status_str.restype, l.rc_status_str.argtypes = ctypes.c_char_p, [i32]
    l.rc_abi_version.restype, l.rc_abi_version.argtypes = i32, []
    if l.rc_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {l.rc_abi_version()}, this binding expects "
                           f"{ABI_VERSION}; rebuild the library")
    _lib = l
    return l


def _codec(c) -> Codec:
    if isinstance(c, Codec):
        return c
    if isinstance(c, str):
        return CODECS[c] if c in CODECS else ALL_CODECS[c]
    return Codec(*c)


def _stream(stream, dev: torch.device) -> ctypes.c_void_p:
    """The HIP stream to launch on: the given one (which must belong to the
    tensors' device) or that device's current stream."""
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return ctypes.c_void_p(stream.cuda_stream)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _same_device(dev: torch.device, *named):
    for name, t in named:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _mine(t: torch.Tensor, stream) -> torch.Tensor:
    """A tensor this module allocated on the current stream for work enqueued
    on `stream`: tell torch's caching allocator, so the memory is not handed
    out again before that stream has finished with it."""
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _check_dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ok(status: int, what: str):
    if status != OK:
        raise CodecError(status, what)


def tile_bytes(codec) -> int:
    return lib().rc_tile_bytes(_codec(codec))


def packed_bytes(codec, n: int) -> int:
    return lib().rc_packed_bytes(_codec(codec), n)


def quantize_pack(x: torch.Tensor, codec, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Block-quantize the elements of x (bf16 / fp16 / fp32, any shape, taken
    flat) into ``packed_bytes(codec, x.numel())`` bytes."""
    c = _codec(codec)
    _check_dev(x, "x")
    hs = _stream(stream, x.device)
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    n = x.numel()
    if out is None:
        out = _mine(torch.empty(packed_bytes(c, n), dtype=torch.uint8, device=x.device), stream)
    _check_dev(out, "out")
    _same_device(x.device, ("out", out))
    if out.numel() < packed_bytes(c, n) or out.dtype != torch.uint8:
        raise ValueError("out must be a uint8 tensor of packed_bytes(codec, n) bytes")
    with torch.cuda.device(x.device):
        _ok(lib().rc_quantize_pack(c, _DTYPES[x.dtype], x.data_ptr(), n, out.data_ptr(), hs),
            "rc_quantize_pack")
    return out


def unpack_dequant(packed: torch.Tensor, codec, n: int, dtype: torch.dtype = torch.float32,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode the first n elements of a packed stream to dtype."""
    c = _codec(codec)
    _check_dev(packed, "packed")
    hs = _stream(stream, packed.device)
    if _nbytes(packed) < packed_bytes(c, n):
        raise ValueError("packed is shorter than packed_bytes(codec, n)")
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported output dtype {dtype}")
    if out is None:
        out = _mine(torch.empty(n, dtype=dtype, device=packed.device), stream)
    _check_dev(out, "out")
    _same_device(packed.device, ("out", out))
    if out.numel() < n or out.dtype != dtype:
        raise ValueError("out must hold n elements of dtype")
    with torch.cuda.device(packed.device):
        _ok(lib().rc_unpack_dequant(c, packed.data_ptr(), n, _DTYPES[dtype], out.data_ptr(), hs),
            "rc_unpack_dequant")
    return out


def dequant_reduce_requant(streams, codec, n: int, out: torch.Tensor | None = None,
                           sum_out: bool | torch.Tensor = False, stream=None):
    """Dequantize K packed streams, add them in FP32 in stream order and
    requantize.  Returns (packed, sums) with sums None unless requested."""
    c = _codec(codec)
    streams = list(streams)
    k = len(streams)
    if not 1 <= k <= MAX_STREAMS:
        raise ValueError(f"need 1..{MAX_STREAMS} streams, got {k}")
    need = packed_bytes(c, n)
    dev = streams[0].device if streams and isinstance(streams[0], torch.Tensor) else None
    for j, s in enumerate(streams):
        _check_dev(s, f"streams[{j}]")
        _same_device(dev, (f"streams[{j}]", s))
        if _nbytes(s) < need:
            raise ValueError(f"streams[{j}] is shorter than packed_bytes(codec, n)")
    hs = _stream(stream, dev)
    if out is None:
        out = _mine(torch.empty(need, dtype=torch.uint8, device=dev), stream)
    _check_dev(out, "out")
    _same_device(dev, ("out", out))
    if _nbytes(out) < need:
        raise ValueError("out is shorter than packed_bytes(codec, n)")
    sums = None
    if isinstance(sum_out, torch.Tensor):
        sums = sum_out
        _check_dev(sums, "sum_out")
        _same_device(dev, ("sum_out", sums))
        if sums.dtype != torch.float32 or sums.numel() < n:
            raise ValueError("sum_out must hold n float32 values")
    elif sum_out:
        sums = _mine(torch.empty(n, dtype=torch.float32, device=dev), stream)
    ptrs = (ctypes.c_void_p * k)(*[s.data_ptr() for s in streams])
    with torch.cuda.device(dev):
        _ok(lib().rc_dequant_reduce_requant(c, ptrs, k, n, out.data_ptr(),
                                            sums.data_ptr() if sums is not None else None, hs),
            "rc_dequant_reduce_requant")
    return out, sums


def allreduce_emulate(msgs, codec, two_shot: bool = True, out: torch.Tensor | None = None,
                      packed_out: bool | torch.Tensor = False, stream=None):
    """Fused one-GPU emulation of a quantized all-reduce of the messages (one
    per emulated rank, same dtype and length).  Returns (out, packed or
    None); see rc_allreduce_emulate in include/rcodec.h."""
    c = _codec(codec)
    msgs = list(msgs)
    k = len(msgs)
    if not 1 <= k <= MAX_STREAMS:
        raise ValueError(f"need 1..{MAX_STREAMS} messages, got {k}")
    dt = msgs[0].dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    n = msgs[0].numel()
    dev = msgs[0].device
    for j, m in enumerate(msgs):
        _check_dev(m, f"msgs[{j}]")
        _same_device(dev, (f"msgs[{j}]", m))
        if m.dtype != dt or m.numel() != n:
            raise ValueError("all messages need the same dtype and length")
    hs = _stream(stream, dev)
    if out is None:
        out = _mine(torch.empty(n, dtype=dt, device=dev), stream)
    _check_dev(out, "out")
    _same_device(dev, ("out", out))
    if out.dtype != dt or out.numel() < n:
        raise ValueError("out must hold n elements of the messages' dtype")
    packed = None
    if isinstance(packed_out, torch.Tensor):
        packed = packed_out
        _check_dev(packed, "packed_out")
        _same_device(dev, ("packed_out", packed))
        if packed.numel() < packed_bytes(c, n) or packed.dtype != torch.uint8:
            raise ValueError("packed_out must be a uint8 tensor of packed_bytes(codec, n) bytes")
    elif packed_out:
        packed = _mine(torch.empty(packed_bytes(c, n), dtype=torch.uint8, device=dev), stream)
    ptrs = (ctypes.c_void_p * k)(*[m.data_ptr() for m in msgs])
    with torch.cuda.device(dev):
        _ok(lib().rc_allreduce_emulate(c, _DTYPES[dt], ptrs, k, n, 1 if two_shot else 0, out.data_ptr(),
                                       packed.data_ptr() if packed is not None else None, hs),
            "rc_allreduce_emulate")
    return out, packed


def mxfp4_gemv(w_packed: torch.Tensor, rows: int, cols: int, x: torch.Tensor, out_dtype=torch.float32,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = W x with W (rows x cols, row-major) packed by quantize_pack with the
    MXFP4 codec; cols a multiple of 2048.  See rc_mxfp4_gemv."""
    _check_dev(w_packed, "w_packed")
    _check_dev(x, "x")
    _same_device(w_packed.device, ("x", x))
    hs = _stream(stream, w_packed.device)
    if w_packed.dtype != torch.uint8 or w_packed.numel() < packed_bytes(MXFP4, rows * cols):
        raise ValueError("w_packed must hold packed_bytes(MXFP4, rows * cols) bytes")
    if x.dtype not in _DTYPES or x.numel() < cols:
        raise ValueError("x must hold cols fp32 / fp16 / bf16 values")
    if out_dtype not in _DTYPES:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    if out is None:
        out = _mine(torch.empty(rows, dtype=out_dtype, device=x.device), stream)
    _check_dev(out, "out")
    _same_device(w_packed.device, ("out", out))
    if out.dtype != out_dtype or out.numel() < rows:
        raise ValueError("out must hold rows values of out_dtype")
    with torch.cuda.device(w_packed.device):
        _ok(lib().rc_mxfp4_gemv(w_packed.data_ptr(), rows, cols, _DTYPES[x.dtype], x.data_ptr(), _DTYPES[out_dtype],
                                out.data_ptr(), hs), "rc_mxfp4_gemv")
    return out


def copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> torch.Tensor:
    """Byte copy through the library's 16-byte vector copy kernel."""
    _check_dev(dst, "dst")
    _check_dev(src, "src")
    _same_device(src.device, ("dst", dst))
    hs = _stream(stream, src.device)
    nbytes = _nbytes(src)
    if _nbytes(dst) < nbytes:
        raise ValueError("dst too small")
    with torch.cuda.device(src.device):
        _ok(lib().rc_copy(src.data_ptr(), dst.data_ptr(), nbytes, hs), "rc_copy")
    return dst
