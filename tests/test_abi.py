"""The C-ABI library loads, exports every function include/rcodec.h declares,
agrees with the oracle on enums and sizes, and returns the documented status
for every invalid argument -- all before any HIP call, so no GPU is needed."""
import ctypes
import os
import re

import pytest

import oracle
import reduction_codec_amd as rca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rcodec.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rc_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = rca.lib()
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version():
    assert rca.lib().rc_abi_version() == 3 == rca.ABI_VERSION


def test_enums_agree_with_oracle():
    src = open(HEADER).read()
    for key, val in [("RC_FMT_INT4", oracle.FMT_INT4), ("RC_FMT_INT3", oracle.FMT_INT3),
                     ("RC_FMT_FP8_E4M3", oracle.FMT_FP8_E4M3), ("RC_FMT_MXFP4", oracle.FMT_MXFP4),
                     ("RC_FMT_FP8_E5M2", oracle.FMT_FP8_E5M2),
                     ("RC_SCALE_FP16", oracle.SCALE_FP16), ("RC_SCALE_FP32", oracle.SCALE_FP32),
                     ("RC_SCALE_E8M0", oracle.SCALE_E8M0), ("RC_DT_FP32", oracle.DT_FP32),
                     ("RC_DT_FP16", oracle.DT_FP16), ("RC_DT_BF16", oracle.DT_BF16),
                     ("RC_OK", oracle.OK), ("RC_ERR_NULL", oracle.ERR_NULL),
                     ("RC_ERR_UNSUPPORTED", oracle.ERR_UNSUPPORTED), ("RC_ERR_ALIGN", oracle.ERR_ALIGN),
                     ("RC_ERR_RANGE", oracle.ERR_RANGE), ("RC_ERR_HIP", oracle.ERR_HIP)]:
        m = re.search(rf"\b{key}\s*=\s*(\d+)", src)
        assert m and int(m.group(1)) == val, key


@pytest.mark.parametrize("name", ["int4", "int3", "fp8", "mxfp4"])
def test_sizes_agree_with_oracle(name):
    c = rca.CODECS[name]
    assert rca.tile_bytes(c) == oracle.tile_bytes(oracle.CODECS[name])
    for n in [0, 1, 2047, 2048, 2049, 33554432, 10**9 + 7]:
        assert rca.packed_bytes(c, n) == oracle.packed_bytes(oracle.CODECS[name], n)


def test_codec_lists_agree_with_oracle():
    assert sorted(rca.ALL_CODECS) == sorted(oracle.ALL_CODECS)
    for name, c in rca.ALL_CODECS.items():
        assert (c.format, c.scale, c.block) == oracle.ALL_CODECS[name]
        assert rca.tile_bytes(c) == oracle.tile_bytes(oracle.ALL_CODECS[name]), name
        assert rca.packed_bytes(c, 5 * 2048 + 7) == oracle.packed_bytes(oracle.ALL_CODECS[name], 5 * 2048 + 7)


def test_unsupported_codecs_have_no_size():
    for c in [(1, 2, 32), (2, 2, 32), (4, 1, 32), (4, 2, 32), (1, 1, 8), (3, 2, 128), (5, 2, 48), (9, 1, 32),
              (0, 3, 32)]:
        assert rca.lib().rc_tile_bytes(rca.Codec(*c)) == 0
        assert oracle.tile_bytes(c) == 0


A = 0x10000          # an aligned, non-null address that is never dereferenced
M = 0x10008          # misaligned


def st_q(codec, dt, inp, n, out):
    return rca.lib().rc_quantize_pack(codec, dt, inp, n, out, None)


def st_u(codec, inp, n, dt, out):
    return rca.lib().rc_unpack_dequant(codec, inp, n, dt, out, None)


def st_r(codec, ptrs, k, n, out, sums=None):
    arr = None if ptrs is None else (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return rca.lib().rc_dequant_reduce_requant(codec, arr, k, n, out, sums, None)


def test_quantize_error_paths():
    c = rca.INT3
    assert st_q(rca.Codec(2, 1, 8), 3, A, 10, A) == rca.ERR_UNSUPPORTED
    assert st_q(rca.Codec(2, 2, 32), 3, A, 10, A) == rca.ERR_UNSUPPORTED
    assert st_q(rca.Codec(9, 1, 32), 3, A, 10, A) == rca.ERR_UNSUPPORTED
    assert st_q(c, 7, A, 10, A) == rca.ERR_UNSUPPORTED
    assert st_q(c, 3, None, 10, A) == rca.ERR_NULL
    assert st_q(c, 3, A, 10, None) == rca.ERR_NULL
    assert st_q(c, 3, M, 10, A) == rca.ERR_ALIGN
    assert st_q(c, 3, A, 10, M) == rca.ERR_ALIGN
    assert st_q(c, 3, None, 0, None) == rca.OK          # n = 0: no-op, no launch
    assert st_q(c, 3, A, (1 << 40) + 1, A) == rca.ERR_RANGE


def test_unpack_error_paths():
    c = rca.MXFP4
    assert st_u(rca.Codec(4, 1, 32), A, 10, 1, A) == rca.ERR_UNSUPPORTED
    assert st_u(rca.Codec(5, 2, 128), A, 10, 1, A) == rca.ERR_UNSUPPORTED
    assert st_u(c, A, 10, 0, A) == rca.ERR_UNSUPPORTED
    assert st_u(c, None, 10, 1, A) == rca.ERR_NULL
    assert st_u(c, A, 10, 1, None) == rca.ERR_NULL
    assert st_u(c, M, 10, 1, A) == rca.ERR_ALIGN
    assert st_u(c, A, 10, 3, M) == rca.ERR_ALIGN
    assert st_u(c, None, 0, 1, None) == rca.OK


def test_reduce_error_paths():
    c = rca.FP8
    assert st_r(rca.Codec(3, 1, 48), [A], 1, 10, A) == rca.ERR_UNSUPPORTED
    assert st_r(rca.Codec(4, 2, 32), [A], 1, 10, A) == rca.ERR_UNSUPPORTED
    assert st_r(c, [A], 0, 10, A) == rca.ERR_RANGE
    assert st_r(c, [A] * 17, 17, 10, A) == rca.ERR_RANGE
    assert st_r(c, None, 2, 10, A) == rca.ERR_NULL
    assert st_r(c, [A, None], 2, 10, A) == rca.ERR_NULL
    assert st_r(c, [A, A], 2, 10, None) == rca.ERR_NULL
    assert st_r(c, [A, M], 2, 10, A) == rca.ERR_ALIGN
    assert st_r(c, [A, A], 2, 10, M) == rca.ERR_ALIGN
    assert st_r(c, [A, A], 2, 10, A, M) == rca.ERR_ALIGN
    assert st_r(c, [A, A], 2, 0, A) == rca.OK
    assert st_r(c, [A, A], 2, (1 << 40) + 1, A) == rca.ERR_RANGE


def test_copy_error_paths():
    l = rca.lib()
    assert l.rc_copy(None, A, 16, None) == rca.ERR_NULL
    assert l.rc_copy(A, M, 16, None) == rca.ERR_ALIGN
    assert l.rc_copy(A, A, 17, None) == rca.ERR_ALIGN
    assert l.rc_copy(None, None, 0, None) == rca.OK


def test_status_strings():
    l = rca.lib()
    for s in range(6):
        assert l.rc_status_str(s)
    assert l.rc_status_str(99) == b"unknown status"


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        rca.quantize_pack(torch.zeros(4), rca.INT3)


def test_product_path_does_not_import_the_oracle():
    """The package and the kernels never reference oracle/ (which is test
    infrastructure) and contain no CPU fallback."""
    pkg = os.path.join(ROOT, "reduction_codec_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "rcodec_oracle" not in text and "rco_" not in text, f


def test_allreduce_emulate_error_paths():
    l = rca.lib()

    def ar(codec, dt, ptrs, k, n, out, packed=None, two_shot=1):
        arr = None if ptrs is None else (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
        return l.rc_allreduce_emulate(codec, dt, arr, k, n, two_shot, out, packed, None)

    assert ar(rca.Codec(2, 2, 32), 3, [A], 1, 10, A) == rca.ERR_UNSUPPORTED       # INT3 with an FP32 scale
    assert ar(rca.Codec(3, 2, 48), 3, [A], 1, 10, A) == rca.ERR_UNSUPPORTED       # block of 48
    for name in rca.ALL_CODECS:                                                    # every codec: n = 0 is a no-op
        assert ar(rca.ALL_CODECS[name], 3, [A], 1, 0, A) == rca.OK, name
    assert ar(rca.INT3, 9, [A], 1, 10, A) == rca.ERR_UNSUPPORTED
    assert ar(rca.INT3, 3, [A], 0, 10, A) == rca.ERR_RANGE
    assert ar(rca.INT3, 3, [A] * 17, 17, 10, A) == rca.ERR_RANGE
    assert ar(rca.INT3, 3, None, 2, 10, A) == rca.ERR_NULL
    assert ar(rca.INT3, 3, [A, None], 2, 10, A) == rca.ERR_NULL
    assert ar(rca.INT3, 3, [A, A], 2, 10, None) == rca.ERR_NULL
    assert ar(rca.INT3, 3, [A, M], 2, 10, A) == rca.ERR_ALIGN
    assert ar(rca.INT3, 3, [A, A], 2, 10, M) == rca.ERR_ALIGN
    assert ar(rca.INT3, 3, [A, A], 2, 10, A, M) == rca.ERR_ALIGN
    assert ar(rca.INT3, 3, [A, A], 2, 0, A) == rca.OK
    assert ar(rca.INT3, 3, [A, A], 2, (1 << 40) + 1, A) == rca.ERR_RANGE


def test_mxfp4_gemv_error_paths():
    l = rca.lib()
    g = lambda w, rows, cols, xt, x, yt, y: l.rc_mxfp4_gemv(w, rows, cols, xt, x, yt, y, None)
    assert g(A, 4, 4096, 7, A, 1, A) == rca.ERR_UNSUPPORTED
    assert g(A, 4, 4096, 3, A, 0, A) == rca.ERR_UNSUPPORTED
    assert g(A, 4, 1000, 3, A, 1, A) == rca.ERR_RANGE
    assert g(A, 4, 0, 3, A, 1, A) == rca.ERR_RANGE
    assert g(A, 0, 4096, 3, A, 1, A) == rca.OK
    assert g(None, 4, 4096, 3, A, 1, A) == rca.ERR_NULL
    assert g(A, 4, 4096, 3, None, 1, A) == rca.ERR_NULL
    assert g(A, 4, 4096, 3, A, 1, None) == rca.ERR_NULL
    assert g(M, 4, 4096, 3, A, 1, A) == rca.ERR_ALIGN
    assert g(A, 4, 4096, 3, M, 1, A) == rca.ERR_ALIGN
    assert g(A, 1 << 40, 4096, 3, A, 1, A) == rca.ERR_RANGE


def test_mxfp4_gemv_rejects_x_of_4_gib_or_more():
    """x is addressed with 32-bit byte offsets: cols * sizeof(x) >= 2^32 is
    refused before any HIP call (fp32 x from 2^30 columns, 16-bit x from
    2^31), and the largest accepted widths still pass validation (rows = 0)."""
    l = rca.lib()
    g = lambda rows, cols, xt: l.rc_mxfp4_gemv(A, rows, cols, xt, A, 1, A, None)
    assert g(1, 1 << 30, 1) == rca.ERR_RANGE          # fp32: exactly 4 GiB
    assert g(1, 1 << 31, 3) == rca.ERR_RANGE          # bf16: exactly 4 GiB
    assert g(1, 1 << 31, 2) == rca.ERR_RANGE          # fp16
    assert g(1, (1 << 30) + 2048, 1) == rca.ERR_RANGE
    assert g(0, (1 << 30) - 2048, 1) == rca.OK         # largest fp32 width, nothing to do
    assert g(0, (1 << 31) - 2048, 3) == rca.OK
