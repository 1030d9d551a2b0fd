"""The C-ABI library loads and exports what include/tq.h declares; host-side
argument checks return their error codes before anything reaches the GPU.

No test here launches a kernel: every call below is rejected by the host-side
validation in tq_api.hip, which runs before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")
PROBE_HEADER = os.path.join(ROOT, "include", "tq_probe.h")


def _lib():
    import ternary_weight_only_amd as tq
    if not os.path.exists(tq.binding.LIB_PATH):
        from ternary_weight_only_amd import build
        build.build_library()
    return tq.lib()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for f in ("tq_quantize_pack", "tq_unpack", "tq_gemv", "tq_gemm"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    import ternary_weight_only_amd.binding as b
    assert sorted(b.SYMBOLS) == declared_functions()


def test_library_exports_every_probe_symbol():
    lib = _lib()
    import ternary_weight_only_amd.binding as b
    assert sorted(b.PROBE_SYMBOLS) == declared_functions(PROBE_HEADER)
    for name in b.PROBE_SYMBOLS:
        assert hasattr(lib, name), name


def test_probe_argument_errors():
    lib = _lib()
    assert lib.tq_probe_read_stream(None, 1024, 4, FAKE, None) == -1
    assert lib.tq_probe_read_stream(FAKE, 1024, 4, None, None) == -1
    assert lib.tq_probe_read_stream(FAKE + 8, 1024, 4, FAKE, None) == -4
    assert lib.tq_probe_read_stream(FAKE, 1000, 4, FAKE, None) == -2   # not 16-byte chunks
    assert lib.tq_probe_read_stream(FAKE, 0, 4, FAKE, None) == -2
    assert lib.tq_probe_read_stream(FAKE, 1024, 0, FAKE, None) == -2
    assert lib.tq_probe_read_stream(FAKE, 1024, 65536, FAKE, None) == -2
    assert lib.tq_probe_mfma_bf16(10, 4, None, None) == -1
    assert lib.tq_probe_mfma_bf16(0, 4, FAKE, None) == -2
    assert lib.tq_probe_mfma_bf16(10, 0, FAKE, None) == -2
    assert lib.tq_probe_mfma_bf16((1 << 24) + 1, 4, FAKE, None) == -2
    assert lib.tq_probe_lds_table(10, 4, None, None, None) == -1
    assert lib.tq_probe_lds_table(0, 4, FAKE, None, None) == -2
    assert lib.tq_probe_lds_table(10, 65536, FAKE, None, None) == -2
    assert lib.tq_probe_valu(0, 10, 4, None, None, None) == -1
    assert lib.tq_probe_valu(2, 10, 4, FAKE, None, None) == -2
    assert lib.tq_probe_valu(-1, 10, 4, FAKE, None, None) == -2
    assert lib.tq_probe_valu(1, 0, 4, FAKE, None, None) == -2
    assert lib.tq_probe_valu(1, 10, 0, FAKE, None, None) == -2


def test_packed_bytes_helper():
    lib = _lib()
    assert lib.tq_packed_bytes(256, 512, 64) == 256 * 8 * 13
    assert lib.tq_packed_bytes(256, 320, 64) == 256 * 65
    assert lib.tq_packed_bytes(3584, 1024, 128) == 3584 * 8 * 26
    assert lib.tq_packed_bytes(1, 100, 64) == 0
    assert lib.tq_packed_bytes(0, 128, 64) == 0
    assert lib.tq_packed_bytes(1 << 62, 4096, 128) == 0   # overflows int64
    assert lib.tq_packed_row_bytes(1024, 128) == 8 * 26
    assert lib.tq_packed_row_bytes(320, 64) == 65
    assert lib.tq_packed_row_bytes(70, 7) == 10 * 2       # any G >= 1
    assert lib.tq_packed_row_bytes(100, 64) == 0
    assert lib.tq_packed_row_bytes(128, 0) == 0


def test_binding_rejects_host_tensors_before_the_library():
    """Every binding entry point refuses host (CPU) tensors with TQError;
    nothing is passed to the library."""
    import torch
    import ternary_weight_only_amd as tq
    w = torch.zeros(4, 64, dtype=torch.bfloat16)
    x = torch.zeros(1, 64, dtype=torch.bfloat16)
    p = torch.zeros(4, 13, dtype=torch.uint8)
    s = torch.zeros(4, 1, dtype=torch.float16)
    calls = [lambda: tq.quantize_pack(w, 64), lambda: tq.fake_quantize(w, 64),
             lambda: tq.quantize_pack_batched([w], 64), lambda: tq.unpack(p, 4, 64, 64),
             lambda: tq.unpack_batched([p], 4, 64, 64), lambda: tq.dequantize(p, s, 4, 64, 64),
             lambda: tq.dequantize_batched([p], [s], 4, 64, 64),
             lambda: tq.gemv(x, p, s, 4, 64, 64), lambda: tq.gemm(x, p, s, 4, 64, 64),
             lambda: tq.gemv_batched([x], [p], [s], 4, 64, 64),
             lambda: tq.gemm_batched([x], [p], [s], 4, 64, 64),
             lambda: tq.gemv_grouped([x], [p], [s], [4], [64], 64),
             lambda: tq.gemm_grouped([x], [p], [s], [4], [64], 64),
             lambda: tq.quantize_pack2(w, 64), lambda: tq.unpack2(p, 4, 52, 64),
             lambda: tq.gemv2(x, p, s, 4, 64, 64),
             lambda: tq.w4a16_gemv(x, torch.zeros(4, 8, dtype=torch.int32), w[:, :1], w[:, :1],
                                   4, 64, 64)]
    for c in calls:
        with pytest.raises(tq.TQError):
            c()


FAKE = 0x100000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("fn", ["tq_gemv", "tq_gemm"])
def test_matmul_argument_errors(fn):
    lib = _lib()
    f = getattr(lib, fn)
    assert f(None, FAKE, FAKE, 1, 8, 128, 64, FAKE, None, None) == -1      # NULL
    assert f(FAKE, FAKE, FAKE, 1, 8, 100, 64, FAKE, None, None) == -2      # K % G
    assert f(FAKE, FAKE, FAKE, 1, 0, 128, 64, FAKE, None, None) == -2      # N < 1
    assert f(FAKE, FAKE, FAKE, 0, 8, 128, 64, FAKE, None, None) == -2      # M < 1
    assert f(FAKE, FAKE, FAKE, 1, 8, 96, 32, FAKE, None, None) == -3       # G
    assert f(FAKE + 2, FAKE, FAKE, 1, 8, 128, 64, FAKE, None, None) == -4  # x alignment
    assert f(FAKE, FAKE, FAKE + 1, 1, 8, 128, 64, FAKE, None, None) == -4  # scales
    assert f(FAKE, FAKE, FAKE, 1, 8, 128, 64, FAKE + 2, None, None) == -4  # y
    assert f(FAKE, FAKE, FAKE, 1, 1, (1 << 22) + 64, 64, FAKE, None, None) == -2  # K cap
    if fn == "tq_gemv":
        assert f(FAKE, FAKE, FAKE, 17, 8, 128, 64, FAKE, None, None) == -2  # M > 16
        assert f(FAKE, FAKE + 8, FAKE, 1, 8, 128, 64, FAKE, None, None) == -4


@pytest.mark.parametrize("fn", ["tq_gemv_batched", "tq_gemm_batched"])
def test_batched_argument_errors(fn):
    lib = _lib()
    arr = ctypes.c_void_p * 2
    good = arr(FAKE, FAKE + 4096)
    bad_al = arr(FAKE, FAKE + 4)
    nul = arr(FAKE, None)
    f = getattr(lib, fn)
    assert f(0, None, None, None, None, 1, 8, 128, 64, None, None) == 0      # nothing to do
    assert f(-1, good, good, good, good, 1, 8, 128, 64, None, None) == -2
    assert f(2, None, good, good, good, 1, 8, 128, 64, None, None) == -1
    assert f(2, nul, good, good, good, 1, 8, 128, 64, None, None) == -1
    assert f(2, good, good, good, good, 1, 8, 100, 64, None, None) == -2
    if fn == "tq_gemv_batched":
        assert f(2, good, good, good, good, 17, 8, 128, 64, None, None) == -2
    assert f(2, good, good, good, good, 1, 1, (1 << 22) + 64, 64, None, None) == -2
    assert f(2, good, good, good, good, 0, 8, 128, 64, None, None) == -2
    assert f(2, good, good, good, good, 1, 8, 96, 32, None, None) == -3
    assert f(2, bad_al, good, good, good, 1, 8, 128, 64, None, None) == -4


def test_gemm_grouped_argument_errors():
    lib = _lib()
    f = lib.tq_gemm_grouped
    arr = ctypes.c_void_p * 2
    i64 = ctypes.c_int64 * 2
    good = arr(FAKE, FAKE + 4096)
    bad_al = arr(FAKE, FAKE + 4)
    nul = arr(FAKE, None)
    ns, ks = i64(8, 16), i64(128, 256)
    assert f(0, None, None, None, None, 1, None, None, 64, None, None) == 0   # nothing to do
    assert f(-1, good, good, good, good, 1, ns, ks, 64, None, None) == -2
    assert f(2, good, good, good, good, 1, ns, None, 64, None, None) == -1
    assert f(2, good, nul, good, good, 1, ns, ks, 64, None, None) == -1
    assert f(2, good, good, good, good, 0, ns, ks, 64, None, None) == -2     # M < 1
    assert f(2, good, good, good, good, 1, ns, i64(128, 100), 64, None, None) == -2  # K % G
    assert f(2, good, good, good, good, 1, i64(8, 0), ks, 64, None, None) == -2      # N < 1
    assert f(2, good, good, good, good, 1, ns, i64(128, (1 << 22) + 64), 64, None, None) == -2
    assert f(2, good, good, good, good, 1, ns, i64(96, 96), 32, None, None) == -3    # G
    assert f(2, bad_al, good, good, good, 1, ns, ks, 64, None, None) == -4   # x alignment
    assert f(2, good, good, good, arr(FAKE, FAKE + 2), 1, ns, ks, 64, None, None) == -4  # y
    assert f(2, good, good, good, good, 1, ns, ks, 64, FAKE + 2, None) == -4  # status


def test_grouped_argument_errors():
    lib = _lib()
    f = lib.tq_gemv_grouped
    arr = ctypes.c_void_p * 2
    i64 = ctypes.c_int64 * 2
    good = arr(FAKE, FAKE + 4096)
    bad_al = arr(FAKE, FAKE + 4)
    nul = arr(FAKE, None)
    ns, ks = i64(8, 16), i64(128, 256)
    assert f(0, None, None, None, None, None, None, 64, None, None) == 0     # nothing to do
    assert f(-1, good, good, good, good, ns, ks, 64, None, None) == -2
    assert f(2, good, good, good, good, None, ks, 64, None, None) == -1
    assert f(2, nul, good, good, good, ns, ks, 64, None, None) == -1
    assert f(2, good, good, good, good, ns, i64(128, 100), 64, None, None) == -2   # K % G
    assert f(2, good, good, good, good, i64(8, 0), ks, 64, None, None) == -2       # N < 1
    assert f(2, good, good, good, good, ns, i64(128, (1 << 22) + 64), 64, None, None) == -2
    assert f(2, good, good, good, good, ns, ks, 32, None, None) == -3
    assert f(2, bad_al, good, good, good, ns, ks, 64, None, None) == -4
    assert f(2, good, good, good, good, ns, ks, 64, FAKE + 2, None) == -4        # status


def test_quantize_unpack_argument_errors():
    lib = _lib()
    q, u = lib.tq_quantize_pack, lib.tq_unpack
    assert q(None, 4, 128, 64, FAKE, FAKE, None, None) == -1
    assert q(FAKE, 4, 130, 64, FAKE, FAKE, None, None) == -2
    assert q(FAKE, 4, 128, 5, FAKE, FAKE, None, None) == -3
    assert q(FAKE + 2, 4, 128, 64, FAKE, FAKE, None, None) == -4
    assert q(FAKE, 4, 128, 64, FAKE, FAKE + 1, None, None) == -4
    assert q(FAKE, 4, 128, 64, FAKE, FAKE, FAKE + 1, None) == -4
    assert u(None, 4, 128, 64, FAKE, None, None) == -1
    assert u(FAKE, 4, 128, 64, FAKE + 4, None, None) == -4
    assert u(FAKE, 4, 128, 48, FAKE, None, None) == -3
    for rc in (0, -1, -2, -3, -4, -5):
        assert lib.tq_status_string(rc)


def test_fake_quantize_argument_errors():
    f = _lib().tq_fake_quantize
    assert f(None, 4, 128, 64, FAKE, None, None, None) == -1
    assert f(FAKE, 4, 128, 64, None, None, None, None) == -1
    assert f(FAKE, 4, 130, 64, FAKE, None, None, None) == -2
    assert f(FAKE, 4, 128, 48, FAKE, None, None, None) == -3
    assert f(FAKE + 2, 4, 128, 64, FAKE, None, None, None) == -4
    assert f(FAKE, 4, 128, 64, FAKE + 8, None, None, None) == -4
    assert f(FAKE, 4, 128, 64, FAKE, FAKE + 1, None, None) == -4
    assert f(FAKE, 4, 128, 64, FAKE, None, FAKE + 2, None) == -4


def test_quantize_unpack_batched_argument_errors():
    import ctypes
    lib = _lib()
    arr = ctypes.c_void_p * 2

    def ps(*v):
        return arr(*v)
    good = ps(FAKE, FAKE + 4096)
    for f in (lib.tq_quantize_pack_batched, lib.tq_fake_quantize_batched):
        assert f(0, None, 4, 128, 64, None, None, None, None) == 0
        assert f(-1, good, 4, 128, 64, good, good, None, None) == -2
        assert f(2, None, 4, 128, 64, good, good, None, None) == -1
        assert f(2, ps(FAKE, None), 4, 128, 64, good, good, None, None) == -1
        assert f(2, good, 4, 130, 64, good, good, None, None) == -2
        assert f(2, good, 4, 128, 32, good, good, None, None) == -3
        assert f(2, ps(FAKE, FAKE + 8), 4, 128, 64, good, good, None, None) == -4
        assert f(2, good, 4, 128, 64, good, ps(FAKE, FAKE + 1), None, None) == -4
        assert f(2, good, 4, 128, 64, good, good, FAKE + 2, None) == -4
    q, fq = lib.tq_quantize_pack_batched, lib.tq_fake_quantize_batched
    assert q(2, good, 4, 128, 64, good, None, None, None) == -1        # scales required
    assert fq(2, good, 4, 128, 64, None, None, None, None) == -1       # w_hats required
    assert fq(2, good, 4, 128, 64, ps(FAKE, FAKE + 8), None, None, None) == -4
    u = lib.tq_unpack_batched
    assert u(0, None, 4, 128, 64, None, None, None) == 0
    assert u(2, None, 4, 128, 64, good, None, None) == -1
    assert u(2, good, 4, 128, 64, ps(FAKE, None), None, None) == -1
    assert u(2, good, 4, 128, 64, ps(FAKE, FAKE + 4), None, None) == -4
    assert u(2, good, 4, 128, 48, good, None, None) == -3


def test_dequantize_argument_errors():
    d = _lib().tq_dequantize
    assert d(None, FAKE, 4, 128, 64, FAKE, None, None) == -1
    assert d(FAKE, None, 4, 128, 64, FAKE, None, None) == -1
    assert d(FAKE, FAKE, 4, 128, 64, None, None, None) == -1
    assert d(FAKE, FAKE, 0, 128, 64, FAKE, None, None) == -2
    assert d(FAKE, FAKE, 4, 160, 64, FAKE, None, None) == -2
    assert d(FAKE, FAKE, 4, 128, 32, FAKE, None, None) == -3
    assert d(FAKE, FAKE, 4, 128, 64, FAKE + 8, None, None) == -4    # w_hat 16-byte
    assert d(FAKE, FAKE + 1, 4, 128, 64, FAKE, None, None) == -4    # scales 2-byte
    assert d(FAKE, FAKE, 4, 128, 64, FAKE, FAKE + 2, None) == -4    # status 4-byte


def test_dequantize_batched_argument_errors():
    import ctypes
    d = _lib().tq_dequantize_batched
    arr = ctypes.c_void_p * 2

    def ps(*v):
        return arr(*v)
    good = ps(FAKE, FAKE + 64)
    assert d(0, None, None, None, 4, 128, 64, None, None) == 0          # nothing to do
    assert d(-1, good, good, good, 4, 128, 64, None, None) == -2
    assert d(2, None, good, good, 4, 128, 64, None, None) == -1
    assert d(2, good, ps(FAKE, None), good, 4, 128, 64, None, None) == -1
    assert d(2, good, good, good, 4, 100, 64, None, None) == -2
    assert d(2, good, good, good, 4, 128, 96, None, None) == -3
    assert d(2, good, good, ps(FAKE, FAKE + 8), 4, 128, 64, None, None) == -4
    assert d(2, good, ps(FAKE + 1, FAKE), good, 4, 128, 64, None, None) == -4
    assert d(2, good, good, good, 4, 128, 64, FAKE + 1, None) == -4


def test_two_bit_argument_errors():
    import ctypes
    lib = _lib()
    q, u, g = lib.tq_quantize_pack2, lib.tq_unpack2, lib.tq_gemv2
    assert q(None, 4, 128, 64, FAKE, FAKE, None, None) == -1
    assert q(FAKE, 4, 128, 64, None, FAKE, None, None) == -1
    assert q(FAKE, 4, 128, 64, FAKE, None, None, None) == -1
    assert q(FAKE, 4, 130, 64, FAKE, FAKE, None, None) == -2
    assert q(FAKE, 4, 128, 32, FAKE, FAKE, None, None) == -3
    assert q(FAKE + 8, 4, 128, 64, FAKE, FAKE, None, None) == -4
    assert q(FAKE, 4, 128, 64, FAKE + 1, FAKE, None, None) == -4
    assert u(None, 4, 128, 64, FAKE, None, None) == -1
    assert u(FAKE, 0, 128, 64, FAKE, None, None) == -2
    assert u(FAKE + 2, 4, 128, 64, FAKE, None, None) == -4
    assert u(FAKE, 4, 128, 64, FAKE + 8, None, None) == -4
    assert g(None, FAKE, FAKE, 4, 128, 64, FAKE, None, None) == -1
    assert g(FAKE, FAKE, FAKE, 1 << 20, 8192, 64, FAKE, None, None) == -2   # N*K/4 >= 2^31
    assert g(FAKE, FAKE, FAKE, 4, 128, 96, FAKE, None, None) == -3
    assert g(FAKE, FAKE + 4, FAKE, 4, 128, 64, FAKE, None, None) == -4
    assert g(FAKE + 8, FAKE, FAKE, 4, 128, 64, FAKE, None, None) == -4
    assert g(FAKE, FAKE, FAKE, 4, 128, 64, FAKE + 2, None, None) == -4
    arr = ctypes.c_void_p * 2
    good = arr(FAKE, FAKE + 4096)
    b = lib.tq_gemv2_batched
    assert b(0, None, None, None, None, 4, 128, 64, None, None) == 0
    assert b(-1, good, good, good, good, 4, 128, 64, None, None) == -2
    assert b(2, good, None, good, good, 4, 128, 64, None, None) == -1
    assert b(2, good, good, arr(FAKE, None), good, 4, 128, 64, None, None) == -1
    assert b(2, good, arr(FAKE, FAKE + 8), good, good, 4, 128, 64, None, None) == -4
    assert b(2, good, good, good, good, 4, 128, 64, FAKE + 1, None) == -4
    qb = lib.tq_quantize_pack2_batched
    assert qb(0, None, 4, 128, 64, None, None, None, None) == 0
    assert qb(-1, good, 4, 128, 64, good, good, None, None) == -2
    assert qb(2, good, 4, 128, 64, None, good, None, None) == -1
    assert qb(2, good, 4, 130, 64, good, good, None, None) == -2
    assert qb(2, good, 4, 128, 32, good, good, None, None) == -3
    assert qb(2, arr(FAKE, FAKE + 8), 4, 128, 64, good, good, None, None) == -4
    assert qb(2, good, 4, 128, 64, arr(FAKE, FAKE + 1), good, None, None) == -4
    gr = lib.tq_gemv2_grouped
    i64s = ctypes.c_int64 * 2
    ns, ks = i64s(4, 8), i64s(128, 256)
    assert gr(0, None, None, None, None, None, None, 64, None, None) == 0
    assert gr(-1, good, good, good, good, ns, ks, 64, None, None) == -2
    assert gr(2, good, good, good, good, None, ks, 64, None, None) == -1
    assert gr(2, good, good, good, good, i64s(4, 1 << 20), i64s(128, 8192), 64, None, None) == -2
    assert gr(2, good, good, good, good, ns, i64s(128, 200), 64, None, None) == -2
    assert gr(2, good, good, good, good, ns, ks, 96, None, None) == -3
    assert gr(2, good, arr(FAKE, FAKE + 8), good, good, ns, ks, 64, None, None) == -4
    assert gr(2, good, good, good, arr(FAKE, None), ns, ks, 64, None, None) == -1


def test_w4a16_argument_errors():
    import ctypes
    lib = _lib()
    g = lib.tq_w4a16_gemv
    assert g(None, FAKE, FAKE, FAKE, 4, 128, 128, FAKE, None) == -1
    assert g(FAKE, FAKE, FAKE, None, 4, 128, 128, FAKE, None) == -1
    assert g(FAKE, FAKE, FAKE, FAKE, 1 << 20, 8192, 128, FAKE, None) == -2  # codes >= 2^31 B
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 200, 100, FAKE, None) == -3
    assert g(FAKE + 8, FAKE, FAKE, FAKE, 4, 128, 128, FAKE, None) == -4
    assert g(FAKE, FAKE + 4, FAKE, FAKE, 4, 128, 128, FAKE, None) == -4
    assert g(FAKE, FAKE, FAKE, FAKE + 1, 4, 128, 128, FAKE, None) == -4
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 128, 128, FAKE + 1, None) == -4
    arr = ctypes.c_void_p * 2
    good = arr(FAKE, FAKE + 4096)
    b = lib.tq_w4a16_gemv_batched
    assert b(0, None, None, None, None, None, 4, 128, 128, None) == 0
    assert b(-1, good, good, good, good, good, 4, 128, 128, None) == -2
    assert b(2, good, good, good, None, good, 4, 128, 128, None) == -1
    assert b(2, good, good, good, arr(FAKE, None), good, 4, 128, 128, None) == -1
    assert b(2, good, arr(FAKE, FAKE + 8), good, good, good, 4, 128, 128, None) == -4
    gr = lib.tq_w4a16_gemv_grouped
    i64s = ctypes.c_int64 * 2
    ns, ks = i64s(4, 8), i64s(128, 256)
    assert gr(0, None, None, None, None, None, None, None, 128, None) == 0
    assert gr(-1, good, good, good, good, good, ns, ks, 128, None) == -2
    assert gr(2, good, good, good, good, good, ns, None, 128, None) == -1
    assert gr(2, good, good, good, good, good, i64s(4, 1 << 20), i64s(128, 8192), 128,
              None) == -2
    assert gr(2, good, good, good, good, good, ns, ks, 100, None) == -3
    assert gr(2, good, arr(FAKE, FAKE + 8), good, good, good, ns, ks, 128, None) == -4
    assert gr(2, good, good, good, arr(FAKE, None), good, ns, ks, 128, None) == -1


def test_w4a16_gemm_argument_errors():
    lib = _lib()
    f = lib.tq_w4a16_gemm
    assert f(None, FAKE, FAKE, FAKE, 2, 4, 128, 128, FAKE, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 128, None, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 4, 128, 128, FAKE, None) == -2     # M < 1
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 0, 128, 128, FAKE, None) == -2     # N < 1
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 4, 192, 128, FAKE, None) == -2     # K % G
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 32, FAKE, None) == -3      # G
    assert f(FAKE, FAKE, FAKE, FAKE, 1 << 17, 4, 8192, 128, FAKE, None) == -2  # x >= 2^31 B
    assert f(FAKE, FAKE, FAKE, FAKE, 5000000, 4, 128, 128, FAKE, None) == -2  # grid rows
    assert f(FAKE + 8, FAKE, FAKE, FAKE, 2, 4, 128, 128, FAKE, None) == -4
    assert f(FAKE, FAKE + 2, FAKE, FAKE, 2, 4, 128, 128, FAKE, None) == -4
    assert f(FAKE, FAKE, FAKE + 1, FAKE, 2, 4, 128, 128, FAKE, None) == -4
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 128, FAKE + 1, None) == -4


def test_w4a16_gemm_batched_argument_errors():
    lib = _lib()
    f = lib.tq_w4a16_gemm_batched
    P = ctypes.c_void_p
    one = (P * 1)(FAKE)
    null = (P * 1)(None)
    odd = (P * 1)(FAKE + 1)
    assert f(0, None, None, None, None, 2, 4, 128, 128, None, None) == 0   # nothing to do
    assert f(-1, one, one, one, one, 2, 4, 128, 128, one, None) == -2
    assert f(1, None, one, one, one, 2, 4, 128, 128, one, None) == -1
    assert f(1, one, one, one, one, 2, 4, 128, 128, null, None) == -1
    assert f(1, one, one, one, one, 0, 4, 128, 128, one, None) == -2       # M < 1
    assert f(1, one, one, one, one, 2, 4, 192, 128, one, None) == -2       # K % G
    assert f(1, one, one, one, one, 2, 4, 128, 32, one, None) == -3        # G
    assert f(1, one, one, one, one, 2, 4, 128, 128, odd, None) == -4       # y alignment
    assert f(1, odd, one, one, one, 2, 4, 128, 128, one, None) == -4       # x alignment


def test_gemm2_argument_errors():
    lib = _lib()
    f = lib.tq_gemm2
    assert f(None, FAKE, FAKE, 2, 4, 128, 128, FAKE, None, None) == -1
    assert f(FAKE, FAKE, FAKE, 2, 4, 128, 128, None, None, None) == -1
    assert f(FAKE, FAKE, FAKE, 0, 4, 128, 128, FAKE, None, None) == -2     # M < 1
    assert f(FAKE, FAKE, FAKE, 2, 0, 128, 128, FAKE, None, None) == -2     # N < 1
    assert f(FAKE, FAKE, FAKE, 2, 4, 192, 128, FAKE, None, None) == -2     # K % G
    assert f(FAKE, FAKE, FAKE, 2, 4, 128, 32, FAKE, None, None) == -3      # G
    assert f(FAKE, FAKE, FAKE, 1 << 17, 4, 8192, 128, FAKE, None, None) == -2  # x >= 2^31 B
    assert f(FAKE + 8, FAKE, FAKE, 2, 4, 128, 128, FAKE, None, None) == -4
    assert f(FAKE, FAKE + 1, FAKE, 2, 4, 128, 128, FAKE, None, None) == -4
    assert f(FAKE, FAKE, FAKE + 1, 2, 4, 128, 128, FAKE, None, None) == -4
    assert f(FAKE, FAKE, FAKE, 2, 4, 128, 128, FAKE + 2, None, None) == -4
    assert f(FAKE, FAKE, FAKE, 2, 4, 128, 128, FAKE, FAKE + 2, None) == -4  # status
    g = lib.tq_gemm2_batched
    P = ctypes.c_void_p
    one = (P * 1)(FAKE)
    assert g(0, None, None, None, None, 2, 4, 128, 128, None, None) == 0
    assert g(-1, one, one, one, one, 2, 4, 128, 128, None, None) == -2
    assert g(1, None, one, one, one, 2, 4, 128, 128, None, None) == -1
    assert g(1, one, one, one, (P * 1)(None), 2, 4, 128, 128, None, None) == -1


def test_fake_quantize_f32_argument_errors():
    lib = _lib()
    f = lib.tq_fake_quantize_f32
    assert f(None, 4, 128, 64, FAKE, None, None, None) == -1
    assert f(FAKE, 4, 128, 64, None, None, None, None) == -1
    assert f(FAKE, 0, 128, 64, FAKE, None, None, None) == -2
    assert f(FAKE, 4, 100, 64, FAKE, None, None, None) == -2
    assert f(FAKE, 4, 128, 32, FAKE, None, None, None) == -3
    assert f(FAKE + 8, 4, 128, 64, FAKE, None, None, None) == -4
    assert f(FAKE, 4, 128, 64, FAKE + 8, None, None, None) == -4
    assert f(FAKE, 4, 128, 64, FAKE, FAKE + 1, None, None) == -4
    assert f(FAKE, 4, 128, 64, FAKE, None, FAKE + 2, None) == -4
    g = lib.tq_fake_quantize_f32_batched
    P = ctypes.c_void_p
    one = (P * 1)(FAKE)
    assert g(0, None, 4, 128, 64, None, None, None, None) == 0
    assert g(-1, one, 4, 128, 64, one, None, None, None) == -2
    assert g(1, one, 4, 128, 64, (P * 1)(None), None, None, None) == -1


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "ternary_weight_only_amd")
    for dirpath, _, files in os.walk(pkg):
        for fname in files:
            if fname.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fname)).read()
                assert "import oracle" not in text and "from oracle" not in text, fname
                assert "tq_oracle" not in text and "liboracle" not in text, fname
