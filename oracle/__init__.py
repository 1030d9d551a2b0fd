"""CPU oracle for ternary quantize/pack/unpack and the packed-ternary matmul.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``ternary_weight_only_amd``) never imports it, and this package imports
nothing from the product path.

The arithmetic lives in ``tq_oracle.c`` (plain scalar C, fp64 for the matmul),
compiled with the host C compiler into ``liboracle.so`` next to this file.
Each function below only marshals numpy arrays to that library.

Sources: precisit "pack-unpack-run" README (codec.py description: absmean
scale rounded to fp16, nearest-even ternary codes, five base-3 digits per
byte, byte-aligned groups with zero-trit padding, bytes 243..255 invalid;
scale-rule and payload-rate paragraphs) and tiny-llm "Week 2 Day 3: Quantize
the Model" ("Mathematical Formulation", "Computation Flow").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Status bits (same values as the library's device status bits).
NONFINITE = 1
SCALE_OVERFLOW = 2
INVALID_BYTE = 4
BAD_PADDING = 8

ERR_NULL = -1
ERR_SHAPE = -2

_lib = None


def build(force: bool = False) -> str:
    """Compile tq_oracle.c into liboracle.so with gcc; returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC",
                               "-pthread", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_packed_row_bytes.argtypes = [i64, i64]
        lib.oracle_packed_row_bytes.restype = i64
        lib.oracle_quantize_pack.argtypes = [p, i64, i64, i64, p, p, p]
        lib.oracle_quantize_pack.restype = ctypes.c_int
        lib.oracle_unpack.argtypes = [p, i64, i64, i64, p, p]
        lib.oracle_unpack.restype = ctypes.c_int
        lib.oracle_matmul.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p]
        lib.oracle_matmul.restype = ctypes.c_int
        lib.oracle_dequantize.argtypes = [p, p, i64, i64, i64, p, p]
        lib.oracle_dequantize.restype = ctypes.c_int
        lib.oracle_fake_quantize.argtypes = [p, i64, i64, i64, p, p, p]
        lib.oracle_fake_quantize.restype = ctypes.c_int
        lib.oracle_fake_quantize_f32.argtypes = [p, i64, i64, i64, p, p, p]
        lib.oracle_fake_quantize_f32.restype = ctypes.c_int
        lib.oracle_quantize_pack2.argtypes = [p, i64, i64, i64, p, p, p]
        lib.oracle_quantize_pack2.restype = ctypes.c_int
        lib.oracle_unpack2.argtypes = [p, i64, i64, i64, p, p]
        lib.oracle_unpack2.restype = ctypes.c_int
        lib.oracle_matmul2.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p]
        lib.oracle_matmul2.restype = ctypes.c_int
        lib.oracle_w4_unpack.argtypes = [p, i64, i64, p]
        lib.oracle_w4_unpack.restype = ctypes.c_int
        lib.oracle_w4a16_dequantize.argtypes = [p, p, p, i64, i64, i64, p]
        lib.oracle_w4a16_dequantize.restype = ctypes.c_int
        lib.oracle_w4a16_matmul.argtypes = [p, p, p, p, i64, i64, i64, i64, p, p]
        lib.oracle_w4a16_matmul.restype = ctypes.c_int
        i32 = ctypes.c_int
        lib.oracle_quantize_pack_mt.argtypes = [p, i64, i64, i64, p, p, p, i32]
        lib.oracle_quantize_pack_mt.restype = i32
        for f in (lib.oracle_matmul_mt, lib.oracle_matmul2_mt):
            f.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p, i32]
            f.restype = i32
        lib.oracle_w4a16_matmul_mt.argtypes = [p, p, p, p, i64, i64, i64, i64, p, p, i32]
        lib.oracle_w4a16_matmul_mt.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    """Threads the row-partitioned entry points use when none is given: the
    host's cores, at most 16.  Results do not depend on the count."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _threads(threads) -> int:
    return default_threads() if threads is None else max(1, int(threads))


class OracleError(RuntimeError):
    pass


def packed_row_bytes(K: int, G: int) -> int:
    """Packed bytes per row: (K/G) * ceil(G/5); 0 for invalid arguments."""
    return int(_load().oracle_packed_row_bytes(K, G))


def quantize_pack(w_bits: np.ndarray, G: int, threads=None):
    """w_bits: uint16 [N,K] bf16 bit patterns.

    Returns (packed uint8 [N, (K/G)*ceil(G/5)], scales uint16 [N, K/G] fp16 bits,
    status bits int).  The rows are split over `threads` host threads (default:
    the host's cores, at most 16); the result does not depend on the split.
    """
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N,K]")
    N, K = w.shape
    rb = packed_row_bytes(K, G)
    if rb == 0:
        raise OracleError("invalid shape K=%d G=%d" % (K, G))
    packed = np.empty((N, rb), np.uint8)
    scales = np.empty((N, K // G), np.uint16)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_quantize_pack_mt(_ptr(w), N, K, G, _ptr(packed), _ptr(scales), _ptr(st),
                                         _threads(threads))
    if rc:
        raise OracleError("oracle_quantize_pack rc=%d" % rc)
    return packed, scales, int(st[0])


def unpack(packed: np.ndarray, N: int, K: int, G: int):
    """Returns (codes int8 [N,K] in {-1,0,1}, status bits int)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    rb = packed_row_bytes(K, G)
    if rb == 0 or p.size != N * rb:
        raise OracleError("packed has %d bytes, expected %d" % (p.size, N * rb))
    codes = np.empty((N, K), np.int8)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_unpack(_ptr(p), N, K, G, _ptr(codes), _ptr(st))
    if rc:
        raise OracleError("oracle_unpack rc=%d" % rc)
    return codes, int(st[0])


def dequantize(packed: np.ndarray, scales: np.ndarray, N: int, K: int, G: int):
    """Decode to bf16: w_hat[n,k] = bf16_RNE(c[n,k] * s[n,k/G]).

    Returns (w_hat uint16 [N,K] bf16 bits, status bits int)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    rb = packed_row_bytes(K, G)
    if rb == 0 or p.size != N * rb or s.size != N * (K // G):
        raise OracleError("bad packed/scales sizes")
    out = np.empty((N, K), np.uint16)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_dequantize(_ptr(p), _ptr(s), N, K, G, _ptr(out), _ptr(st))
    if rc:
        raise OracleError("oracle_dequantize rc=%d" % rc)
    return out, int(st[0])


def fake_quantize(w_bits: np.ndarray, G: int):
    """QAT forward: w_hat = bf16_RNE(c * s) from bf16 weights.

    Returns (w_hat uint16 [N,K] bf16 bits, scales uint16 [N,K/G] fp16 bits,
    status bits int)."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise OracleError("w must be 2-D")
    N, K = w.shape
    if G < 1 or K % G:
        raise OracleError("K % G != 0")
    out = np.empty((N, K), np.uint16)
    sc = np.empty((N, K // G), np.uint16)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_fake_quantize(_ptr(w), N, K, G, _ptr(out), _ptr(sc), _ptr(st))
    if rc:
        raise OracleError("oracle_fake_quantize rc=%d" % rc)
    return out, sc, int(st[0])


def fake_quantize_f32(w: np.ndarray, G: int):
    """QAT forward from fp32 latent weights: w_hat = c * s in fp32 (exact).

    w: float32 [N,K] (or its uint32 bits).  Returns (w_hat float32 [N,K],
    scales uint16 [N,K/G] fp16 bits, status bits int)."""
    wb = np.ascontiguousarray(w).view(np.uint32) if np.asarray(w).dtype == np.float32 \
        else np.ascontiguousarray(w, dtype=np.uint32)
    if wb.ndim != 2:
        raise OracleError("w must be 2-D")
    N, K = wb.shape
    if G < 1 or K % G:
        raise OracleError("K % G != 0")
    out = np.empty((N, K), np.uint32)
    sc = np.empty((N, K // G), np.uint16)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_fake_quantize_f32(_ptr(wb), N, K, G, _ptr(out), _ptr(sc), _ptr(st))
    if rc:
        raise OracleError("oracle_fake_quantize_f32 rc=%d" % rc)
    return out.view(np.float32), sc, int(st[0])


def quantize_pack2(w_bits: np.ndarray, G: int):
    """2-bit format: w_bits uint16 [N,K] bf16 -> (packed uint8 [N, K/4], scales
    uint16 [N, K/G] fp16 bits, status bits int)."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N,K]")
    N, K = w.shape
    if G < 4 or G % 4 or K % G:
        raise OracleError("invalid shape K=%d G=%d" % (K, G))
    packed = np.empty((N, K // 4), np.uint8)
    scales = np.empty((N, K // G), np.uint16)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_quantize_pack2(_ptr(w), N, K, G, _ptr(packed), _ptr(scales), _ptr(st))
    if rc:
        raise OracleError("oracle_quantize_pack2 rc=%d" % rc)
    return packed, scales, int(st[0])


def unpack2(packed: np.ndarray, N: int, K: int, G: int):
    """2-bit packed [N, K/4] -> (codes int8 [N,K], status bits int)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    if p.size != N * K // 4:
        raise OracleError("bad packed size")
    codes = np.empty((N, K), np.int8)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_unpack2(_ptr(p), N, K, G, _ptr(codes), _ptr(st))
    if rc:
        raise OracleError("oracle_unpack2 rc=%d" % rc)
    return codes, int(st[0])


def matmul2(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, N: int, K: int, G: int,
            threads=None):
    """As matmul, over the 2-bit format."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M,K]")
    M = x.shape[0]
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    if p.size != N * K // 4 or s.size != N * (K // G):
        raise OracleError("bad packed/scales sizes")
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_matmul2_mt(_ptr(x), _ptr(p), _ptr(s), M, N, K, G, _ptr(y), _ptr(bound),
                                   _ptr(st), _threads(threads))
    if rc:
        raise OracleError("oracle_matmul2 rc=%d" % rc)
    return y, bound, int(st[0])


def matmul(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, N: int, K: int, G: int,
           threads=None):
    """y[m,n] = sum_k x[m,k] c[n,k] s[n,k/G] in fp64.

    x_bits: uint16 [M,K] bf16 bits.  Returns (y float64 [M,N],
    bound float64 [M,N] = sum_k |x c s|, status bits int).  Weight rows are
    split over `threads` host threads; each output's sum runs in k order
    whatever the split.
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M,K]")
    M = x.shape[0]
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    rb = packed_row_bytes(K, G)
    if rb == 0 or p.size != N * rb or s.size != N * (K // G):
        raise OracleError("bad packed/scales sizes")
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    st = np.zeros(1, np.int32)
    rc = _load().oracle_matmul_mt(_ptr(x), _ptr(p), _ptr(s), M, N, K, G, _ptr(y), _ptr(bound),
                                  _ptr(st), _threads(threads))
    if rc:
        raise OracleError("oracle_matmul rc=%d" % rc)
    return y, bound, int(st[0])


# W4A16 (tiny-llm "Week 2 Day 3: Quantize the Model": "Group-Wise Affine
# Quantization", "Reconstruct a Stored Group", "Packed Storage Layout",
# "Computation Flow").  packed: uint32 [N, K/8], weight 8p + i in bits
# 4i..4i+3 of word p; scales, biases: bf16 bits [N, K/G]; w_hat = q*s + b.

def w4_unpack(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """uint32 [N, K/8] -> unsigned codes uint8 [N, K]."""
    p = np.ascontiguousarray(packed, dtype=np.uint32)
    if p.size * 8 != N * K:
        raise OracleError("bad packed size")
    codes = np.empty((N, K), np.uint8)
    rc = _load().oracle_w4_unpack(_ptr(p), N, K, _ptr(codes))
    if rc:
        raise OracleError("oracle_w4_unpack rc=%d" % rc)
    return codes


def w4a16_dequantize(packed, scales, biases, N: int, K: int, G: int) -> np.ndarray:
    """-> w_hat float64 [N, K] = q*s + b."""
    p = np.ascontiguousarray(packed, dtype=np.uint32)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    b = np.ascontiguousarray(biases, dtype=np.uint16)
    if p.size * 8 != N * K or G <= 0 or s.size != N * (K // G) or b.size != s.size:
        raise OracleError("bad packed/scales/biases sizes")
    w = np.empty((N, K), np.float64)
    rc = _load().oracle_w4a16_dequantize(_ptr(p), _ptr(s), _ptr(b), N, K, G, _ptr(w))
    if rc:
        raise OracleError("oracle_w4a16_dequantize rc=%d" % rc)
    return w


def w4a16_matmul(x_bits, packed, scales, biases, N: int, K: int, G: int, threads=None):
    """x bf16 bits [M,K] -> (y float64 [M,N], bound float64 [M,N] =
    sum_k |x| (|q s| + |b|))."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M,K]")
    M = x.shape[0]
    p = np.ascontiguousarray(packed, dtype=np.uint32)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    b = np.ascontiguousarray(biases, dtype=np.uint16)
    if p.size * 8 != N * K or G <= 0 or s.size != N * (K // G) or b.size != s.size:
        raise OracleError("bad packed/scales/biases sizes")
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    rc = _load().oracle_w4a16_matmul_mt(_ptr(x), _ptr(p), _ptr(s), _ptr(b), M, N, K, G, _ptr(y),
                                        _ptr(bound), _threads(threads))
    if rc:
        raise OracleError("oracle_w4a16_matmul rc=%d" % rc)
    return y, bound
