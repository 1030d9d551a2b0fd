"""ctypes binding of libtq.so (C ABI: include/tq.h).

Argument marshalling only: shape/dtype/device/contiguity checks on torch
tensors, output allocation, raw device pointers and the current HIP stream.
Every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

DEV_NONFINITE = 1
DEV_SCALE_OVERFLOW = 2
DEV_INVALID_BYTE = 4
DEV_BAD_PADDING = 8

# Every symbol include/tq.h declares.
SYMBOLS = ("tq_status_string", "tq_packed_bytes", "tq_quantize_pack", "tq_quantize_pack_batched",
           "tq_fake_quantize", "tq_fake_quantize_batched", "tq_unpack", "tq_unpack_batched",
           "tq_dequantize", "tq_dequantize_batched", "tq_quantize_pack2", "tq_quantize_pack2_batched", "tq_unpack2",
           "tq_gemv2", "tq_gemv2_batched", "tq_gemv2_grouped", "tq_w4a16_gemv", "tq_w4a16_gemv_batched",
           "tq_w4a16_gemv_grouped", "tq_gemv", "tq_gemv_batched", "tq_gemv_grouped", "tq_gemm", "tq_gemm_batched")

_lib = None


class TQError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libtq.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TQError("libtq.so is not built (%s); run "
                          "`python -m ternary_weight_only_amd.build`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        l.tq_status_string.argtypes = [i32]
        l.tq_status_string.restype = ctypes.c_char_p
        l.tq_packed_bytes.argtypes = [i64, i64, i32]
        l.tq_packed_bytes.restype = i64
        l.tq_quantize_pack.argtypes = [p, i64, i64, i32, p, p, p, p]
        l.tq_quantize_pack.restype = i32
        l.tq_fake_quantize.argtypes = [p, i64, i64, i32, p, p, p, p]
        l.tq_fake_quantize.restype = i32
        for f in (l.tq_quantize_pack_batched, l.tq_fake_quantize_batched):
            f.argtypes = [i32, p, i64, i64, i32, p, p, p, p]
            f.restype = i32
        l.tq_quantize_pack2.argtypes = [p, i64, i64, i32, p, p, p, p]
        l.tq_quantize_pack2.restype = i32
        l.tq_quantize_pack2_batched.argtypes = [i32, p, i64, i64, i32, p, p, p, p]
        l.tq_quantize_pack2_batched.restype = i32
        l.tq_unpack2.argtypes = [p, i64, i64, i32, p, p, p]
        l.tq_unpack2.restype = i32
        l.tq_gemv2.argtypes = [p, p, p, i64, i64, i32, p, p, p]
        l.tq_gemv2.restype = i32
        l.tq_gemv2_batched.argtypes = [i32, p, p, p, p, i64, i64, i32, p, p]
        l.tq_gemv2_batched.restype = i32
        l.tq_gemv2_grouped.argtypes = [i32, p, p, p, p, p, p, i32, p, p]
        l.tq_gemv2_grouped.restype = i32
        l.tq_w4a16_gemv.argtypes = [p, p, p, p, i64, i64, i32, p, p]
        l.tq_w4a16_gemv.restype = i32
        l.tq_w4a16_gemv_batched.argtypes = [i32, p, p, p, p, p, i64, i64, i32, p]
        l.tq_w4a16_gemv_batched.restype = i32
        l.tq_w4a16_gemv_grouped.argtypes = [i32, p, p, p, p, p, p, p, i32, p]
        l.tq_w4a16_gemv_grouped.restype = i32
        l.tq_unpack_batched.argtypes = [i32, p, i64, i64, i32, p, p, p]
        l.tq_unpack_batched.restype = i32
        l.tq_unpack.argtypes = [p, i64, i64, i32, p, p, p]
        l.tq_unpack.restype = i32
        l.tq_dequantize.argtypes = [p, p, i64, i64, i32, p, p, p]
        l.tq_dequantize.restype = i32
        l.tq_dequantize_batched.argtypes = [i32, p, p, p, i64, i64, i32, p, p]
        l.tq_dequantize_batched.restype = i32
        for f in (l.tq_gemv, l.tq_gemm):
            f.argtypes = [p, p, p, i64, i64, i64, i32, p, p, p]
            f.restype = i32
        for f in (l.tq_gemv_batched, l.tq_gemm_batched):
            f.argtypes = [i32, p, p, p, p, i64, i64, i64, i32, p, p]
            f.restype = i32
        l.tq_gemv_grouped.argtypes = [i32, p, p, p, p, p, p, i32, p, p]
        l.tq_gemv_grouped.restype = i32
        _lib = l
    return _lib


def _rc(rc: int, what: str):
    if rc != 0:
        raise TQError("%s failed: %s" % (what, lib().tq_status_string(rc).decode()))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TQError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise TQError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.dim() != ndim or not t.is_contiguous():
        raise TQError("%s must be a contiguous %d-D tensor" % (name, ndim))


def _st(status):
    return 0 if status is None else status.data_ptr()


def packed_bytes(N: int, K: int, G: int) -> int:
    return int(lib().tq_packed_bytes(N, K, G))


def new_status(device=None) -> torch.Tensor:
    """A zeroed device int32 status word."""
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


def check(status: torch.Tensor) -> int:
    """Synchronize-free read of a status word (forces a device->host copy)."""
    return int(status.item())


def quantize_pack(w: torch.Tensor, G: int, status=None, out=None):
    """w: [N,K] bf16 -> (packed uint8 [N, (K/G)*ceil(G/5)], scales fp16 [N, K/G])."""
    _dev(w, "w", (torch.bfloat16, torch.int16), 2)
    N, K = w.shape
    rb = (K // G) * ((G + 4) // 5) if G > 0 and K % G == 0 else 0
    if out is None:
        packed = torch.empty((N, max(rb, 1)), dtype=torch.uint8, device=w.device)
        scales = torch.empty((N, max(K // G, 1)), dtype=torch.float16, device=w.device)
    else:
        packed, scales = out
    _rc(lib().tq_quantize_pack(w.data_ptr(), N, K, G, packed.data_ptr(), scales.data_ptr(),
                               _st(status), _stream()), "tq_quantize_pack")
    return packed, scales


def fake_quantize(w: torch.Tensor, G: int, status=None, out=None, scales_out=None):
    """QAT forward: w [N,K] bf16 -> w_hat bf16 [N,K] = bf16(c * s).

    scales_out, if given, is an fp16 [N, K/G] tensor that receives the
    scales.  Use FakeQuantize.apply for the straight-through gradient."""
    _dev(w, "w", (torch.bfloat16, torch.int16), 2)
    N, K = w.shape
    w_hat = torch.empty((N, K), dtype=torch.bfloat16, device=w.device) if out is None else out
    sp = 0
    if scales_out is not None:
        _dev(scales_out, "scales_out", (torch.float16, torch.int16), scales_out.dim())
        if G <= 0 or scales_out.numel() != N * (K // G):
            raise TQError("scales_out has %d entries, expected %d" % (scales_out.numel(),
                                                                    N * (K // max(G, 1))))
        sp = scales_out.data_ptr()
    _rc(lib().tq_fake_quantize(w.data_ptr(), N, K, G, w_hat.data_ptr(), sp, _st(status),
                               _stream()), "tq_fake_quantize")
    return w_hat


def _ptrs(ts):
    return (ctypes.c_void_p * max(len(ts), 1))(*[t.data_ptr() for t in ts])


def _same_shape(ws, name):
    for w in ws:
        _dev(w, name, (torch.bfloat16, torch.int16), 2)
    shapes = {tuple(w.shape) for w in ws}
    if len(shapes) > 1:
        raise TQError("%s: matrices of different shapes %s" % (name, sorted(shapes)))
    return shapes.pop() if shapes else (0, 0)


def quantize_pack_batched(ws, G: int, status=None):
    """Same-shaped bf16 matrices -> list of (packed, scales), one launch per 64."""
    N, K = _same_shape(ws, "w")
    if not ws:
        return []
    rb = (K // G) * ((G + 4) // 5) if G > 0 and K % G == 0 else 0
    dev = ws[0].device
    pk = [torch.empty((N, max(rb, 1)), dtype=torch.uint8, device=dev) for _ in ws]
    sc = [torch.empty((N, max(K // max(G, 1), 1)), dtype=torch.float16, device=dev) for _ in ws]
    _rc(lib().tq_quantize_pack_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(pk), _ptrs(sc),
                                       _st(status), _stream()), "tq_quantize_pack_batched")
    return list(zip(pk, sc))


def fake_quantize_batched(ws, G: int, status=None, with_scales: bool = False):
    """Same-shaped bf16 matrices -> list of bf16 w_hat (and, with_scales, of
    (w_hat, scales)), one launch per 64."""
    N, K = _same_shape(ws, "w")
    if not ws:
        return []
    dev = ws[0].device
    wh = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in ws]
    sc = [torch.empty((N, max(K // max(G, 1), 1)), dtype=torch.float16, device=dev)
          for _ in ws] if with_scales else None
    _rc(lib().tq_fake_quantize_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(wh),
                                       _ptrs(sc) if with_scales else None, _st(status),
                                       _stream()), "tq_fake_quantize_batched")
    return list(zip(wh, sc)) if with_scales else wh


def unpack_batched(packeds, N: int, K: int, G: int, status=None):
    """Same-shaped packed matrices -> list of int8 codes [N,K], one launch per 64."""
    for p in packeds:
        _dev(p, "packed", (torch.uint8,), p.dim())
        if p.numel() != packed_bytes(N, K, G):
            raise TQError("packed has %d bytes, expected %d" % (p.numel(), packed_bytes(N, K, G)))
    if not packeds:
        return []
    codes = [torch.empty((N, K), dtype=torch.int8, device=p.device) for p in packeds]
    _rc(lib().tq_unpack_batched(len(packeds), _ptrs(packeds), N, K, G, _ptrs(codes), _st(status),
                                _stream()), "tq_unpack_batched")
    return codes


def quantize_pack2(w: torch.Tensor, G: int, status=None):
    """2-bit format: w [N,K] bf16 -> (packed2 uint8 [N, K/4], scales fp16 [N, K/G])."""
    _dev(w, "w", (torch.bfloat16, torch.int16), 2)
    N, K = w.shape
    packed = torch.empty((N, max(K // 4, 1)), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, max(K // max(G, 1), 1)), dtype=torch.float16, device=w.device)
    _rc(lib().tq_quantize_pack2(w.data_ptr(), N, K, G, packed.data_ptr(), scales.data_ptr(),
                                _st(status), _stream()), "tq_quantize_pack2")
    return packed, scales


def quantize_pack2_batched(ws, G: int, status=None):
    """2-bit format, same-shaped bf16 matrices -> list of (packed2, scales),
    one launch per 64."""
    N, K = _same_shape(ws, "w")
    if not ws:
        return []
    dev = ws[0].device
    pk = [torch.empty((N, max(K // 4, 1)), dtype=torch.uint8, device=dev) for _ in ws]
    sc = [torch.empty((N, max(K // max(G, 1), 1)), dtype=torch.float16, device=dev) for _ in ws]
    _rc(lib().tq_quantize_pack2_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(pk), _ptrs(sc),
                                        _st(status), _stream()), "tq_quantize_pack2_batched")
    return list(zip(pk, sc))


def unpack2(packed: torch.Tensor, N: int, K: int, G: int, status=None):
    """2-bit packed [N, K/4] -> codes int8 [N,K]."""
    _dev(packed, "packed", (torch.uint8,), packed.dim())
    if packed.numel() * 4 != N * K:
        raise TQError("packed has %d bytes, expected %d" % (packed.numel(), N * K // 4))
    codes = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _rc(lib().tq_unpack2(packed.data_ptr(), N, K, G, codes.data_ptr(), _st(status), _stream()),
        "tq_unpack2")
    return codes


def gemv2(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, N: int, K: int, G: int,
          status=None, out=None):
    """2-bit format, M = 1: x [1,K] bf16 -> y fp32 [1,N]."""
    _dev(x, "x", (torch.bfloat16, torch.int16), 2)
    _dev(packed, "packed", (torch.uint8,), packed.dim())
    _dev(scales, "scales", (torch.float16, torch.int16), scales.dim())
    if tuple(x.shape) != (1, K) or packed.numel() * 4 != N * K or scales.numel() != N * (K // G):
        raise TQError("gemv2: shapes do not match N=%d K=%d G=%d" % (N, K, G))
    y = torch.empty((1, N), dtype=torch.float32, device=x.device) if out is None else out
    _rc(lib().tq_gemv2(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), N, K, G, y.data_ptr(),
                       _st(status), _stream()), "tq_gemv2")
    return y


def gemv2_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """2-bit format, M = 1, same-shaped problems: list of y fp32 [1,N], one launch per 64."""
    n = len(xs)
    if len(packeds) != n or len(scales_list) != n:
        raise TQError("xs, packeds and scales differ in length")
    for x, pk, sc in zip(xs, packeds, scales_list):
        _dev(x, "x", (torch.bfloat16, torch.int16), 2)
        _dev(pk, "packed", (torch.uint8,), pk.dim())
        _dev(sc, "scales", (torch.float16, torch.int16), sc.dim())
        if (tuple(x.shape) != (1, K) or pk.numel() * 4 != N * K or G <= 0
                or sc.numel() != N * (K // G)):
            raise TQError("gemv2_batched: shapes do not match N=%d K=%d G=%d" % (N, K, G))
    if outs is None:
        outs = [torch.empty((1, N), dtype=torch.float32, device=x.device) for x in xs]
    _rc(lib().tq_gemv2_batched(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(outs),
                               N, K, G, _st(status), _stream()), "tq_gemv2_batched")
    return outs


def _w4_check(x, packed, scales, biases, N, K, G):
    _dev(x, "x", (torch.bfloat16, torch.int16), 2)
    _dev(packed, "packed", (torch.int32, torch.uint32), packed.dim())
    _dev(scales, "scales", (torch.bfloat16, torch.int16), scales.dim())
    _dev(biases, "biases", (torch.bfloat16, torch.int16), biases.dim())
    if (tuple(x.shape) != (1, K) or packed.numel() * 8 != N * K or G <= 0
            or scales.numel() != N * (K // G) or biases.numel() != scales.numel()):
        raise TQError("w4a16: shapes do not match N=%d K=%d G=%d" % (N, K, G))


def w4a16_gemv(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
               biases: torch.Tensor, N: int, K: int, G: int, out=None):
    """W4A16, M = 1: x [1,K] bf16, packed int32/uint32 [N, K/8], scales and
    biases bf16 [N, K/G] -> y bf16 [1,N]."""
    _w4_check(x, packed, scales, biases, N, K, G)
    y = torch.empty((1, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _rc(lib().tq_w4a16_gemv(x.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                            biases.data_ptr(), N, K, G, y.data_ptr(), _stream()),
        "tq_w4a16_gemv")
    return y


def w4a16_gemv_batched(xs, packeds, scales_list, biases_list, N: int, K: int, G: int,
                       outs=None):
    """Same-shaped W4A16 problems -> list of y bf16 [1,N], one launch per 64."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(biases_list) == n):
        raise TQError("xs, packeds, scales and biases differ in length")
    for x, pk, sc, bi in zip(xs, packeds, scales_list, biases_list):
        _w4_check(x, pk, sc, bi, N, K, G)
    if outs is None:
        outs = [torch.empty((1, N), dtype=torch.bfloat16, device=x.device) for x in xs]
    _rc(lib().tq_w4a16_gemv_batched(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list),
                                    _ptrs(biases_list), _ptrs(outs), N, K, G, _stream()),
        "tq_w4a16_gemv_batched")
    return outs


def gemv2_grouped(xs, packeds, scales_list, Ns, Ks, G: int, status=None, outs=None):
    """2-bit format, M = 1, problems of mixed shapes in one launch:
    list of y fp32 [1, Ns[i]]."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(Ns) == len(Ks) == n):
        raise TQError("xs, packeds, scales, Ns and Ks differ in length")
    for x, pk, sc, N, K in zip(xs, packeds, scales_list, Ns, Ks):
        _dev(x, "x", (torch.bfloat16, torch.int16), 2)
        _dev(pk, "packed", (torch.uint8,), pk.dim())
        _dev(sc, "scales", (torch.float16, torch.int16), sc.dim())
        if (tuple(x.shape) != (1, K) or pk.numel() * 4 != N * K or G <= 0
                or sc.numel() != N * (K // G)):
            raise TQError("gemv2_grouped: shapes do not match N=%d K=%d G=%d" % (N, K, G))
    if outs is None:
        outs = [torch.empty((1, N), dtype=torch.float32, device=x.device) for x, N in zip(xs, Ns)]
    i64s = ctypes.c_int64 * max(n, 1)
    _rc(lib().tq_gemv2_grouped(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(outs),
                               i64s(*Ns), i64s(*Ks), G, _st(status), _stream()),
        "tq_gemv2_grouped")
    return outs


def w4a16_gemv_grouped(xs, packeds, scales_list, biases_list, Ns, Ks, G: int, outs=None):
    """W4A16 problems of mixed shapes in one launch -> list of y bf16 [1, Ns[i]]."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(biases_list) == len(Ns) == len(Ks) == n):
        raise TQError("xs, packeds, scales, biases, Ns and Ks differ in length")
    for x, pk, sc, bi, N, K in zip(xs, packeds, scales_list, biases_list, Ns, Ks):
        _w4_check(x, pk, sc, bi, N, K, G)
    if outs is None:
        outs = [torch.empty((1, N), dtype=torch.bfloat16, device=x.device) for x, N in zip(xs, Ns)]
    i64s = ctypes.c_int64 * max(n, 1)
    _rc(lib().tq_w4a16_gemv_grouped(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list),
                                    _ptrs(biases_list), _ptrs(outs), i64s(*Ns), i64s(*Ks), G,
                                    _stream()), "tq_w4a16_gemv_grouped")
    return outs


class FakeQuantize(torch.autograd.Function):
    """w_hat = fake_quantize(w, G) in the forward pass; the backward pass is
    straight-through: the gradient of w_hat is returned as the gradient of w
    unchanged (no kernel runs)."""

    @staticmethod
    def forward(ctx, w, G):
        return fake_quantize(w, G)

    @staticmethod
    def backward(ctx, grad):
        return grad, None


def unpack(packed: torch.Tensor, N: int, K: int, G: int, status=None, out=None):
    """packed -> codes int8 [N,K]."""
    _dev(packed, "packed", (torch.uint8,), packed.dim())
    if packed.numel() != packed_bytes(N, K, G):
        raise TQError("packed has %d bytes, expected %d" % (packed.numel(), packed_bytes(N, K, G)))
    codes = torch.empty((N, K), dtype=torch.int8, device=packed.device) if out is None else out
    _rc(lib().tq_unpack(packed.data_ptr(), N, K, G, codes.data_ptr(), _st(status), _stream()),
        "tq_unpack")
    return codes


def dequantize(packed: torch.Tensor, scales: torch.Tensor, N: int, K: int, G: int, status=None,
               out=None):
    """(packed, fp16 scales) -> w_hat bf16 [N,K] = bf16(c * s)."""
    _dev(packed, "packed", (torch.uint8,), packed.dim())
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16), scales.dim())
    if packed.numel() != packed_bytes(N, K, G):
        raise TQError("packed has %d bytes, expected %d" % (packed.numel(), packed_bytes(N, K, G)))
    if G <= 0 or scales.numel() != N * (K // G):
        raise TQError("scales has %d entries, expected %d" % (scales.numel(), N * (K // max(G, 1))))
    w_hat = torch.empty((N, K), dtype=torch.bfloat16, device=packed.device) if out is None else out
    _rc(lib().tq_dequantize(packed.data_ptr(), scales.data_ptr(), N, K, G, w_hat.data_ptr(),
                            _st(status), _stream()), "tq_dequantize")
    return w_hat


def dequantize_batched(packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """Same-shaped (packed, scales) pairs -> list of bf16 [N,K], one launch per 64."""
    n = len(packeds)
    if len(scales_list) != n:
        raise TQError("packeds and scales differ in length")
    for pk, sc in zip(packeds, scales_list):
        _dev(pk, "packed", (torch.uint8,), pk.dim())
        _dev(sc, "scales", (torch.float16, torch.int16, torch.uint16), sc.dim())
        if pk.numel() != packed_bytes(N, K, G) or G <= 0 or sc.numel() != N * (K // G):
            raise TQError("a packed/scales pair does not match N=%d K=%d G=%d" % (N, K, G))
    if outs is None:
        outs = [torch.empty((N, K), dtype=torch.bfloat16, device=pk.device) for pk in packeds]
    arr = ctypes.c_void_p * max(n, 1)
    _rc(lib().tq_dequantize_batched(n, arr(*[t.data_ptr() for t in packeds]),
                                    arr(*[t.data_ptr() for t in scales_list]),
                                    arr(*[t.data_ptr() for t in outs]), N, K, G, _st(status),
                                    _stream()), "tq_dequantize_batched")
    return outs


def _mm(fn, name, x, packed, scales, N, K, G, status, out):
    _dev(x, "x", (torch.bfloat16, torch.int16), 2)
    _dev(packed, "packed", (torch.uint8,), packed.dim())
    _dev(scales, "scales", (torch.float16, torch.int16), scales.dim())
    M = x.shape[0]
    if x.shape[1] != K:
        raise TQError("x has K=%d, expected %d" % (x.shape[1], K))
    if packed.numel() != packed_bytes(N, K, G) or scales.numel() != N * (K // G):
        raise TQError("packed/scales sizes do not match N=%d K=%d G=%d" % (N, K, G))
    y = torch.empty((M, N), dtype=torch.float32, device=x.device) if out is None else out
    _rc(fn(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), M, N, K, G, y.data_ptr(),
           _st(status), _stream()), name)
    return y


def gemv(x, packed, scales, N: int, K: int, G: int, status=None, out=None):
    """y[M,N] = x[M,K] * W_hat^T for 1 <= M <= 16 (decode path)."""
    return _mm(lib().tq_gemv, "tq_gemv", x, packed, scales, N, K, G, status, out)


def _batched(fn, name, xs, packeds, scales_list, N, K, G, status, outs):
    count = len(xs)
    if not (len(packeds) == len(scales_list) == count):
        raise TQError("%s: lists of different lengths" % name)
    ys = []
    for i in range(count):
        _dev(xs[i], "x", (torch.bfloat16, torch.int16), 2)
        _dev(packeds[i], "packed", (torch.uint8,), packeds[i].dim())
        _dev(scales_list[i], "scales", (torch.float16, torch.int16), scales_list[i].dim())
        if xs[i].shape != xs[0].shape or xs[i].shape[1] != K:
            raise TQError("%s: every x must be [M,%d]" % (name, K))
        if packeds[i].numel() != packed_bytes(N, K, G) or scales_list[i].numel() != N * (K // G):
            raise TQError("%s: packed/scales sizes do not match N=%d K=%d G=%d" % (name, N, K, G))
        ys.append(torch.empty((xs[0].shape[0], N), dtype=torch.float32, device=xs[i].device)
                  if outs is None else outs[i])
    arr = ctypes.c_void_p * max(count, 1)
    ax = arr(*[t.data_ptr() for t in xs])
    ap = arr(*[t.data_ptr() for t in packeds])
    asc = arr(*[t.data_ptr() for t in scales_list])
    ay = arr(*[t.data_ptr() for t in ys])
    M = xs[0].shape[0] if count else 1
    _rc(fn(count, ax, ap, asc, ay, M, N, K, G, _st(status), _stream()), name)
    return ys


def gemv_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """[x_i] ([M,K] bf16 each, M <= 16), [packed_i], [scales_i] -> [y_i] ([M,N] fp32), one call."""
    return _batched(lib().tq_gemv_batched, "tq_gemv_batched", xs, packeds, scales_list, N, K, G,
                    status, outs)


def gemv_grouped(xs, packeds, scales_list, Ns, Ks, G: int, status=None, outs=None):
    """[x_i] ([1,K_i] bf16), [packed_i], [scales_i] of shapes (N_i, K_i) -> [y_i] ([1,N_i]
    fp32): M = 1 GEMVs of mixed shapes in as few launches as possible."""
    count = len(xs)
    if not (len(packeds) == len(scales_list) == len(Ns) == len(Ks) == count):
        raise TQError("tq_gemv_grouped: lists of different lengths")
    ys = []
    for i in range(count):
        _dev(xs[i], "x", (torch.bfloat16, torch.int16), 2)
        _dev(packeds[i], "packed", (torch.uint8,), packeds[i].dim())
        _dev(scales_list[i], "scales", (torch.float16, torch.int16), scales_list[i].dim())
        N, K = int(Ns[i]), int(Ks[i])
        if tuple(xs[i].shape) != (1, K):
            raise TQError("tq_gemv_grouped: x %d must be [1,%d]" % (i, K))
        if packeds[i].numel() != packed_bytes(N, K, G) or scales_list[i].numel() != N * (K // G):
            raise TQError("tq_gemv_grouped: packed/scales %d do not match N=%d K=%d G=%d"
                          % (i, N, K, G))
        ys.append(torch.empty((1, N), dtype=torch.float32, device=xs[i].device)
                  if outs is None else outs[i])
    arr = ctypes.c_void_p * max(count, 1)
    i64s = ctypes.c_int64 * max(count, 1)
    _rc(lib().tq_gemv_grouped(count, arr(*[t.data_ptr() for t in xs]),
                              arr(*[t.data_ptr() for t in packeds]),
                              arr(*[t.data_ptr() for t in scales_list]),
                              arr(*[t.data_ptr() for t in ys]),
                              i64s(*[int(n) for n in Ns]), i64s(*[int(k) for k in Ks]), G,
                              _st(status), _stream()), "tq_gemv_grouped")
    return ys


def gemm_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """[x_i] ([M,K] bf16 each), [packed_i], [scales_i] -> [y_i] ([M,N] fp32), one call."""
    return _batched(lib().tq_gemm_batched, "tq_gemm_batched", xs, packeds, scales_list, N, K, G,
                    status, outs)


def gemm(x, packed, scales, N: int, K: int, G: int, status=None, out=None):
    """y[M,N] = x[M,K] * W_hat^T for any M (prefill path)."""
    return _mm(lib().tq_gemm, "tq_gemm", x, packed, scales, N, K, G, status, out)
