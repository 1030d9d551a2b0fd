"""ctypes binding of libtq.so (C ABI: include/tq.h).

Argument marshalling only: shape/dtype/device/contiguity checks on torch
tensors -- inputs, caller-supplied outputs and status words alike -- output
allocation, raw device pointers and the current HIP stream.  Every step of
the computation runs in the library's kernels.
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
SYMBOLS = ("tq_status_string", "tq_packed_row_bytes", "tq_packed_bytes", "tq_quantize_pack",
           "tq_quantize_pack_batched", "tq_fake_quantize", "tq_fake_quantize_batched",
           "tq_fake_quantize_f32", "tq_fake_quantize_f32_batched", "tq_unpack",
           "tq_unpack_batched", "tq_dequantize", "tq_dequantize_batched", "tq_quantize_pack2",
           "tq_quantize_pack2_batched", "tq_unpack2", "tq_gemv2", "tq_gemv2_batched",
           "tq_gemv2_grouped", "tq_gemm2", "tq_gemm2_batched", "tq_w4a16_gemv", "tq_w4a16_gemv_batched", "tq_w4a16_gemv_grouped",
           "tq_w4a16_gemm", "tq_w4a16_gemm_batched", "tq_gemv", "tq_gemv_batched", "tq_gemv_grouped", "tq_gemm", "tq_gemm_batched", "tq_gemm_grouped")
# Every symbol include/tq_probe.h declares (measurement probes).
PROBE_SYMBOLS = ("tq_probe_lds_table", "tq_probe_mfma_bf16", "tq_probe_read_stream",
                 "tq_probe_valu")

_lib = None

BF16 = (torch.bfloat16, torch.int16)
F16 = (torch.float16, torch.int16)
U8 = (torch.uint8,)
I8 = (torch.int8,)
F32 = (torch.float32,)
W4 = (torch.int32, torch.uint32)


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
        l.tq_packed_row_bytes.argtypes = [i64, i32]
        l.tq_packed_row_bytes.restype = i64
        l.tq_packed_bytes.argtypes = [i64, i64, i32]
        l.tq_packed_bytes.restype = i64
        l.tq_quantize_pack.argtypes = [p, i64, i64, i32, p, p, p, p]
        l.tq_quantize_pack.restype = i32
        l.tq_fake_quantize.argtypes = [p, i64, i64, i32, p, p, p, p]
        l.tq_fake_quantize.restype = i32
        l.tq_fake_quantize_f32.argtypes = [p, i64, i64, i32, p, p, p, p]
        l.tq_fake_quantize_f32.restype = i32
        l.tq_fake_quantize_f32_batched.argtypes = [i32, p, i64, i64, i32, p, p, p, p]
        l.tq_fake_quantize_f32_batched.restype = i32
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
        l.tq_gemm2.argtypes = [p, p, p, i64, i64, i64, i32, p, p, p]
        l.tq_gemm2.restype = i32
        l.tq_gemm2_batched.argtypes = [i32, p, p, p, p, i64, i64, i64, i32, p, p]
        l.tq_gemm2_batched.restype = i32
        l.tq_w4a16_gemv.argtypes = [p, p, p, p, i64, i64, i32, p, p]
        l.tq_w4a16_gemv.restype = i32
        l.tq_w4a16_gemv_batched.argtypes = [i32, p, p, p, p, p, i64, i64, i32, p]
        l.tq_w4a16_gemv_batched.restype = i32
        l.tq_w4a16_gemv_grouped.argtypes = [i32, p, p, p, p, p, p, p, i32, p]
        l.tq_w4a16_gemv_grouped.restype = i32
        l.tq_w4a16_gemm.argtypes = [p, p, p, p, i64, i64, i64, i32, p, p]
        l.tq_w4a16_gemm.restype = i32
        l.tq_w4a16_gemm_batched.argtypes = [i32, p, p, p, p, i64, i64, i64, i32, p, p]
        l.tq_w4a16_gemm_batched.restype = i32
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
        l.tq_gemm_grouped.argtypes = [i32, p, p, p, p, i64, p, p, i32, p, p]
        l.tq_gemm_grouped.restype = i32
        # measurement probes (include/tq_probe.h)
        l.tq_probe_read_stream.argtypes = [p, i64, i32, p, p]
        l.tq_probe_read_stream.restype = i32
        l.tq_probe_mfma_bf16.argtypes = [i64, i32, p, p]
        l.tq_probe_mfma_bf16.restype = i32
        l.tq_probe_lds_table.argtypes = [i32, i32, p, p, p]
        l.tq_probe_lds_table.restype = i32
        l.tq_probe_valu.argtypes = [i32, i32, i32, p, p, p]
        l.tq_probe_valu.restype = i32
        _lib = l
    return _lib


def _rc(rc: int, what: str):
    if rc != 0:
        raise TQError("%s failed: %s" % (what, lib().tq_status_string(rc).decode()))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# validation: nothing reaches the library unless every tensor it will read
# or write is a contiguous device tensor of the expected dtype and size on
# the device of the call's first input
# ---------------------------------------------------------------------------

def _dev(t, name: str, dtypes, ndim=None, device=None):
    """An input: a contiguous device tensor of one of `dtypes` (and `ndim`
    dimensions, and on `device`, when given)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TQError("%s must be a device tensor" % name)
    if device is not None and t.device != device:
        raise TQError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype not in dtypes:
        raise TQError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise TQError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise TQError("%s must be a %d-D tensor" % (name, ndim))
    return t


def _out(t, name: str, shape, dtype, dtypes, device):
    """A call's output: allocated here as `shape` of `dtype` when `t` is
    None; otherwise it must be a contiguous tensor of one of `dtypes` on
    `device` holding exactly as many elements as `shape`."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name, dtypes, None, device)
    n = 1
    for d in shape:
        n *= int(d)
    if t.numel() != n:
        raise TQError("%s has %d elements, expected %d (%s)" % (name, t.numel(), n, tuple(shape)))
    return t


def _outs(ts, name: str, shapes, dtype, dtypes, device):
    """Outputs of a batched call: one per problem, as _out."""
    if ts is None:
        return [torch.empty(s, dtype=dtype, device=device) for s in shapes]
    ts = list(ts)
    if len(ts) != len(shapes):
        raise TQError("%s: %d outputs for %d problems" % (name, len(ts), len(shapes)))
    return [_out(t, "%s[%d]" % (name, i), s, dtype, dtypes, device)
            for i, (t, s) in enumerate(zip(ts, shapes))]


def _st(status, device) -> int:
    """The device address of a status word: an int32 tensor of at least one
    element on `device`, or None (no reporting)."""
    if status is None:
        return 0
    if not isinstance(status, torch.Tensor) or not status.is_cuda or status.device != device:
        raise TQError("status must be an int32 tensor on %s" % device)
    if status.dtype != torch.int32 or status.numel() < 1 or not status.is_contiguous():
        raise TQError("status must be a contiguous int32 tensor of at least one element")
    return status.data_ptr()


def packed_row_bytes(K: int, G: int) -> int:
    """Packed bytes of one row: (K/G) * ceil(G/5); 0 for invalid arguments."""
    return int(lib().tq_packed_row_bytes(K, G))


def packed_bytes(N: int, K: int, G: int) -> int:
    return int(lib().tq_packed_bytes(N, K, G))


def _groups(K: int, G: int) -> int:
    return K // G if G > 0 and K % G == 0 else 0


def _check_packed(packed, scales, N, K, G, device, what):
    _dev(packed, "packed", U8, None, device)
    _dev(scales, "scales", F16 + (torch.uint16,), None, device)
    if packed.numel() != packed_bytes(N, K, G) or scales.numel() != N * _groups(K, G) \
            or packed.numel() == 0:
        raise TQError("%s: packed/scales sizes (%d, %d) do not match N=%d K=%d G=%d"
                      % (what, packed.numel(), scales.numel(), N, K, G))


def _ptrs(ts):
    return (ctypes.c_void_p * max(len(ts), 1))(*[t.data_ptr() for t in ts])


def _i64s(vals):
    return (ctypes.c_int64 * max(len(vals), 1))(*[int(v) for v in vals])


def new_status(device=None) -> torch.Tensor:
    """A zeroed device int32 status word."""
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


def check(status: torch.Tensor) -> int:
    """Synchronize-free read of a status word (forces a device->host copy)."""
    return int(status.item())


# ---------------------------------------------------------------------------
# quantize / QAT forward / unpack / decode
# ---------------------------------------------------------------------------

def quantize_pack(w: torch.Tensor, G: int, status=None, out=None):
    """w: [N,K] bf16 -> (packed uint8 [N, (K/G)*ceil(G/5)], scales fp16 [N, K/G]).
    `out`, if given, is a (packed, scales) pair of that size."""
    _dev(w, "w", BF16, 2)
    N, K = w.shape
    rb, ng = packed_row_bytes(K, G), _groups(K, G)
    if rb == 0:
        raise TQError("quantize_pack: K=%d is not a multiple of G=%d" % (K, G))
    packed, scales = (None, None) if out is None else out
    packed = _out(packed, "packed", (N, rb), torch.uint8, U8, w.device)
    scales = _out(scales, "scales", (N, ng), torch.float16, F16, w.device)
    _rc(lib().tq_quantize_pack(w.data_ptr(), N, K, G, packed.data_ptr(), scales.data_ptr(),
                               _st(status, w.device), _stream()), "tq_quantize_pack")
    return packed, scales


def fake_quantize(w: torch.Tensor, G: int, status=None, out=None, scales_out=None):
    """QAT forward: w [N,K] bf16 -> w_hat bf16 [N,K] = bf16(c * s).

    scales_out, if given, is an fp16 [N, K/G] tensor that receives the
    scales.  Use FakeQuantize.apply for the straight-through gradient."""
    _dev(w, "w", BF16, 2)
    N, K = w.shape
    w_hat = _out(out, "w_hat", (N, K), torch.bfloat16, BF16, w.device)
    sp = 0
    if scales_out is not None:
        if _groups(K, G) == 0:
            raise TQError("fake_quantize: K=%d is not a multiple of G=%d" % (K, G))
        sp = _out(scales_out, "scales_out", (N, _groups(K, G)), torch.float16, F16,
                  w.device).data_ptr()
    _rc(lib().tq_fake_quantize(w.data_ptr(), N, K, G, w_hat.data_ptr(), sp,
                               _st(status, w.device), _stream()), "tq_fake_quantize")
    return w_hat


def fake_quantize_f32(w: torch.Tensor, G: int, status=None, out=None, scales_out=None):
    """QAT forward from fp32 latent weights: w [N,K] fp32 -> w_hat fp32 [N,K]
    = c * s (exact).  scales_out as for fake_quantize."""
    _dev(w, "w", F32, 2)
    N, K = w.shape
    w_hat = _out(out, "w_hat", (N, K), torch.float32, F32, w.device)
    if w_hat.data_ptr() == w.data_ptr():
        raise TQError("fake_quantize_f32: w_hat may not alias w")
    sp = 0
    if scales_out is not None:
        if _groups(K, G) == 0:
            raise TQError("fake_quantize_f32: K=%d is not a multiple of G=%d" % (K, G))
        sp = _out(scales_out, "scales_out", (N, _groups(K, G)), torch.float16, F16,
                  w.device).data_ptr()
    _rc(lib().tq_fake_quantize_f32(w.data_ptr(), N, K, G, w_hat.data_ptr(), sp,
                                   _st(status, w.device), _stream()), "tq_fake_quantize_f32")
    return w_hat


def fake_quantize_f32_batched(ws, G: int, status=None, outs=None):
    """Same-shaped fp32 latent matrices -> list of w_hat fp32, one launch per 64."""
    if not ws:
        return []
    for w in ws:
        _dev(w, "w", F32, 2, ws[0].device)
    shapes = {tuple(w.shape) for w in ws}
    if len(shapes) > 1:
        raise TQError("fake_quantize_f32_batched: matrices of different shapes %s"
                      % sorted(shapes))
    N, K = shapes.pop()
    dev = ws[0].device
    outs = _outs(outs, "outs", [(N, K)] * len(ws), torch.float32, F32, dev)
    _rc(lib().tq_fake_quantize_f32_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(outs), None,
                                           _st(status, dev), _stream()),
        "tq_fake_quantize_f32_batched")
    return outs


def _same_shape(ws, name):
    for w in ws:
        _dev(w, name, BF16, 2, ws[0].device)
    shapes = {tuple(w.shape) for w in ws}
    if len(shapes) > 1:
        raise TQError("%s: matrices of different shapes %s" % (name, sorted(shapes)))
    return shapes.pop() if shapes else (0, 0)


def quantize_pack_batched(ws, G: int, status=None):
    """Same-shaped bf16 matrices -> list of (packed, scales), one launch per 64."""
    N, K = _same_shape(ws, "w")
    if not ws:
        return []
    rb, ng = packed_row_bytes(K, G), _groups(K, G)
    if rb == 0:
        raise TQError("quantize_pack_batched: K=%d is not a multiple of G=%d" % (K, G))
    dev = ws[0].device
    pk = [torch.empty((N, rb), dtype=torch.uint8, device=dev) for _ in ws]
    sc = [torch.empty((N, ng), dtype=torch.float16, device=dev) for _ in ws]
    _rc(lib().tq_quantize_pack_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(pk), _ptrs(sc),
                                       _st(status, dev), _stream()), "tq_quantize_pack_batched")
    return list(zip(pk, sc))


def fake_quantize_batched(ws, G: int, status=None, with_scales: bool = False):
    """Same-shaped bf16 matrices -> list of bf16 w_hat (and, with_scales, of
    (w_hat, scales)), one launch per 64."""
    N, K = _same_shape(ws, "w")
    if not ws:
        return []
    dev = ws[0].device
    wh = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in ws]
    if with_scales and _groups(K, G) == 0:
        raise TQError("fake_quantize_batched: K=%d is not a multiple of G=%d" % (K, G))
    sc = [torch.empty((N, _groups(K, G)), dtype=torch.float16, device=dev)
          for _ in ws] if with_scales else None
    _rc(lib().tq_fake_quantize_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(wh),
                                       _ptrs(sc) if with_scales else None, _st(status, dev),
                                       _stream()), "tq_fake_quantize_batched")
    return list(zip(wh, sc)) if with_scales else wh


def unpack(packed: torch.Tensor, N: int, K: int, G: int, status=None, out=None):
    """packed -> codes int8 [N,K]."""
    _dev(packed, "packed", U8)
    if packed.numel() != packed_bytes(N, K, G) or packed.numel() == 0:
        raise TQError("packed has %d bytes, expected %d" % (packed.numel(), packed_bytes(N, K, G)))
    codes = _out(out, "codes", (N, K), torch.int8, I8, packed.device)
    _rc(lib().tq_unpack(packed.data_ptr(), N, K, G, codes.data_ptr(), _st(status, packed.device),
                        _stream()), "tq_unpack")
    return codes


def unpack_batched(packeds, N: int, K: int, G: int, status=None):
    """Same-shaped packed matrices -> list of int8 codes [N,K], one launch per 64."""
    if not packeds:
        return []
    dev = packeds[0].device if isinstance(packeds[0], torch.Tensor) else None
    for p in packeds:
        _dev(p, "packed", U8, None, dev)
        if p.numel() != packed_bytes(N, K, G) or p.numel() == 0:
            raise TQError("packed has %d bytes, expected %d" % (p.numel(), packed_bytes(N, K, G)))
    codes = [torch.empty((N, K), dtype=torch.int8, device=dev) for _ in packeds]
    _rc(lib().tq_unpack_batched(len(packeds), _ptrs(packeds), N, K, G, _ptrs(codes),
                                _st(status, dev), _stream()), "tq_unpack_batched")
    return codes


def dequantize(packed: torch.Tensor, scales: torch.Tensor, N: int, K: int, G: int, status=None,
               out=None):
    """(packed, fp16 scales) -> w_hat bf16 [N,K] = bf16(c * s)."""
    _dev(packed, "packed", U8)
    _check_packed(packed, scales, N, K, G, packed.device, "dequantize")
    w_hat = _out(out, "w_hat", (N, K), torch.bfloat16, BF16, packed.device)
    _rc(lib().tq_dequantize(packed.data_ptr(), scales.data_ptr(), N, K, G, w_hat.data_ptr(),
                            _st(status, packed.device), _stream()), "tq_dequantize")
    return w_hat


def dequantize_batched(packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """Same-shaped (packed, scales) pairs -> list of bf16 [N,K], one launch per 64."""
    n = len(packeds)
    if len(scales_list) != n:
        raise TQError("packeds and scales differ in length")
    if n == 0:
        return []
    _dev(packeds[0], "packed", U8)
    dev = packeds[0].device
    for pk, sc in zip(packeds, scales_list):
        _check_packed(pk, sc, N, K, G, dev, "dequantize_batched")
    outs = _outs(outs, "outs", [(N, K)] * n, torch.bfloat16, BF16, dev)
    _rc(lib().tq_dequantize_batched(n, _ptrs(packeds), _ptrs(scales_list), _ptrs(outs), N, K, G,
                                    _st(status, dev), _stream()), "tq_dequantize_batched")
    return outs


class FakeQuantize(torch.autograd.Function):
    """w_hat = fake_quantize(w, G) (bf16 latent weights) or
    fake_quantize_f32(w, G) (fp32 latent weights) in the forward pass; the
    backward pass is straight-through: the gradient of w_hat is returned as
    the gradient of w unchanged (no kernel runs)."""

    @staticmethod
    def forward(ctx, w, G):
        return fake_quantize_f32(w, G) if w.dtype == torch.float32 else fake_quantize(w, G)

    @staticmethod
    def backward(ctx, grad):
        return grad, None


# ---------------------------------------------------------------------------
# base-3 matmuls
# ---------------------------------------------------------------------------

def _mm(fn, name, x, packed, scales, N, K, G, status, out):
    _dev(x, "x", BF16, 2)
    dev = x.device
    M = x.shape[0]
    if x.shape[1] != K:
        raise TQError("x has K=%d, expected %d" % (x.shape[1], K))
    _check_packed(packed, scales, N, K, G, dev, name)
    y = _out(out, "y", (M, N), torch.float32, F32, dev)
    _rc(fn(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), M, N, K, G, y.data_ptr(),
           _st(status, dev), _stream()), name)
    return y


def gemv(x, packed, scales, N: int, K: int, G: int, status=None, out=None):
    """y[M,N] = x[M,K] * W_hat^T for 1 <= M <= 16 (decode path)."""
    return _mm(lib().tq_gemv, "tq_gemv", x, packed, scales, N, K, G, status, out)


def gemm(x, packed, scales, N: int, K: int, G: int, status=None, out=None):
    """y[M,N] = x[M,K] * W_hat^T for any M (prefill path)."""
    return _mm(lib().tq_gemm, "tq_gemm", x, packed, scales, N, K, G, status, out)


def _batched(fn, name, xs, packeds, scales_list, N, K, G, status, outs):
    count = len(xs)
    if not (len(packeds) == len(scales_list) == count):
        raise TQError("%s: lists of different lengths" % name)
    if count == 0:
        return []
    _dev(xs[0], "x", BF16, 2)
    dev = xs[0].device
    M = xs[0].shape[0]
    for i in range(count):
        _dev(xs[i], "x", BF16, 2, dev)
        if tuple(xs[i].shape) != (M, K):
            raise TQError("%s: every x must be [%d,%d]" % (name, M, K))
        _check_packed(packeds[i], scales_list[i], N, K, G, dev, name)
    ys = _outs(outs, "outs", [(M, N)] * count, torch.float32, F32, dev)
    _rc(fn(count, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(ys), M, N, K, G,
           _st(status, dev), _stream()), name)
    return ys


def gemv_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """[x_i] ([M,K] bf16 each, M <= 16), [packed_i], [scales_i] -> [y_i] ([M,N] fp32), one call."""
    return _batched(lib().tq_gemv_batched, "tq_gemv_batched", xs, packeds, scales_list, N, K, G,
                    status, outs)


def gemm_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """[x_i] ([M,K] bf16 each), [packed_i], [scales_i] -> [y_i] ([M,N] fp32), one call."""
    return _batched(lib().tq_gemm_batched, "tq_gemm_batched", xs, packeds, scales_list, N, K, G,
                    status, outs)


def gemv_grouped(xs, packeds, scales_list, Ns, Ks, G: int, status=None, outs=None):
    """[x_i] ([1,K_i] bf16), [packed_i], [scales_i] of shapes (N_i, K_i) -> [y_i] ([1,N_i]
    fp32): M = 1 GEMVs of mixed shapes in as few launches as possible."""
    count = len(xs)
    if not (len(packeds) == len(scales_list) == len(Ns) == len(Ks) == count):
        raise TQError("tq_gemv_grouped: lists of different lengths")
    if count == 0:
        return []
    _dev(xs[0], "x", BF16, 2)
    dev = xs[0].device
    for i in range(count):
        N, K = int(Ns[i]), int(Ks[i])
        _dev(xs[i], "x", BF16, 2, dev)
        if tuple(xs[i].shape) != (1, K):
            raise TQError("tq_gemv_grouped: x %d must be [1,%d]" % (i, K))
        _check_packed(packeds[i], scales_list[i], N, K, G, dev, "tq_gemv_grouped")
    ys = _outs(outs, "outs", [(1, int(N)) for N in Ns], torch.float32, F32, dev)
    _rc(lib().tq_gemv_grouped(count, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(ys),
                              _i64s(Ns), _i64s(Ks), G, _st(status, dev), _stream()),
        "tq_gemv_grouped")
    return ys


def gemm_grouped(xs, packeds, scales_list, Ns, Ks, G: int, status=None, outs=None):
    """[x_i] ([M,K_i] bf16, one M), [packed_i], [scales_i] of shapes (N_i, K_i) -> [y_i]
    ([M,N_i] fp32): prefill matmuls of mixed shapes, one persistent launch where possible."""
    count = len(xs)
    if not (len(packeds) == len(scales_list) == len(Ns) == len(Ks) == count):
        raise TQError("tq_gemm_grouped: lists of different lengths")
    if count == 0:
        return []
    _dev(xs[0], "x", BF16, 2)
    dev = xs[0].device
    M = int(xs[0].shape[0])
    for i in range(count):
        N, K = int(Ns[i]), int(Ks[i])
        _dev(xs[i], "x", BF16, 2, dev)
        if tuple(xs[i].shape) != (M, K):
            raise TQError("tq_gemm_grouped: x %d must be [%d,%d]" % (i, M, K))
        _check_packed(packeds[i], scales_list[i], N, K, G, dev, "tq_gemm_grouped")
    ys = _outs(outs, "outs", [(M, int(N)) for N in Ns], torch.float32, F32, dev)
    _rc(lib().tq_gemm_grouped(count, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(ys),
                              M, _i64s(Ns), _i64s(Ks), G, _st(status, dev), _stream()),
        "tq_gemm_grouped")
    return ys


# ---------------------------------------------------------------------------
# the 2-bit format
# ---------------------------------------------------------------------------

def _check_packed2(packed, scales, N, K, G, device, what):
    _dev(packed, "packed", U8, None, device)
    _dev(scales, "scales", F16, None, device)
    if (N < 1 or K < 1 or K % 4 or packed.numel() * 4 != N * K
            or scales.numel() != N * _groups(K, G)):
        raise TQError("%s: shapes do not match N=%d K=%d G=%d" % (what, N, K, G))


def quantize_pack2(w: torch.Tensor, G: int, status=None):
    """2-bit format: w [N,K] bf16 -> (packed2 uint8 [N, K/4], scales fp16 [N, K/G])."""
    _dev(w, "w", BF16, 2)
    N, K = w.shape
    if _groups(K, G) == 0 or K % 4:
        raise TQError("quantize_pack2: K=%d does not fit G=%d" % (K, G))
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // G), dtype=torch.float16, device=w.device)
    _rc(lib().tq_quantize_pack2(w.data_ptr(), N, K, G, packed.data_ptr(), scales.data_ptr(),
                                _st(status, w.device), _stream()), "tq_quantize_pack2")
    return packed, scales


def quantize_pack2_batched(ws, G: int, status=None):
    """2-bit format, same-shaped bf16 matrices -> list of (packed2, scales),
    one launch per 64."""
    N, K = _same_shape(ws, "w")
    if not ws:
        return []
    if _groups(K, G) == 0 or K % 4:
        raise TQError("quantize_pack2_batched: K=%d does not fit G=%d" % (K, G))
    dev = ws[0].device
    pk = [torch.empty((N, K // 4), dtype=torch.uint8, device=dev) for _ in ws]
    sc = [torch.empty((N, K // G), dtype=torch.float16, device=dev) for _ in ws]
    _rc(lib().tq_quantize_pack2_batched(len(ws), _ptrs(ws), N, K, G, _ptrs(pk), _ptrs(sc),
                                        _st(status, dev), _stream()), "tq_quantize_pack2_batched")
    return list(zip(pk, sc))


def unpack2(packed: torch.Tensor, N: int, K: int, G: int, status=None):
    """2-bit packed [N, K/4] -> codes int8 [N,K]."""
    _dev(packed, "packed", U8)
    if N < 1 or K < 1 or packed.numel() * 4 != N * K:
        raise TQError("packed has %d bytes, expected %d" % (packed.numel(), N * K // 4))
    codes = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _rc(lib().tq_unpack2(packed.data_ptr(), N, K, G, codes.data_ptr(),
                         _st(status, packed.device), _stream()), "tq_unpack2")
    return codes


def gemv2(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, N: int, K: int, G: int,
          status=None, out=None):
    """2-bit format, M = 1: x [1,K] bf16 -> y fp32 [1,N]."""
    _dev(x, "x", BF16, 2)
    dev = x.device
    if tuple(x.shape) != (1, K):
        raise TQError("gemv2: x must be [1,%d]" % K)
    _check_packed2(packed, scales, N, K, G, dev, "gemv2")
    y = _out(out, "y", (1, N), torch.float32, F32, dev)
    _rc(lib().tq_gemv2(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), N, K, G, y.data_ptr(),
                       _st(status, dev), _stream()), "tq_gemv2")
    return y


def gemm2(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, N: int, K: int, G: int,
          status=None, out=None):
    """2-bit format, any M: x [M,K] bf16 -> y fp32 [M,N]."""
    _dev(x, "x", BF16, 2)
    dev = x.device
    if x.shape[1] != K:
        raise TQError("gemm2: x must be [M,%d]" % K)
    M = x.shape[0]
    _check_packed2(packed, scales, N, K, G, dev, "gemm2")
    y = _out(out, "y", (M, N), torch.float32, F32, dev)
    _rc(lib().tq_gemm2(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), M, N, K, G,
                       y.data_ptr(), _st(status, dev), _stream()), "tq_gemm2")
    return y


def gemm2_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """2-bit format, same-shaped problems (every x [M,K] with the same M):
    list of y fp32 [M,N], one launch per 64."""
    n = len(xs)
    if len(packeds) != n or len(scales_list) != n:
        raise TQError("xs, packeds and scales differ in length")
    if n == 0:
        return []
    _dev(xs[0], "x", BF16, 2)
    dev = xs[0].device
    M = xs[0].shape[0]
    for x, pk, sc in zip(xs, packeds, scales_list):
        _dev(x, "x", BF16, 2, dev)
        if tuple(x.shape) != (M, K):
            raise TQError("gemm2_batched: every x must be [%d,%d]" % (M, K))
        _check_packed2(pk, sc, N, K, G, dev, "gemm2_batched")
    outs = _outs(outs, "outs", [(M, N)] * n, torch.float32, F32, dev)
    _rc(lib().tq_gemm2_batched(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(outs),
                               M, N, K, G, _st(status, dev), _stream()), "tq_gemm2_batched")
    return outs


def gemv2_batched(xs, packeds, scales_list, N: int, K: int, G: int, status=None, outs=None):
    """2-bit format, M = 1, same-shaped problems: list of y fp32 [1,N], one launch per 128."""
    n = len(xs)
    if len(packeds) != n or len(scales_list) != n:
        raise TQError("xs, packeds and scales differ in length")
    if n == 0:
        return []
    _dev(xs[0], "x", BF16, 2)
    dev = xs[0].device
    for x, pk, sc in zip(xs, packeds, scales_list):
        _dev(x, "x", BF16, 2, dev)
        if tuple(x.shape) != (1, K):
            raise TQError("gemv2_batched: every x must be [1,%d]" % K)
        _check_packed2(pk, sc, N, K, G, dev, "gemv2_batched")
    outs = _outs(outs, "outs", [(1, N)] * n, torch.float32, F32, dev)
    _rc(lib().tq_gemv2_batched(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(outs),
                               N, K, G, _st(status, dev), _stream()), "tq_gemv2_batched")
    return outs


def gemv2_grouped(xs, packeds, scales_list, Ns, Ks, G: int, status=None, outs=None):
    """2-bit format, M = 1, problems of mixed shapes in one launch:
    list of y fp32 [1, Ns[i]]."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(Ns) == len(Ks) == n):
        raise TQError("xs, packeds, scales, Ns and Ks differ in length")
    if n == 0:
        return []
    _dev(xs[0], "x", BF16, 2)
    dev = xs[0].device
    for x, pk, sc, N, K in zip(xs, packeds, scales_list, Ns, Ks):
        _dev(x, "x", BF16, 2, dev)
        if tuple(x.shape) != (1, K):
            raise TQError("gemv2_grouped: x must be [1,%d]" % K)
        _check_packed2(pk, sc, N, K, G, dev, "gemv2_grouped")
    outs = _outs(outs, "outs", [(1, int(N)) for N in Ns], torch.float32, F32, dev)
    _rc(lib().tq_gemv2_grouped(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list), _ptrs(outs),
                               _i64s(Ns), _i64s(Ks), G, _st(status, dev), _stream()),
        "tq_gemv2_grouped")
    return outs


# ---------------------------------------------------------------------------
# W4A16
# ---------------------------------------------------------------------------

def _w4_check(x, packed, scales, biases, N, K, G, device=None, any_m=False):
    _dev(x, "x", BF16, 2, device)
    dev = x.device
    _dev(packed, "packed", W4, None, dev)
    _dev(scales, "scales", BF16, None, dev)
    _dev(biases, "biases", BF16, None, dev)
    if ((x.shape[1] != K or (not any_m and x.shape[0] != 1)) or N < 1 or K < 1
            or packed.numel() * 8 != N * K or _groups(K, G) == 0
            or scales.numel() != N * (K // G) or biases.numel() != scales.numel()):
        raise TQError("w4a16: shapes do not match N=%d K=%d G=%d" % (N, K, G))
    return dev


def w4a16_gemm(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
               biases: torch.Tensor, N: int, K: int, G: int, out=None):
    """W4A16, any M: x [M,K] bf16, packed int32/uint32 [N, K/8], scales and
    biases bf16 [N, K/G] -> y bf16 [M,N]."""
    dev = _w4_check(x, packed, scales, biases, N, K, G, any_m=True)
    M = x.shape[0]
    y = _out(out, "y", (M, N), torch.bfloat16, BF16, dev)
    _rc(lib().tq_w4a16_gemm(x.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                            biases.data_ptr(), M, N, K, G, y.data_ptr(), _stream()),
        "tq_w4a16_gemm")
    return y


def w4a16_gemm_batched(xs, packeds, scales_list, biases_list, N: int, K: int, G: int,
                       outs=None):
    """Same-shaped W4A16 matmuls (every x [M,K] with the same M) -> list of
    y bf16 [M,N], one launch per 64."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(biases_list) == n):
        raise TQError("xs, packeds, scales and biases differ in length")
    if n == 0:
        return []
    dev = None
    for x, pk, sc, bi in zip(xs, packeds, scales_list, biases_list):
        dev = _w4_check(x, pk, sc, bi, N, K, G, dev, any_m=True)
    M = xs[0].shape[0]
    if any(x.shape[0] != M for x in xs):
        raise TQError("w4a16_gemm_batched: every x needs the same number of rows")
    outs = _outs(outs, "outs", [(M, N)] * n, torch.bfloat16, BF16, dev)
    _rc(lib().tq_w4a16_gemm_batched(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list),
                                    _ptrs(biases_list), M, N, K, G, _ptrs(outs), _stream()),
        "tq_w4a16_gemm_batched")
    return outs


def w4a16_gemv(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
               biases: torch.Tensor, N: int, K: int, G: int, out=None):
    """W4A16, M = 1: x [1,K] bf16, packed int32/uint32 [N, K/8], scales and
    biases bf16 [N, K/G] -> y bf16 [1,N]."""
    dev = _w4_check(x, packed, scales, biases, N, K, G)
    y = _out(out, "y", (1, N), torch.bfloat16, BF16, dev)
    _rc(lib().tq_w4a16_gemv(x.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                            biases.data_ptr(), N, K, G, y.data_ptr(), _stream()),
        "tq_w4a16_gemv")
    return y


def w4a16_gemv_batched(xs, packeds, scales_list, biases_list, N: int, K: int, G: int,
                       outs=None):
    """Same-shaped W4A16 problems -> list of y bf16 [1,N], one launch per 128."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(biases_list) == n):
        raise TQError("xs, packeds, scales and biases differ in length")
    if n == 0:
        return []
    dev = None
    for x, pk, sc, bi in zip(xs, packeds, scales_list, biases_list):
        dev = _w4_check(x, pk, sc, bi, N, K, G, dev)
    outs = _outs(outs, "outs", [(1, N)] * n, torch.bfloat16, BF16, dev)
    _rc(lib().tq_w4a16_gemv_batched(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list),
                                    _ptrs(biases_list), _ptrs(outs), N, K, G, _stream()),
        "tq_w4a16_gemv_batched")
    return outs


def w4a16_gemv_grouped(xs, packeds, scales_list, biases_list, Ns, Ks, G: int, outs=None):
    """W4A16 problems of mixed shapes in one launch -> list of y bf16 [1, Ns[i]]."""
    n = len(xs)
    if not (len(packeds) == len(scales_list) == len(biases_list) == len(Ns) == len(Ks) == n):
        raise TQError("xs, packeds, scales, biases, Ns and Ks differ in length")
    if n == 0:
        return []
    dev = None
    for x, pk, sc, bi, N, K in zip(xs, packeds, scales_list, biases_list, Ns, Ks):
        dev = _w4_check(x, pk, sc, bi, N, K, G, dev)
    outs = _outs(outs, "outs", [(1, int(N)) for N in Ns], torch.bfloat16, BF16, dev)
    _rc(lib().tq_w4a16_gemv_grouped(n, _ptrs(xs), _ptrs(packeds), _ptrs(scales_list),
                                    _ptrs(biases_list), _ptrs(outs), _i64s(Ns), _i64s(Ks), G,
                                    _stream()), "tq_w4a16_gemv_grouped")
    return outs
