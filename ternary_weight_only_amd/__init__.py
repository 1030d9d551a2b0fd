"""ternary_weight_only_amd -- group-wise ternary weight quantization and the
packed-ternary x bf16 matmul on AMD MI355X (gfx950).

The work happens in libtq.so (hand-written HIP; C ABI in include/tq.h).  This
package only marshals torch tensors to that ABI:

    packed, scales = quantize_pack(w_bf16, G)      # scale, codes, base-3 bytes
    w_hat          = fake_quantize(w_bf16, G)      # QAT forward, bf16 c * s
    w_hat          = fake_quantize_f32(w_f32, G)   # the same from fp32 latent weights
    w_hat          = FakeQuantize.apply(w, G)      # same, straight-through gradient
    codes          = unpack(packed, N, K, G)       # codes + validation
    (the *_batched forms take lists of same-shaped matrices, one launch per 64)
    w_hat          = dequantize(packed, scales, N, K, G)  # bf16 c * s
    packed2, scales = quantize_pack2(w_bf16, G)     # 2-bit format, four codes a byte
    y              = gemv2(x_bf16, packed2, scales, N, K, G)  # its M = 1 GEMV
    y              = gemm2(x_bf16, packed2, scales, N, K, G)  # any M, any K
    w_hats         = dequantize_batched(packeds, scales, N, K, G)  # many same-shaped
    y              = gemv(x_bf16, packed, scales, N, K, G)   # M <= 16
    ys             = gemv_batched(xs, packeds, scales, N, K, G)  # many same-shaped
    ys             = gemv_grouped(xs, packeds, scales, Ns, Ks, G)  # M = 1, mixed shapes
    y              = gemm(x_bf16, packed, scales, N, K, G)   # any M
    ys             = gemm_batched(xs, packeds, scales, N, K, G)  # many same-shaped
    ys             = gemm_grouped(xs, packeds, scales, Ns, Ks, G)  # one M, mixed shapes

`ternary_weight_only_amd.package` writes and reads the per-tensor package
(codes + fp16 scales + sha256 hashes) and decodes it to bf16 on the device.

torch supplies device memory and the current stream; no arithmetic of the
method runs in Python or torch.  The library is loaded on first use and a
missing build raises immediately; there is no CPU fallback.
"""
from .binding import (  # noqa: F401
    FakeQuantize,
    TQError,
    DEV_BAD_PADDING,
    DEV_INVALID_BYTE,
    DEV_NONFINITE,
    DEV_SCALE_OVERFLOW,
    check,
    dequantize,
    dequantize_batched,
    fake_quantize,
    fake_quantize_batched,
    fake_quantize_f32,
    fake_quantize_f32_batched,
    gemm,
    gemm_batched,
    gemm_grouped,
    gemv,
    gemv_batched,
    gemv_grouped,
    gemm2,
    gemm2_batched,
    gemv2,
    gemv2_batched,
    gemv2_grouped,
    w4a16_gemv,
    w4a16_gemv_batched,
    w4a16_gemv_grouped,
    w4a16_gemm,
    w4a16_gemm_batched,
    lib,
    new_status,
    packed_bytes,
    packed_row_bytes,
    quantize_pack,
    quantize_pack_batched,
    quantize_pack2,
    quantize_pack2_batched,
    unpack,
    unpack_batched,
    unpack2,
)
