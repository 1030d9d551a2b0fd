// tq_api.hip -- the extern "C" entry points of libtq.so (declared in
// include/tq.h): host-side argument validation, then one launch on the
// caller's stream.  Nothing here allocates, synchronizes or falls back to
// another implementation; bad arguments return an error with nothing
// enqueued (tiny-llm "Week 2 Day 3: Quantize the Model", task 3: validate the
// layout before encoding the kernel and reject explicitly instead of
// falling back).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/tq.h"
#include "tq_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape rules shared by every call: N, K >= 1, G in {64,128}, K % G == 0
// (precisit "pack-unpack-run" README, scale-rule paragraph), and every byte
// count below 2^62.
int check_nkg(int64_t N, int64_t K, int G) {
  if (G != 64 && G != 128) return TQ_ERR_GROUP;
  if (N < 1 || K < 1 || K % G != 0) return TQ_ERR_SHAPE;
  if (N > (int64_t(1) << 40) / K) return TQ_ERR_SHAPE;  // N*K*4 stays far below 2^62
  return TQ_OK;
}

int finish_launch() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char *tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_NULL: return "TQ_ERR_NULL: a required pointer is NULL";
    case TQ_ERR_SHAPE: return "TQ_ERR_SHAPE: bad M/N/K or K not divisible by G";
    case TQ_ERR_GROUP: return "TQ_ERR_GROUP: G must be 64 or 128";
    case TQ_ERR_ALIGN: return "TQ_ERR_ALIGN: pointer not aligned as required";
    case TQ_ERR_LAUNCH: return "TQ_ERR_LAUNCH: HIP launch failed";
    default: return "unknown tq status";
  }
}

int64_t tq_packed_row_bytes(int64_t K, int G) {
  if (K < 1 || G < 1 || K % G != 0) return 0;
  return (K / G) * (int64_t)((G + 4) / 5);
}

int64_t tq_packed_bytes(int64_t N, int64_t K, int G) {
  const int64_t rb = tq_packed_row_bytes(K, G);
  if (N < 1 || rb == 0 || N > INT64_MAX / rb) return 0;
  return N * rb;
}

int tq_quantize_pack(const uint16_t *w, int64_t N, int64_t K, int G, uint8_t *packed,
                     uint16_t *scales, int32_t *d_status, void *stream) {
  if (!w || !packed || !scales) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(w, 16) || !aligned(scales, 2) || !aligned(d_status, 4)) return TQ_ERR_ALIGN;
  (void)hipGetLastError();  // clear a stale error so the check below sees only ours
  tq::launch_quantize_pack(w, N, K, G, packed, scales, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_fake_quantize(const uint16_t *w, int64_t N, int64_t K, int G, uint16_t *w_hat,
                     uint16_t *scales, int32_t *d_status, void *stream) {
  if (!w || !w_hat) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(w, 16) || !aligned(w_hat, 16) || !aligned(scales, 2) || !aligned(d_status, 4))
    return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_fake_quantize(w, N, K, G, w_hat, scales, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_fake_quantize_f32_batched(int count, const float *const *ws, int64_t N, int64_t K, int G,
                                 float *const *w_hats, uint16_t *const *scales,
                                 int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!ws || !w_hats) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!ws[i] || !w_hats[i]) return TQ_ERR_NULL;
    if (!aligned(ws[i], 16) || !aligned(w_hats[i], 16)) return TQ_ERR_ALIGN;
    if (scales && !aligned(scales[i], 2)) return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_fake_quantize_f32_batched(count, ws, N, K, G, w_hats, scales, d_status,
                                       (hipStream_t)stream);
  return finish_launch();
}

int tq_fake_quantize_f32(const float *w, int64_t N, int64_t K, int G, float *w_hat,
                         uint16_t *scales, int32_t *d_status, void *stream) {
  if (!w || !w_hat) return TQ_ERR_NULL;
  uint16_t *const sc[1] = {scales};
  return tq_fake_quantize_f32_batched(1, &w, N, K, G, &w_hat, scales ? sc : nullptr, d_status,
                                      stream);
}

int tq_quantize_pack_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                             uint8_t *const *packeds, uint16_t *const *scales,
                             int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!ws || !packeds || !scales) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!ws[i] || !packeds[i] || !scales[i]) return TQ_ERR_NULL;
    if (!aligned(ws[i], 16) || !aligned(scales[i], 2)) return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_quant_batched(count, ws, N, K, G, packeds, scales, nullptr, d_status,
                           (hipStream_t)stream, false);
  return finish_launch();
}

int tq_fake_quantize_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                             uint16_t *const *w_hats, uint16_t *const *scales,
                             int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!ws || !w_hats) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!ws[i] || !w_hats[i]) return TQ_ERR_NULL;
    if (!aligned(ws[i], 16) || !aligned(w_hats[i], 16)) return TQ_ERR_ALIGN;
    if (scales && !aligned(scales[i], 2)) return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_quant_batched(count, ws, N, K, G, nullptr, scales, w_hats, d_status,
                           (hipStream_t)stream, false);
  return finish_launch();
}

int tq_unpack_batched(int count, const uint8_t *const *packeds, int64_t N, int64_t K, int G,
                      int8_t *const *codes, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!packeds || !codes) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!packeds[i] || !codes[i]) return TQ_ERR_NULL;
    if (!aligned(codes[i], 8)) return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_unpack_batched(count, packeds, N, K, G, codes, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_unpack(const uint8_t *packed, int64_t N, int64_t K, int G, int8_t *codes,
              int32_t *d_status, void *stream) {
  if (!packed || !codes) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(codes, 8) || !aligned(d_status, 4)) return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_unpack(packed, N, K, G, codes, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_dequantize(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K, int G,
                  uint16_t *w_hat, int32_t *d_status, void *stream) {
  if (!packed || !scales || !w_hat) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(w_hat, 16) || !aligned(scales, 2) || !aligned(d_status, 4)) return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_dequantize(packed, scales, N, K, G, w_hat, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_dequantize_batched(int count, const uint8_t *const *packeds,
                          const uint16_t *const *scales, uint16_t *const *w_hats, int64_t N,
                          int64_t K, int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!packeds || !scales || !w_hats) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!packeds[i] || !scales[i] || !w_hats[i]) return TQ_ERR_NULL;
    if (!aligned(scales[i], 2) || !aligned(w_hats[i], 16)) return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_dequantize_batched(count, packeds, scales, w_hats, N, K, G, d_status,
                                (hipStream_t)stream);
  return finish_launch();
}

int tq_quantize_pack2(const uint16_t *w, int64_t N, int64_t K, int G, uint8_t *packed,
                      uint16_t *scales, int32_t *d_status, void *stream) {
  if (!w || !packed || !scales) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(w, 16) || !aligned(packed, 2) || !aligned(scales, 2) || !aligned(d_status, 4))
    return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_quant_batched(1, &w, N, K, G, &packed, &scales, nullptr, d_status,
                           (hipStream_t)stream, true);
  return finish_launch();
}

int tq_quantize_pack2_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                              uint8_t *const *packeds, uint16_t *const *scales,
                              int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!ws || !packeds || !scales) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!ws[i] || !packeds[i] || !scales[i]) return TQ_ERR_NULL;
    if (!aligned(ws[i], 16) || !aligned(packeds[i], 2) || !aligned(scales[i], 2))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_quant_batched(count, ws, N, K, G, packeds, scales, nullptr, d_status,
                           (hipStream_t)stream, true);
  return finish_launch();
}

int tq_unpack2(const uint8_t *packed, int64_t N, int64_t K, int G, int8_t *codes,
               int32_t *d_status, void *stream) {
  if (!packed || !codes) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (!aligned(packed, 4) || !aligned(codes, 16) || !aligned(d_status, 4)) return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_unpack2(packed, N, K, G, codes, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_gemv2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                     const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                     int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  const bool table = tq::gemv2_supported(N, K, G);
  if (!table && !tq::matmul2_supported(1, N, K, G)) return TQ_ERR_SHAPE;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], 16) || !aligned(scales[i], 2) ||
        !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  if (table)
    tq::launch_gemv2_batched(count, xs, packeds, scales, ys, N, K, G, d_status,
                             (hipStream_t)stream);
  else  // rows longer than the table kernel takes: the matrix-core kernel
    tq::launch_matmul2_batched(count, xs, packeds, scales, ys, 1, N, K, G, d_status,
                               (hipStream_t)stream);
  return finish_launch();
}

int tq_gemv2_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                     const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                     const int64_t *Ks, int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys || !Ns || !Ks) return TQ_ERR_NULL;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    const int rc = check_nkg(Ns[i], Ks[i], G);
    if (rc) return rc;
    if (!tq::gemv2_supported(Ns[i], Ks[i], G) && !tq::matmul2_supported(1, Ns[i], Ks[i], G))
      return TQ_ERR_SHAPE;
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], 16) || !aligned(scales[i], 2) ||
        !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  // the shapes the table kernel takes share launches; longer rows run alone
  // on the matrix-core kernel
  std::vector<const uint16_t *> gx, gs;
  std::vector<const uint8_t *> gp;
  std::vector<float *> gy;
  std::vector<int64_t> gn, gk;
  for (int i = 0; i < count; ++i) {
    if (tq::gemv2_supported(Ns[i], Ks[i], G)) {
      gx.push_back(xs[i]); gp.push_back(packeds[i]); gs.push_back(scales[i]);
      gy.push_back(ys[i]); gn.push_back(Ns[i]); gk.push_back(Ks[i]);
    } else {
      tq::launch_matmul2_batched(1, &xs[i], &packeds[i], &scales[i], &ys[i], 1, Ns[i], Ks[i], G,
                                 d_status, (hipStream_t)stream);
    }
  }
  if (!gx.empty())
    tq::launch_gemv2_grouped((int)gx.size(), gx.data(), gp.data(), gs.data(), gy.data(),
                             gn.data(), gk.data(), G, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_gemv2(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t N,
             int64_t K, int G, float *y, int32_t *d_status, void *stream) {
  return tq_gemv2_batched(1, &x, &packed, &scales, &y, N, K, G, d_status, stream);
}

int tq_gemm2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                     const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                     int64_t K, int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || !tq::matmul2_supported(M, N, K, G)) return TQ_ERR_SHAPE;
  const bool table = M == 1 && tq::gemv2_supported(N, K, G);
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], table ? 16 : 2) || !aligned(scales[i], 2) ||
        !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  if (table)
    tq::launch_gemv2_batched(count, xs, packeds, scales, ys, N, K, G, d_status,
                             (hipStream_t)stream);
  else
    tq::launch_matmul2_batched(count, xs, packeds, scales, ys, M, N, K, G, d_status,
                               (hipStream_t)stream);
  return finish_launch();
}

int tq_gemm2(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
             int64_t N, int64_t K, int G, float *y, int32_t *d_status, void *stream) {
  return tq_gemm2_batched(1, &x, &packed, &scales, &y, M, N, K, G, d_status, stream);
}

int tq_w4a16_gemv_batched(int count, const uint16_t *const *xs, const uint32_t *const *packeds,
                          const uint16_t *const *scales, const uint16_t *const *biases,
                          uint16_t *const *ys, int64_t N, int64_t K, int G, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !biases || !ys) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  const bool table = tq::w4a16_gemv_supported(N, K, G);
  if (!table && !tq::w4a16_mfma_supported(1, N, K, G)) return TQ_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !biases[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], 16) || !aligned(scales[i], 2) ||
        !aligned(biases[i], 2) || !aligned(ys[i], 2))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  if (table) {
    tq::launch_w4a16_gemv_batched(count, xs, packeds, scales, biases, ys, N, K, G,
                                  (hipStream_t)stream);
  } else {
    // rows longer than the table kernel takes (K > 4096): the matrix-core
    // kernel, one launch per 64 problems
    tq::launch_w4a16_mfma_batched(count, xs, packeds, scales, biases, 1, N, K, G, ys,
                                  (hipStream_t)stream);
  }
  return finish_launch();
}

int tq_w4a16_gemv_grouped(int count, const uint16_t *const *xs, const uint32_t *const *packeds,
                          const uint16_t *const *scales, const uint16_t *const *biases,
                          uint16_t *const *ys, const int64_t *Ns, const int64_t *Ks, int G,
                          void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !biases || !ys || !Ns || !Ks) return TQ_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    const int rc = check_nkg(Ns[i], Ks[i], G);
    if (rc) return rc;
    if (!tq::w4a16_gemv_supported(Ns[i], Ks[i], G) &&
        !tq::w4a16_mfma_supported(1, Ns[i], Ks[i], G))
      return TQ_ERR_SHAPE;
    if (!xs[i] || !packeds[i] || !scales[i] || !biases[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], 16) || !aligned(scales[i], 2) ||
        !aligned(biases[i], 2) || !aligned(ys[i], 2))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  // the shapes the table kernel takes share launches; longer rows run alone
  // on the matrix-core kernel
  std::vector<const uint16_t *> gx, gs, gb;
  std::vector<const uint32_t *> gp;
  std::vector<uint16_t *> gy;
  std::vector<int64_t> gn, gk;
  for (int i = 0; i < count; ++i) {
    if (tq::w4a16_gemv_supported(Ns[i], Ks[i], G)) {
      gx.push_back(xs[i]); gp.push_back(packeds[i]); gs.push_back(scales[i]);
      gb.push_back(biases[i]); gy.push_back(ys[i]); gn.push_back(Ns[i]); gk.push_back(Ks[i]);
    } else {
      tq::launch_w4a16_mfma(xs[i], packeds[i], scales[i], biases[i], 1, Ns[i], Ks[i], G, ys[i],
                            (hipStream_t)stream);
    }
  }
  if (!gx.empty())
    tq::launch_w4a16_gemv_grouped((int)gx.size(), gx.data(), gp.data(), gs.data(), gb.data(),
                                  gy.data(), gn.data(), gk.data(), G, (hipStream_t)stream);
  return finish_launch();
}

int tq_w4a16_gemm(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                  const uint16_t *biases, int64_t M, int64_t N, int64_t K, int G, uint16_t *y,
                  void *stream) {
  if (!x || !packed || !scales || !biases || !y) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || !tq::w4a16_mfma_supported(M, N, K, G)) return TQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 4) || !aligned(scales, 2) || !aligned(biases, 2) ||
      !aligned(y, 2))
    return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  if (M == 1 && tq::w4a16_gemv_supported(N, K, G) && aligned(packed, 16))
    tq::launch_w4a16_gemv_batched(1, &x, &packed, &scales, &biases, &y, N, K, G,
                                  (hipStream_t)stream);
  else
    tq::launch_w4a16_mfma(x, packed, scales, biases, M, N, K, G, y, (hipStream_t)stream);
  return finish_launch();
}

int tq_w4a16_gemm_batched(int count, const uint16_t *const *xs, const uint32_t *const *packeds,
                          const uint16_t *const *scales, const uint16_t *const *biases,
                          int64_t M, int64_t N, int64_t K, int G, uint16_t *const *ys,
                          void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !biases || !ys) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || !tq::w4a16_mfma_supported(M, N, K, G)) return TQ_ERR_SHAPE;
  const bool table = M == 1 && tq::w4a16_gemv_supported(N, K, G);
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !biases[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], table ? 16 : 4) || !aligned(scales[i], 2) ||
        !aligned(biases[i], 2) || !aligned(ys[i], 2))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  if (table)
    tq::launch_w4a16_gemv_batched(count, xs, packeds, scales, biases, ys, N, K, G,
                                  (hipStream_t)stream);
  else
    tq::launch_w4a16_mfma_batched(count, xs, packeds, scales, biases, M, N, K, G, ys,
                                  (hipStream_t)stream);
  return finish_launch();
}

int tq_w4a16_gemv(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                  const uint16_t *biases, int64_t N, int64_t K, int G, uint16_t *y,
                  void *stream) {
  return tq_w4a16_gemv_batched(1, &x, &packed, &scales, &biases, &y, N, K, G, stream);
}

int tq_gemv(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
            int64_t N, int64_t K, int G, float *y, int32_t *d_status, void *stream) {
  if (!x || !packed || !scales || !y) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || M > 16) return TQ_ERR_SHAPE;
  if (K > (int64_t(1) << 22)) return TQ_ERR_SHAPE;  // 32-bit offsets into x
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(y, 4) ||
      !aligned(d_status, 4))
    return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_gemv(x, packed, scales, M, N, K, G, y, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_gemv_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                    int64_t K, int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || M > 16) return TQ_ERR_SHAPE;
  if (K > (int64_t(1) << 22)) return TQ_ERR_SHAPE;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], 16) || !aligned(scales[i], 2) ||
        !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_gemv_batched(count, xs, packeds, scales, ys, M, N, K, G, d_status,
                          (hipStream_t)stream);
  return finish_launch();
}

int tq_gemv_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                    const int64_t *Ks, int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys || !Ns || !Ks) return TQ_ERR_NULL;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    const int rc = check_nkg(Ns[i], Ks[i], G);
    if (rc) return rc;
    if (Ks[i] > (int64_t(1) << 22)) return TQ_ERR_SHAPE;
    if (!aligned(xs[i], 16) || !aligned(packeds[i], 16) || !aligned(scales[i], 2) ||
        !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  // the shapes the M = 1 kernel takes share launches; any other goes alone
  std::vector<const uint16_t *> gx, gs;
  std::vector<const uint8_t *> gp;
  std::vector<float *> gy;
  std::vector<int64_t> gn, gk;
  for (int i = 0; i < count; ++i) {
    if (tq::gemv_m1_supported(1, Ns[i], Ks[i])) {
      gx.push_back(xs[i]); gp.push_back(packeds[i]); gs.push_back(scales[i]); gy.push_back(ys[i]);
      gn.push_back(Ns[i]); gk.push_back(Ks[i]);
    } else {
      tq::launch_gemv(xs[i], packeds[i], scales[i], 1, Ns[i], Ks[i], G, ys[i], d_status,
                      (hipStream_t)stream);
    }
  }
  if (!gx.empty())
    tq::launch_gemv_m1_grouped((int)gx.size(), gx.data(), gp.data(), gs.data(), gy.data(),
                               gn.data(), gk.data(), G, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_gemm(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
            int64_t N, int64_t K, int G, float *y, int32_t *d_status, void *stream) {
  if (!x || !packed || !scales || !y) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || M > (int64_t(1) << 40) / K) return TQ_ERR_SHAPE;
  if (K > (int64_t(1) << 22)) return TQ_ERR_SHAPE;  // a 128-row x slab stays under 1 GiB
  if (!aligned(x, 16) || !aligned(scales, 2) || !aligned(y, 4) || !aligned(d_status, 4))
    return TQ_ERR_ALIGN;
  (void)hipGetLastError();
  tq::launch_gemm(x, packed, scales, M, N, K, G, y, d_status, (hipStream_t)stream);
  return finish_launch();
}

int tq_gemm_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                    int64_t K, int G, int32_t *d_status, void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys) return TQ_ERR_NULL;
  const int rc = check_nkg(N, K, G);
  if (rc) return rc;
  if (M < 1 || M > (int64_t(1) << 40) / K) return TQ_ERR_SHAPE;
  if (K > (int64_t(1) << 22)) return TQ_ERR_SHAPE;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    if (!aligned(xs[i], 16) || !aligned(scales[i], 2) || !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_gemm_batched(count, xs, packeds, scales, ys, M, N, K, G, d_status,
                          (hipStream_t)stream);
  return finish_launch();
}

int tq_gemm_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys, int64_t M,
                    const int64_t *Ns, const int64_t *Ks, int G, int32_t *d_status,
                    void *stream) {
  if (count < 0) return TQ_ERR_SHAPE;
  if (count == 0) return TQ_OK;
  if (!xs || !packeds || !scales || !ys || !Ns || !Ks) return TQ_ERR_NULL;
  if (!aligned(d_status, 4)) return TQ_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !packeds[i] || !scales[i] || !ys[i]) return TQ_ERR_NULL;
    const int rc = check_nkg(Ns[i], Ks[i], G);
    if (rc) return rc;
    if (M < 1 || M > (int64_t(1) << 40) / Ks[i]) return TQ_ERR_SHAPE;
    if (Ks[i] > (int64_t(1) << 22)) return TQ_ERR_SHAPE;
    if (!aligned(xs[i], 16) || !aligned(scales[i], 2) || !aligned(ys[i], 4))
      return TQ_ERR_ALIGN;
  }
  (void)hipGetLastError();
  tq::launch_gemm_grouped(count, xs, packeds, scales, ys, M, Ns, Ks, G, d_status,
                          (hipStream_t)stream);
  return finish_launch();
}

}  // extern "C"
