// tq_digits.h -- device helpers shared by the kernels that read packed
// bytes digit by digit (tq_dequant.hip, tq_quant.hip).
//
// Format: precisit "pack-unpack-run" README, codec.py description: five
// base-3 digits d = c + 1 per byte, the first weight least significant;
// byte values 243..255 are invalid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr uint32_t kLutInvalid = 1u << 31;

// Table entry of byte v: its five base-3 digits as 2-bit fields (digit i at
// bits 2i).  An invalid byte reads as five digits 1 (code 0) and carries
// kLutInvalid.
__device__ __forceinline__ uint32_t digit_entry(uint32_t v) {
  if (v >= 243u) return 0x155u | kLutInvalid;
  uint32_t e = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    e |= (v % 3u) << (2 * i);
    v /= 3u;
  }
  return e;
}

}  // namespace tq
