// bf16 hi/lo operand splitting for fp32-accurate products on the bf16 MFMA.
#pragma once

#include "device_common.hpp"

namespace msq {

// Eight fp32 values -> hi and lo bf16 MFMA operands, hi = rne(v), lo = rne(v - hi), so
// hi + lo = v to ~2^-16 relative; products of the pairs are exact in fp32, so
// hi*hi + hi*lo + lo*hi carries ~fp32 accuracy on the MFMA.
__device__ __forceinline__ void split8_bf16(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    l[i] = pack_bf16x2(v[2 * i] - bf16_to_f32(h[i] & 0xffffu), v[2 * i + 1] - bf16_to_f32(h[i] >> 16));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

}  // namespace msq
