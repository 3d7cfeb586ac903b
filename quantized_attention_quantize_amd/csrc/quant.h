// Block and row quantization codes shared by the quantizers and the dense
// attention kernel (which quantizes its own query block).
#pragma once

#include "common.h"

namespace qa {

// The codes of N values of one block or row against its scale s (amax = the
// largest |x| of the block, s = quant_scale(amax)), packed as bytes into
// ceil(N/4) words, the same codes as quant_code. For amax > 0 and rs =
// fl32(1/s) finite and below 3e38 there is no division per value: |x/s| <=
// 127 needs no clamp, and y = fl32(x * rs) lies within 1.5 * 2^-23 * |x/s|
// <= 2.3e-5 of fl32(x / s), so the nearest integer to y is the code unless y
// is within 6.1e-5 of a half-integer; such values take the exact quotient
// (one test per N values, then one branch per value). Adding
// 1.5 * 2^23 rounds to the nearest integer (ties to even) and leaves the
// code in the low byte of the float's bits. amax = 0 gives zero codes.
template <int N>
__device__ __forceinline__ void quant_bytes(const float (&x)[N], float amax, float s, float rs,
                                            uint32_t (&w)[(N + 3) / 4]) {
#pragma clang fp contract(off)
  constexpr float kM = 12582912.0f;   // 1.5 * 2^23
  float t[N];
  if (amax > 0.0f && rs <= 3.0e38f) {
    bool bad = false, near[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float y = x[i] * rs;
      t[i] = y + kM;
      near[i] = fabsf(y - (t[i] - kM)) > 0.49993896484375f;
      bad |= near[i];
    }
    if (bad) {
      // only the values near a half-integer take the exact quotient (with
      // 16-bit inputs such near-ties are common enough that most waves see
      // one, but few lanes share the same value index)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (near[i]) t[i] = rintf(__fdiv_rn(x[i], s)) + kM;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = (float)(amax > 0.0f ? quant_code(x[i], s) : 0) + kM;
  }
  if constexpr (N % 4 == 0) {
    // byte permutes: the low bytes of two values side by side (the upper
    // half zero), then two such halves into one word
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t[4 * q + 1]), __float_as_uint(t[4 * q]), 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t[4 * q + 3]), __float_as_uint(t[4 * q + 2]), 0x0c0c0400u);
      w[q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  } else {
#pragma unroll
    for (int q = 0; q < (N + 3) / 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < N) v |= (__float_as_uint(t[4 * q + i]) & 0xFFu) << (8 * i);
      w[q] = v;
    }
  }
}

}  // namespace qa
