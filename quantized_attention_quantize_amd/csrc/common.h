// Device-side building blocks shared by the gfx950 kernels.
//
// Matrix-instruction lane layout (wave64, checked on gfx950 with one-hot and
// random operands): for v_mfma_i32_16x16x64_i8 and v_mfma_f32_16x16x32_f16,
// lane l supplies row (l % 16) of A and column (l % 16) of B, each with the
// K-slice [kw*(l/16), kw*(l/16) + kw) (kw = 16 int8 or 8 fp16 values), and
// receives C[4*(l/16) + i][l % 16] for i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// p ~= hi + lo with hi = bf16(p) and lo = bf16(p - hi): a two-term bf16
// expansion with relative error near 2^-16, so a bf16 matrix product of
// (hi, lo) against bf16 data keeps about fp32-level accuracy for P.
__device__ __forceinline__ void split_bf16x8(const float (&p)[8], v8bf& hi, v8bf& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hi[j] = (__bf16)p[j];
    lo[j] = (__bf16)(p[j] - (float)hi[j]);
  }
}

// ---- 16-bit storage formats -------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

template <bool BF16>
__device__ __forceinline__ float half_to_f32(uint32_t bits16) {
  return BF16 ? bf16_to_f32(bits16) : f16_to_f32(bits16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// 8 packed bf16 (one 16-byte load) -> 8 fp16 operands. Exact for |v| in the
// fp16 normal range; smaller magnitudes round to fp16 subnormals.
__device__ __forceinline__ v8h bf16x8_to_f16x8(uint4 w) {
  v8h r;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)__uint_as_float(ws[i] << 16);
    r[2 * i + 1] = (_Float16)__uint_as_float(ws[i] & 0xFFFF0000u);
  }
  return r;
}

__device__ __forceinline__ v8h f16x8_from_u4(uint4 w) { return __builtin_bit_cast(v8h, w); }

// 8 int8 codes (one 8-byte load) -> 8 fp16 operands (exact).
__device__ __forceinline__ v8h i8x8_to_f16x8(uint2 w) {
  v8h r;
  const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int v = (int)(int8_t)((ws[i] >> (8 * b)) & 0xFF);
      r[4 * i + b] = (_Float16)v;
    }
  }
  return r;
}

// ---- wave reductions (wave64) ----------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// max / sum across the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- row quantization step ---------------------------------------------------
// code = clamp(rne(fl32(x / s)), -127, 127), s > 0; IEEE-correctly-rounded
// division (never a reciprocal multiply).
__device__ __forceinline__ int quant_code(float x, float s) {
  float r = rintf(__fdiv_rn(x, s));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ float quant_scale(float amax) { return __fdiv_rn(amax, 127.0f); }

}  // namespace qa
