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
typedef float v2f32 __attribute__((ext_vector_type(2)));

// two fp32 -> two fp16, nearest even, in one instruction (v_cvt_pk_f16_f32)
__device__ __forceinline__ v2h cvt2_f16(float a, float b) { return __builtin_convertvector((v2f32){a, b}, v2h); }
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
// fp16 normal range; smaller magnitudes round to fp16 subnormals. Pairs go
// through one packed fp32 -> fp16 conversion each.
__device__ __forceinline__ v8h bf16x8_to_f16x8(uint4 w) {
  v8h r;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2h h = cvt2_f16(__uint_as_float(ws[i] << 16), __uint_as_float(ws[i] & 0xFFFF0000u));
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

__device__ __forceinline__ v8h f16x8_from_u4(uint4 w) { return __builtin_bit_cast(v8h, w); }

// 8 int8 codes (one 8-byte load) -> 8 fp16 operands (exact). Each code c is
// biased to the byte c + 128 and placed under the fp16 exponent of 1024, which
// gives the fp16 value 1152 + c exactly; one packed fp16 subtraction of 1152
// per pair then leaves c.
__device__ __forceinline__ v8h i8x8_to_f16x8(uint2 w) {
  v8h r;
  const uint32_t ws[2] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u};
  const v2h bias = (v2h){(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // bytes [u0, 0x64, u1, 0x64] and [u2, 0x64, u3, 0x64]
    const v2h lo = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, ws[i], 0x04010400u)) - bias;
    const v2h hi = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, ws[i], 0x04030402u)) - bias;
    r[4 * i + 0] = lo[0];
    r[4 * i + 1] = lo[1];
    r[4 * i + 2] = hi[0];
    r[4 * i + 3] = hi[1];
  }
  return r;
}

// ---- wave reductions (wave64) ----------------------------------------------

// A lane's view of another lane of its 16-lane row through a DPP operand
// (no LDS traffic): 0xB1 / 0x4E are the quad permutations [1,0,3,2] and
// [2,3,0,1] (lanes l^1 and l^2), 0x124 / 0x128 rotate the row by 4 and 8.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// max / sum over the 16 lanes of each row (lanes 16r .. 16r+15): quad
// exchanges, then the row rotated by 4 and by 8. Every lane ends with the
// row's result (a sum in an order that depends on the lane, fixed per lane).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  return fmaxf(v, dpp_f<0x128>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x124>(v);
  return v + dpp_f<0x128>(v);
}

__device__ __forceinline__ float group4_max(float v);
__device__ __forceinline__ float group4_sum(float v);

// max / sum over the whole wave: rows of 16, then the four rows
__device__ __forceinline__ float wave_max(float v) { return group4_max(row16_max(v)); }
__device__ __forceinline__ float wave_sum(float v) { return group4_sum(row16_sum(v)); }

// max / sum across the four 16-lane groups (lanes l, l^16, l^32, l^48).
// v_permlane16_swap / v_permlane32_swap with both operands equal to v leave
// the value of lane l^16 (resp. l^32) in one of the two results and v itself
// in the other (lane layout checked on gfx950), so each step is two VALU
// operations and no LDS traffic.
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

// Rotary embedding of the E channels ch .. ch+E-1 of one row (values in v,
// the row's 16-bit inputs at `row`) by table row cs (cos(p w_i) at i, sin at
// rot/2 + i). neox pairs channel c with c +- rot/2, otherwise with c ^ 1;
// channels from rot on are left alone. Each output is
// fl32(fl32(x cos) -+ fl32(y sin)), y the pair partner: no fused multiply-add,
// so the rotated values (and the codes taken from them) do not depend on
// the compiler's contraction choices.
template <int E, bool BF16>
__device__ __forceinline__ void rope_lane(const uint16_t* __restrict__ row, int ch, float (&v)[E],
                                          const float* __restrict__ cs, int rot, bool neox) {
#pragma clang fp contract(off)
  const int half = rot >> 1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = ch + e;
    if (c >= rot) continue;
    const bool first = neox ? c < half : (c & 1) == 0;
    const int i = neox ? (first ? c : c - half) : c >> 1;
    const int pc = neox ? (first ? c + half : c - half) : c ^ 1;
    const float y = half_to_f32<BF16>(row[pc]);
    const float xc = v[e] * cs[i];
    const float ys = y * cs[half + i];
    v[e] = first ? xc - ys : xc + ys;
  }
}

// LDS byte address of a __shared__ object (a constant: no generic-pointer
// null check at run time).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One lane's 16 bytes global -> LDS (global_load_lds_dwordx4): the wave's
// 64 lanes fill the 1 KB at the wave-uniform LDS address `lds`. Issued as
// inline assembly, so the compiler does not treat the LDS destination as
// aliasing the reads of the other buffer; the caller waits (vmcnt) before
// the barrier. GFX9 parts need one wait state between an SALU write of M0
// and an LDS-DMA instruction that reads it: the s_nop provides it.
// The source is a wave-uniform base (scalar registers) plus each lane's own
// 32-bit offset (`voff`, 16 * lane for a 1 KB chunk), so the address math
// of a copy is scalar.
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  // the base is wave-uniform by contract; readfirstlane states it to the
  // compiler (free when it already sits in scalar registers)
  // (readfirstlane returns a signed int: each half is widened through
  // uint32_t, so the low half is not sign-extended into the high one)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t sb = (hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(sb)
               : "memory", "m0");
}

// Wait until every vector memory operation of the wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima, gfx9
// encoding). The builtin, unlike inline assembly, is seen by the compiler's
// wait insertion, which then knows that the loads issued before it (query
// fragments, scales) are complete and places no waits for them in the tile
// loop, where any vmcnt wait would also wait for the copies in flight.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace qa
