// Measurement probes: a grid-stride streaming read, matrix-instruction
// throughput loops and vector-ALU loops (declared in qa_probe.h). Separate from the attention
// library; used to state the practical ceilings next to the kernels'
// throughputs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/qa_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_stream_read(const int4* __restrict__ p, size_t n, int* sink) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  int acc = 0;
  for (; i < n; i += stride) {
    const int4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one value per workgroup (thread 0's), written unconditionally
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

typedef int v8i __attribute__((ext_vector_type(8)));

// One matrix instruction of each measured form, on register operands.
template <int KIND>
struct Mfma;
template <>
struct Mfma<0> {   // v_mfma_i32_32x32x32_i8: 65536 ops
  typedef v16i C;
  static constexpr double kOps = 32.0 * 32 * 32 * 2;
  static __device__ C run(v4i a, v4i b, v8h, v8h, v8i, v8i, C c) { return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0); }
};
template <>
struct Mfma<1> {   // v_mfma_f32_32x32x16_f16: 32768 flops
  typedef v16f C;
  static __device__ C run(v4i, v4i, v8h a, v8h b, v8i, v8i, C c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};
template <>
struct Mfma<2> {   // v_mfma_i32_16x16x64_i8: 32768 ops
  typedef v4i C;
  static __device__ C run(v4i a, v4i b, v8h, v8h, v8i, v8i, C c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }
};
template <>
struct Mfma<3> {   // v_mfma_f32_16x16x32_f16: 16384 flops
  typedef v4f C;
  static __device__ C run(v4i, v4i, v8h a, v8h b, v8i, v8i, C c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
};
template <>
struct Mfma<4> {   // v_mfma_f32_32x32x64_f8f6f4, E4M3 operands (zero scales: unscaled): 131072 flops
  typedef v16f C;
  static __device__ C run(v4i, v4i, v8h, v8h, v8i a, v8i b, C c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// NACC independent accumulator chains per wave; every element of every
// accumulator feeds the value written at the end (an accumulator element
// left unread lets the compiler overlap and copy accumulator registers
// inside the loop, which then measures the copies).
template <int KIND, int NACC>
__global__ __launch_bounds__(256) void k_mfma(int iters, float* sink) {
  const int l = threadIdx.x & 63;
  const v4i a = {l, l + 1, l + 2, l + 3}, b = {l * 3, l ^ 5, l + 7, l * 11};
  v8h ha, hb;
  v8i fa, fb;
  for (int j = 0; j < 8; ++j) {
    ha[j] = (_Float16)(0.001f * (l + j));
    hb[j] = (_Float16)(0.002f * (l - j));
    fa[j] = 0x38383838 ^ (((l + j) & 7) * 0x01010101);       // E4M3 1.0 .. 1.875 (mantissa bits only)
    fb[j] = 0x30303030 ^ (((l * 7 + j) & 7) * 0x01010101);   // E4M3 0.5 .. 0.9375
  }
  typedef typename Mfma<KIND>::C C;
  C c[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k)
    for (int j = 0; j < (int)(sizeof(C) / 4); ++j) c[k][j] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) c[k] = Mfma<KIND>::run(a, b, ha, hb, fa, fb, c[k]);
  }
  float r = 0.0f;
#pragma unroll
  for (int k = 0; k < NACC; ++k)
    for (int j = 0; j < (int)(sizeof(C) / 4); ++j) r += (float)c[k][j];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

// 8 independent chains per lane of one vector operation: the base-2
// exponential (v_exp_f32, x -> 2^-x with the negation as a source modifier,
// so every value stays in (0.5, 1]) or the fused multiply-add (v_fma_f32,
// x -> 0.999 x + 1e-7).
template <int KIND>
__global__ __launch_bounds__(256) void k_valu(int iters, float* sink) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 1e-6f * (float)(threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      else x[i] = __builtin_fmaf(x[i], 0.999f, 1e-7f);
    }
  }
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += x[i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" int qa_probe_stream_read(const void* src, size_t bytes, int wgs, int* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes % 16 != 0 || wgs < 1 || wgs > 65535) return 1;
  if (bytes == 0) return 0;
  k_stream_read<<<wgs, 256, 0, stream>>>(static_cast<const int4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int qa_probe_mfma(int kind, int iters, int wgs, float* sink, hipStream_t stream) {
  if (sink == nullptr || kind < 0 || kind > 8 || iters < 1 || wgs < 1 || wgs > 65535) return 1;
  switch (kind) {
    case 0: k_mfma<0, 4><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 1: k_mfma<1, 4><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 2: k_mfma<2, 8><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 3: k_mfma<3, 8><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 4: k_mfma<2, 16><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 5: k_mfma<3, 16><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 6: k_mfma<2, 4><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 7: k_mfma<3, 4><<<wgs, 256, 0, stream>>>(iters, sink); break;
    default: k_mfma<4, 4><<<wgs, 256, 0, stream>>>(iters, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int qa_probe_valu(int kind, int iters, int wgs, float* sink, hipStream_t stream) {
  if (sink == nullptr || kind < 0 || kind > 1 || iters < 1 || wgs < 1 || wgs > 65535) return 1;
  if (kind == 0) k_valu<0><<<wgs, 256, 0, stream>>>(iters, sink);
  else k_valu<1><<<wgs, 256, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
