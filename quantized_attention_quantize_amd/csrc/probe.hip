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

template <int KIND>
__global__ __launch_bounds__(256) void k_mfma(int iters, float* sink) {
  const int l = threadIdx.x & 63;
  const v4i a = {l, l + 1, l + 2, l + 3}, b = {l * 3, l ^ 5, l + 7, l * 11};
  v8h ha, hb;
  for (int j = 0; j < 8; ++j) {
    ha[j] = (_Float16)(0.001f * (l + j));
    hb[j] = (_Float16)(0.002f * (l - j));
  }
  float r = 0.0f;
  if constexpr (KIND == 0) {
    v16i c[4];
    for (int k = 0; k < 4; ++k)
      for (int j = 0; j < 16; ++j) c[k][j] = 0;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k], 0, 0, 0);
    for (int k = 0; k < 4; ++k) r += (float)(c[k][0] + c[k][15]);
  } else if constexpr (KIND == 1) {
    v16f c[4];
    for (int k = 0; k < 4; ++k)
      for (int j = 0; j < 16; ++j) c[k][j] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, hb, c[k], 0, 0, 0);
    for (int k = 0; k < 4; ++k) r += c[k][0] + c[k][15];
  } else if constexpr (KIND == 2) {
    v4i c[8];
    for (int k = 0; k < 8; ++k) c[k] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[k], 0, 0, 0);
    for (int k = 0; k < 8; ++k) r += (float)(c[k][0] + c[k][3]);
  } else {
    v4f c[8];
    for (int k = 0; k < 8; ++k) c[k] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, c[k], 0, 0, 0);
    for (int k = 0; k < 8; ++k) r += c[k][0] + c[k][3];
  }
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
  if (sink == nullptr || kind < 0 || kind > 3 || iters < 1 || wgs < 1 || wgs > 65535) return 1;
  switch (kind) {
    case 0: k_mfma<0><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 1: k_mfma<1><<<wgs, 256, 0, stream>>>(iters, sink); break;
    case 2: k_mfma<2><<<wgs, 256, 0, stream>>>(iters, sink); break;
    default: k_mfma<3><<<wgs, 256, 0, stream>>>(iters, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int qa_probe_valu(int kind, int iters, int wgs, float* sink, hipStream_t stream) {
  if (sink == nullptr || kind < 0 || kind > 1 || iters < 1 || wgs < 1 || wgs > 65535) return 1;
  if (kind == 0) k_valu<0><<<wgs, 256, 0, stream>>>(iters, sink);
  else k_valu<1><<<wgs, 256, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
