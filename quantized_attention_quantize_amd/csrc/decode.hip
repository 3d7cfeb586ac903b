// Paged decode attention: INT8 Q x INT8 paged K (INT32 accumulation), score
// recovery per element, online softmax in base 2, fp16 P.V with fp32
// accumulation, split-K partials and their combine.
//
// Mapping onto v_mfma_i32_16x16x64_i8 (see common.h for the lane layout).
// The kernel computes S^T = K Q^T per 32-token tile:
//   A operand = 16 key tokens x 64 channels (INT8, straight from the cache)
//   B operand = 64 channels x 16 query heads (the G heads of one KV head,
//               [QK-MMAC] §5.1; columns >= G are zero)
// A tile covers 32 tokens with two instructions u = 0, 1; matrix row r of
// instruction u holds token 8*(r/4) + 4u + (r%4). With that permutation the
// result lane l (column = head l%16, group g = l/16) owns tokens
// 8g .. 8g+7 of the tile, which is exactly the K-slice lane l must supply as
// the B operand of the fp16 product O^T = V^T P^T. So P never leaves the
// registers, and the per-token key scale ([QK-MMAC] §1, "per column" of S)
// is read as 8 consecutive floats that follow the result layout.
#include "common.h"
#include "internal.h"

namespace qa {
namespace {

constexpr int kWaves = 4;

template <int D, bool V_I8, bool EXPORT_QK>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
  constexpr int KS = D / 64;   // INT8 K-steps
  constexpr int CG = D / 16;   // 16-channel groups of the output
  extern __shared__ float smem[];

  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int G = a.G, Hq = a.Hq, Hkv = a.Hkv, S = a.num_splits;

  const int ctx = a.ctx_lens[seq];
  const int nblk = (ctx + 15) >> 4;
  const int per = (nblk + S - 1) / S;
  const int t0 = min(split * per * 16, ctx);
  const int t1 = min(t0 + per * 16, ctx);
  const int ntiles = (t1 - t0 + 31) >> 5;

  // Query fragments (B operand): head n of this KV group, channels 64s+16g..+15.
  const int h = kvh * G + n;
  const bool live_col = n < G;
  v4i qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (live_col)
      qf[s] = *reinterpret_cast<const v4i*>(a.q + ((int64_t)seq * Hq + h) * D + 64 * s + 16 * g);
    else
      qf[s] = v4i{0, 0, 0, 0};
  }
  const float qsc = live_col ? a.q_scale[(int64_t)seq * Hq + h] * a.scale_log2 : 0.0f;

  float m_run = kNegInf, l_run = 0.0f;
  v4f O[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) O[c] = v4f{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  // token of matrix row n in instruction u, relative to the tile start
  const int tau0 = 8 * (n >> 2) + (n & 3);

  for (int tile = wave; tile < ntiles; tile += kWaves) {
    const int tb = t0 + tile * 32;
    const int lb = tb >> 4;
    const int p0 = trow[lb];
    const int p1 = (tb + 16 < t1) ? trow[lb + 1] : p0;

    v4i acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tau = tau0 + 4 * u;
      const int pb = tau >= 16 ? p1 : p0;
      const int8_t* kb = a.k_cache + ((int64_t)pb * Hkv + kvh) * (D / 16) * 256 + (tau & 15) * 16;
      acc[u] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        v4i kf = *reinterpret_cast<const v4i*>(kb + (4 * s + g) * 256);
        acc[u] = mfma_i8(kf, qf[s], acc[u]);
      }
    }

    if constexpr (EXPORT_QK) {
      if (live_col) {
        int32_t* dst = a.acc_out + ((int64_t)seq * Hq + h) * (int64_t)a.max_blocks * 16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = tb + 8 * g + j;
          if (t < t1) dst[t] = acc[j >> 2][j & 3];
        }
      }
      continue;
    }

    // Tokens 8g .. 8g+7 of the tile live in one block at slots so .. so+7.
    const int pbs = g >= 2 ? p1 : p0;
    const int so = 8 * (g & 1);
    const int64_t sidx = ((int64_t)pbs * Hkv + kvh) * 16 + so;
    const float4 ska = *reinterpret_cast<const float4*>(a.k_scale + sidx);
    const float4 skb = *reinterpret_cast<const float4*>(a.k_scale + sidx + 4);
    const float sk[8] = {ska.x, ska.y, ska.z, ska.w, skb.x, skb.y, skb.z, skb.w};
    const int tl = tb + 8 * g;   // first token of this lane's slice

    // [QK-MMAC] §1: recover each score before the softmax (base-2 units).
    float sc[8];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = (float)acc[j >> 2][j & 3] * qsc * sk[j];
      sc[j] = (tl + j < t1) ? v : kNegInf;
      mt = fmaxf(mt, sc[j]);
    }
    mt = group4_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float mref = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - mref);
    float p[8], psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(sc[j] - mref);
      psum += p[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    v8h pf;
    if constexpr (V_I8) {
      // fold the per-token V scale into P: sum_t p_t (code_t * sV_t) v-code
      const float4 sva = *reinterpret_cast<const float4*>(a.v_scale + sidx);
      const float4 svb = *reinterpret_cast<const float4*>(a.v_scale + sidx + 4);
      const float sv[8] = {sva.x, sva.y, sva.z, sva.w, svb.x, svb.y, svb.z, svb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (_Float16)((tl + j < t1) ? p[j] * sv[j] : 0.0f);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (_Float16)p[j];
    }

#pragma unroll
    for (int c = 0; c < CG; ++c) O[c] *= alpha;

    // V^T operand: channel 16c+n, tokens 8g..8g+7 of the tile.
    const bool full = tl + 8 <= t1;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int64_t vrow = (((int64_t)pbs * Hkv + kvh) * D + 16 * c + n) * 16 + so;
      v8h vf;
      if constexpr (V_I8) {
        vf = i8x8_to_f16x8(*reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(a.v_cache) + vrow));
      } else {
        vf = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v_cache) + vrow));
      }
      if (!full) {
        // slots past the context may hold anything (even NaN): zero them
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (tl + j >= t1) vf[j] = (_Float16)0.0f;
      }
      O[c] = mfma_f16(vf, pf, O[c]);
    }
  }
  if constexpr (EXPORT_QK) return;

  // ---- merge the waves of this workgroup ----------------------------------
  l_run = group4_sum(l_run);
  float* sm_ml = smem;                       // [kWaves][16][2]
  float* sm_o = smem + kWaves * 32;          // [kWaves][G][D]
  if (g == 0) {
    sm_ml[(wave * 16 + n) * 2] = m_run;
    sm_ml[(wave * 16 + n) * 2 + 1] = l_run;
  }
  if (live_col) {
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[((int64_t)wave * G + n) * D + 16 * c + 4 * g + i] = O[c][i];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int hn = idx / D, ch = idx - hn * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[(w * 16 + hn) * 2]);
    float lsum = 0.0f, o = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(sm_ml[(w * 16 + hn) * 2] - M);
        lsum += wt * sm_ml[(w * 16 + hn) * 2 + 1];
        o += wt * sm_o[((int64_t)w * G + hn) * D + ch];
      }
    }
    const int hh = kvh * G + hn;
    if (S == 1) {
      const float r = lsum > 0.0f ? o / lsum : 0.0f;
      const int64_t oi = ((int64_t)seq * Hq + hh) * D + ch;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(r);
      else reinterpret_cast<float*>(a.out)[oi] = r;
    } else {
      const int64_t pi = ((int64_t)seq * Hq + hh) * S + split;
      a.ws_o[pi * D + ch] = o;
      if (ch == 0) {
        a.ws_ml[pi * 2] = M;
        a.ws_ml[pi * 2 + 1] = lsum;
      }
    }
  }
}

// One workgroup of D threads per (query head, sequence): merges S partials.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ws_o,
                                                 const float* __restrict__ ws_ml, int32_t Hq,
                                                 int32_t D, int32_t S, bool out_bf16, void* out) {
  const int h = blockIdx.x, seq = blockIdx.y, ch = threadIdx.x;
  const int64_t base = ((int64_t)seq * Hq + h) * S;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ws_ml[(base + s) * 2]);
  float lsum = 0.0f, o = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float m = ws_ml[(base + s) * 2];
      const float wt = fast_exp2(m - M);
      lsum += wt * ws_ml[(base + s) * 2 + 1];
      o += wt * ws_o[(base + s) * D + ch];
    }
  }
  const float r = lsum > 0.0f ? o / lsum : 0.0f;
  const int64_t oi = ((int64_t)seq * Hq + h) * D + ch;
  if (out_bf16) reinterpret_cast<uint16_t*>(out)[oi] = (uint16_t)f32_to_bf16_bits(r);
  else reinterpret_cast<float*>(out)[oi] = r;
}

template <int D, bool V_I8, bool EXPORT_QK>
hipError_t run_decode(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.num_splits, a.Hkv, a.num_seqs);
  const size_t lds = EXPORT_QK ? 0 : (size_t)(kWaves * 32 + kWaves * a.G * D) * sizeof(float);
  auto kern = k_decode<D, V_I8, EXPORT_QK>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<grid, 256, lds, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || EXPORT_QK || a.num_splits == 1) return e;
  k_combine<<<dim3(a.Hq, a.num_seqs), D, 0, st>>>(a.ws_o, a.ws_ml, a.Hq, D, a.num_splits, a.out_bf16, a.out);
  return hipGetLastError();
}

template <bool EXPORT_QK>
hipError_t dispatch(const DecodeArgs& a, hipStream_t st) {
#define QA_DEC(DD)                                                          \
  return a.v_int8 ? run_decode<DD, true, EXPORT_QK>(a, st) : run_decode<DD, false, EXPORT_QK>(a, st)
  switch (a.D) {
    case 64: QA_DEC(64);
    case 128: QA_DEC(128);
    default: QA_DEC(256);
  }
#undef QA_DEC
}

}  // namespace

int32_t choose_decode_splits(int32_t num_seqs, int32_t Hkv, int32_t max_blocks) {
  // Aim for about two workgroups per compute unit (256 CUs), but keep at
  // least 8 blocks (128 tokens, one 32-token tile per wave) per segment.
  const int64_t units = (int64_t)num_seqs * Hkv;
  int64_t s = (512 + units - 1) / units;
  const int64_t cap = max_blocks / 8 > 0 ? max_blocks / 8 : 1;
  if (s > cap) s = cap;
  if (s > 256) s = 256;
  return (int32_t)(s < 1 ? 1 : s);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) { return dispatch<false>(a, st); }

hipError_t launch_debug_qk(const DecodeArgs& a, hipStream_t st) {
  DecodeArgs b = a;
  b.num_splits = 1;
  return dispatch<true>(b, st);
}

}  // namespace qa
