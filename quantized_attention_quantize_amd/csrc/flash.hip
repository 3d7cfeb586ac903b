// Chunked prefill over a paged history ([QK-MMAC] §5.2) and dense
// SageAttention-style forward ([SAGE-MACA] attention-kernel pipeline), one
// kernel template.
//
// Workgroup = 4 waves = 128 query rows of one query head. Each 64-token
// KV tile (4 blocks of 16) is staged in LDS and shared by the 4 waves.
// Matrix products are computed transposed, as in the decode kernel:
//   S^T = K Q^T   (v_mfma_i32_16x16x64_i8; A = 16 keys from LDS, B = 16 queries
//                  held in registers for the whole KV loop)
//   O^T += V^T P^T (v_mfma_f32_16x16x32_f16; A = 16 channels x 32 keys from LDS,
//                  B = P straight from the score registers)
// Key rows are permuted within each 32-token half so that every lane owns
// 8 consecutive keys of one query (see decode.hip).
//
// The dense path reads its K codes and V from the same 16-token block layout
// the cache uses, written by the preprocessing step, with block b*ceil(N/16) + t/16.
#include "common.h"
#include "internal.h"

namespace qa {
namespace {

constexpr int QT = 128;    // query rows per workgroup
constexpr int KT = 64;     // keys per LDS tile

enum VKind { kVBf16 = 0, kVF16 = 1, kVI8 = 2 };

template <int D, int VK, bool DENSE, bool CAUSAL>
__global__ __launch_bounds__(256) void k_flash(FlashArgs a) {
  constexpr int KS = D / 64;
  constexpr int CG = D / 16;
  constexpr int VB = VK == kVI8 ? 1 : 2;                 // bytes per V element
  constexpr int K_BYTES = KT * D;                        // int8 K tile
  constexpr int V_BYTES = KT * D * VB;
  __shared__ __attribute__((aligned(16))) int8_t s_k[K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[V_BYTES];
  __shared__ float s_ks[KT];
  __shared__ float s_vs[KT];

  const int qtile = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int Hq = a.Hq, Hkv = a.Hkv;
  const int kvh = h / a.G;

  int64_t q_row0;  // global row of query 0 of this sequence / batch
  int Tq, kv_len;
  const int32_t* trow = nullptr;
  int64_t blk_base = 0;  // dense: first block of this batch
  if constexpr (DENSE) {
    q_row0 = (int64_t)z * a.Nq;
    Tq = a.Nq;
    kv_len = a.Nk;
    blk_base = (int64_t)z * ((a.Nk + 15) / 16);
  } else {
    q_row0 = a.cu_q[z];
    Tq = a.cu_q[z + 1] - (int)q_row0;
    kv_len = a.ctx_lens[z];
    trow = a.tables + (int64_t)z * a.max_blocks;
  }
  const int q0 = qtile * QT;
  if (q0 >= Tq) return;
  const int offset = kv_len - Tq;   // bottom-right causal alignment

  // ---- query fragments and scales -----------------------------------------
  v4i qf[2][KS];
  float qsc[2];
  int qi[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    qi[qg] = q0 + 32 * wave + 16 * qg + n;
    const bool ok = qi[qg] < Tq;
    const int8_t* qp = a.q + ((q_row0 + qi[qg]) * Hq + h) * D + 16 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qg][s] = ok ? *reinterpret_cast<const v4i*>(qp + 64 * s) : v4i{0, 0, 0, 0};
    if constexpr (DENSE) {
      const int nqb = (a.Nq + QT - 1) / QT;
      qsc[qg] = a.q_scale[((int64_t)z * Hq + h) * nqb + qtile] * a.scale_log2;
    } else {
      qsc[qg] = ok ? a.q_scale[(q_row0 + qi[qg]) * Hq + h] * a.scale_log2 : 0.0f;
    }
  }

  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};
  v4f O[2][CG];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int c = 0; c < CG; ++c) O[qg][c] = v4f{0.f, 0.f, 0.f, 0.f};

  int kv_end = kv_len;
  if constexpr (CAUSAL) kv_end = min(kv_len, min(q0 + QT, Tq) - 1 + offset + 1);
  const int ntiles = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;
  const int nblk_seq = (kv_len + 15) / 16;

  for (int tile = 0; tile < ntiles; ++tile) {
    const int kbase = tile * KT;
    // ---- stage K, V (and per-token scales) of 4 blocks into LDS -----------
    {
      // K: 4 blocks x D/16 chunks x 256 bytes, 16 bytes per thread per step
      constexpr int KU = 4 * D;                  // 16-byte units
      for (int u = threadIdx.x; u < KU; u += 256) {
        const int b = u / D, r = u % D;          // r = 16-byte unit within the block
        const int lb = kbase / 16 + b;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (lb < nblk_seq) {
          const int64_t pb = DENSE ? blk_base + lb : (int64_t)trow[lb];
          w = *reinterpret_cast<const uint4*>(a.k_blocks + (pb * Hkv + kvh) * (int64_t)D * 16 + (int64_t)r * 16);
        }
        *reinterpret_cast<uint4*>(s_k + u * 16) = w;
      }
      constexpr int VU = 4 * D * 16 * VB / 16;   // 16-byte units of V
      constexpr int TPU = 16 / VB;               // tokens per unit
      for (int u = threadIdx.x; u < VU; u += 256) {
        const int b = u / (VU / 4), r = u % (VU / 4);
        const int lb = kbase / 16 + b;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (lb < nblk_seq) {
          const int64_t pb = DENSE ? blk_base + lb : (int64_t)trow[lb];
          w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.v_blocks) +
                                               (pb * Hkv + kvh) * (int64_t)D * 16 * VB + (int64_t)r * 16);
          // zero the slots past the context (they may hold anything)
          const int t_first = lb * 16 + (r % (16 / TPU)) * TPU;
          if (t_first + TPU > kv_len) {
            uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < TPU; ++e) {
              if (t_first + e >= kv_len) {
                const int bit = e * VB * 8;
                ws[bit / 32] &= ~(((VB == 2) ? 0xFFFFu : 0xFFu) << (bit % 32));
              }
            }
            w = make_uint4(ws[0], ws[1], ws[2], ws[3]);
          }
        }
        *reinterpret_cast<uint4*>(s_v + u * 16) = w;
      }
      if constexpr (!DENSE) {
        if (threadIdx.x < KT) {
          const int t = kbase + threadIdx.x;
          const int lb = t / 16;
          float ks = 0.0f, vs = 0.0f;
          if (t < kv_len) {
            const int64_t si = ((int64_t)trow[lb] * Hkv + kvh) * 16 + (t & 15);
            ks = a.k_scale[si];
            if constexpr (VK == kVI8) vs = a.v_scale[si];
          }
          s_ks[threadIdx.x] = ks;
          s_vs[threadIdx.x] = vs;
        }
      }
    }
    __syncthreads();

    float tsc = 1.0f;   // dense: key-block scale of this tile
    if constexpr (DENSE) {
      const int nkb = (a.Nk + KT - 1) / KT;
      tsc = a.k_scale[((int64_t)z * Hkv + kvh) * nkb + tile];
    }

#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // ---- S^T = K Q^T for 32 keys x 32 queries --------------------------
      v4i acc[2][2];   // [qg][u]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tau = 32 * half + 8 * (n >> 2) + 4 * u + (n & 3);
        const int8_t* kp = s_k + (tau >> 4) * (D * 16) + (tau & 15) * 16;
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) acc[qg][u] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const v4i kf = *reinterpret_cast<const v4i*>(kp + (4 * s + g) * 256);
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) acc[qg][u] = mfma_i8(kf, qf[qg][s], acc[qg][u]);
        }
      }

      const int tl = 32 * half + 8 * g;     // this lane's first key within the tile
      float sk[8], sv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sk[j] = DENSE ? 1.0f : s_ks[tl + j];
        sv[j] = VK == kVI8 ? s_vs[tl + j] : 1.0f;
      }

      v8h pf[2];
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        const int pos = qi[qg] + offset;    // newest visible key of this query
        const float rs = DENSE ? qsc[qg] * tsc : qsc[qg];
        float sc[8];
        float mt = kNegInf;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = kbase + tl + j;
          bool vis = t < kv_len;
          if constexpr (CAUSAL) vis = vis && t <= pos;
          const float v = (float)acc[qg][j >> 2][j & 3] * rs * sk[j];
          sc[j] = vis ? v : kNegInf;
          mt = fmaxf(mt, sc[j]);
        }
        mt = group4_max(mt);
        const float m_new = fmaxf(m_run[qg], mt);
        const float mref = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run[qg] - mref);
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = fast_exp2(sc[j] - mref);
          psum += p;
          pf[qg][j] = (_Float16)(VK == kVI8 ? p * sv[j] : p);
        }
        l_run[qg] = l_run[qg] * alpha + psum;
        m_run[qg] = m_new;
#pragma unroll
        for (int c = 0; c < CG; ++c) O[qg][c] *= alpha;
      }

      // ---- O^T += V^T P^T ----------------------------------------------------
      const int vb = tl >> 4, so = tl & 15;
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const uint8_t* vp = s_v + ((vb * D + 16 * c + n) * 16 + so) * VB;
        v8h vf;
        if constexpr (VK == kVI8) vf = i8x8_to_f16x8(*reinterpret_cast<const uint2*>(vp));
        else if constexpr (VK == kVF16) vf = f16x8_from_u4(*reinterpret_cast<const uint4*>(vp));
        else vf = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(vp));
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) O[qg][c] = mfma_f16(vf, pf[qg], O[qg][c]);
      }
    }
    __syncthreads();
  }

  // ---- normalize and store ----------------------------------------------------
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const float l = group4_sum(l_run[qg]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi[qg] >= Tq) continue;
    const int64_t ob = ((q_row0 + qi[qg]) * Hq + h) * D + 4 * g;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const v4f o = O[qg][c] * inv;
      const int64_t oi = ob + 16 * c;
      if (a.out_bf16) {
        uint2 w;
        w.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
        w.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = w;
      } else if (a.out_f16) {
        uint2 w;
        w.x = f32_to_f16_bits(o[0]) | (f32_to_f16_bits(o[1]) << 16);
        w.y = f32_to_f16_bits(o[2]) | (f32_to_f16_bits(o[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = w;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <int D, int VK, bool DENSE, bool CAUSAL>
hipError_t run_flash(const FlashArgs& a, hipStream_t st) {
  const int qtiles = ((DENSE ? a.Nq : a.max_seqlen_q) + QT - 1) / QT;
  if (qtiles == 0 || a.num_seqs == 0) return hipSuccess;
  const dim3 grid(qtiles, a.Hq, a.num_seqs);
  k_flash<D, VK, DENSE, CAUSAL><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t flash_d(const FlashArgs& a, hipStream_t st) {
  if (a.dense) {
    if (a.v_f16) return a.causal ? run_flash<D, kVF16, true, true>(a, st) : run_flash<D, kVF16, true, false>(a, st);
    return a.causal ? run_flash<D, kVBf16, true, true>(a, st) : run_flash<D, kVBf16, true, false>(a, st);
  }
  return a.v_int8 ? run_flash<D, kVI8, false, true>(a, st) : run_flash<D, kVBf16, false, true>(a, st);
}

}  // namespace

hipError_t launch_flash(const FlashArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return flash_d<64>(a, st);
    case 128: return flash_d<128>(a, st);
    default: return flash_d<256>(a, st);
  }
}

}  // namespace qa
