// Paged decode attention: INT8 Q x INT8 paged K (INT32 accumulation), score
// recovery per element, online softmax in base 2, fp16 P.V with fp32
// accumulation, split-K partials and their combine.
//
// Mapping onto v_mfma_i32_16x16x64_i8 (see common.h for the lane layout).
// The kernel computes S^T = K Q^T per 32-token tile:
//   A operand = 16 key tokens x 64 channels (INT8, straight from the cache)
//   B operand = 64 channels x 16 query columns: the G heads of one KV head
//               ([QK-MMAC] §5.1), times the tq query tokens of a multi-token
//               step (column n = token n / G, head n % G); columns >= G*tq
//               are zero
// A tile covers 32 tokens with two instructions u = 0, 1; matrix row r of
// instruction u holds token 8*(r/4) + 4u + (r%4). With that permutation the
// result lane l (column = head l%16, group g = l/16) owns tokens
// 8g .. 8g+7 of the tile, which is exactly the K-slice lane l must supply as
// the B operand of the fp16 product O^T = V^T P^T. So P never leaves the
// registers, and the per-token key scale ([QK-MMAC] §1, "per column" of S)
// is read as 8 consecutive floats that follow the result layout.
#include <mutex>

#include "common.h"
#include "internal.h"

// Scratch for the allocation-free decode entry point: the split partials
// live here instead of in a caller workspace. Each GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` names a
// host-side stand-in, not a device address: host code only ever uses the
// address decode_scratch() obtains for the current device.
static __device__ __attribute__((aligned(256))) char scratch[qa::kDecodeScratchBytes];

namespace qa {
namespace {

// Workgroup shape: waves per workgroup, each with one 32-token tile in
// flight (more waves, or two tiles per wave, measured slower on MI355X).
constexpr int kWaves = 8;

// Mask words for 8 values held in 16-bit (bf16) or 8-bit (int8) lanes of
// 32-bit words: keep the first `nvalid` values, zero the rest. Slots past
// the context may hold anything (even NaN patterns), and 0 * NaN would
// poison the matrix product, so they are cleared first.
__device__ __forceinline__ uint32_t keep_mask16(int w, int nvalid) {
  return (2 * w < nvalid ? 0x0000FFFFu : 0u) | (2 * w + 1 < nvalid ? 0xFFFF0000u : 0u);
}
__device__ __forceinline__ uint32_t keep_mask8(int w, int nvalid) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) m |= (4 * w + b < nvalid ? 0xFFu : 0u) << (8 * b);
  return m;
}

// Registers of one 32-token tile: K fragments, V^T fragments and scales.
template <int D, bool V_I8>
struct Tile {
  static constexpr int KS = D / 64, CG = D / 16;
  v4i kr[2][KS];
  uint4 v16[V_I8 ? 1 : CG];
  uint2 v8[V_I8 ? CG : 1];
  float4 ska, skb, sva, svb;
};

struct DecodeLane {
  int n, g, kvh, Hkv, tau0;
};

// Issue every load of one tile whose two blocks are p0, p1.
template <int D, bool V_I8, bool EXPORT_QK>
__device__ __forceinline__ void issue_tile(Tile<D, V_I8>& t, const DecodeArgs& a, const DecodeLane& L,
                                           int p0, int p1) {
  constexpr int KS = D / 64, CG = D / 16;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tau = L.tau0 + 4 * u;
    const int pb = tau >= 16 ? p1 : p0;
    const int8_t* kp = a.k_cache + ((int64_t)pb * L.Hkv + L.kvh) * (D / 16) * 256 + (tau & 15) * 16 + L.g * 256;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.kr[u][s] = *reinterpret_cast<const v4i*>(kp + s * 1024);
  }
  if constexpr (!EXPORT_QK) {
    // tokens 8g .. 8g+7 of the tile live in one block at slots so .. so+7
    const int pbs = L.g >= 2 ? p1 : p0;
    const int so = 8 * (L.g & 1);
    const int64_t sidx = ((int64_t)pbs * L.Hkv + L.kvh) * 16 + so;
    t.ska = *reinterpret_cast<const float4*>(a.k_scale + sidx);
    t.skb = *reinterpret_cast<const float4*>(a.k_scale + sidx + 4);
    if constexpr (V_I8) {
      t.sva = *reinterpret_cast<const float4*>(a.v_scale + sidx);
      t.svb = *reinterpret_cast<const float4*>(a.v_scale + sidx + 4);
    }
    const int64_t vbase = (((int64_t)pbs * L.Hkv + L.kvh) * D + L.n) * 16 + so;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      if constexpr (V_I8)
        t.v8[c] = *reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(a.v_cache) + vbase + c * 256);
      else
        t.v16[c] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v_cache) + vbase + c * 256);
    }
  }
}

// Per-wave online-softmax state.
template <int D>
struct Acc {
  v4f O[D / 16];
  float m, l;
};

// Consume one tile: INT8 QK, score recovery, online softmax, P.V.
// tl = first token of this lane's 8-token slice, t1 = end of the segment,
// t1c = end of the keys this lane's query column sees (<= t1; less for the
// earlier tokens of a multi-token step).
template <int D, bool V_I8, bool EXPORT_QK>
__device__ __forceinline__ void consume_tile(Tile<D, V_I8>& t, Acc<D>& A, const v4i (&qf)[D / 64], float qsc,
                                             int tl, int t1, int t1c, int32_t* qk_dst) {
  constexpr int KS = D / 64, CG = D / 16;
  // ---- S^T = K Q^T ----------------------------------------------------------
  v4i acc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    acc[u] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc[u] = mfma_i8(t.kr[u][s], qf[s], acc[u]);
  }
  if constexpr (EXPORT_QK) {
    if (qk_dst != nullptr) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tl + j < t1) qk_dst[tl + j] = acc[j >> 2][j & 3];
    }
    return;
  }
  const int nvalid = min(max(t1 - tl, 0), 8);     // slots holding keys of the context (V kept)
  const int nvis = min(max(t1c - tl, 0), 8);       // keys this query column sees

  // ---- [QK-MMAC] §1: recover each score before the softmax (base 2) -------
  const float sk[8] = {t.ska.x, t.ska.y, t.ska.z, t.ska.w, t.skb.x, t.skb.y, t.skb.z, t.skb.w};
  float sc[8];
  float mt = kNegInf;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v = (float)acc[j >> 2][j & 3] * qsc * sk[j];
    sc[j] = j < nvis ? v : kNegInf;
    mt = fmaxf(mt, sc[j]);
  }
  mt = group4_max(mt);
  const float m_new = fmaxf(A.m, mt);
  const float mref = m_new == kNegInf ? 0.0f : m_new;
  const float alpha = fast_exp2(A.m - mref);
  float p[8], psum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = fast_exp2(sc[j] - mref);
    psum += p[j];
  }
  A.l = A.l * alpha + psum;
  A.m = m_new;

  // P operand. INT8 V: fp16 P with the per-token V scale folded in, and
  // fp16 codes. bf16 V: the raw bf16 values with P as a two-term bf16
  // expansion (two products), so V needs no conversion.
  v8h pf;
  v8bf ph, pl;
  if constexpr (V_I8) {
    const float sv[8] = {t.sva.x, t.sva.y, t.sva.z, t.sva.w, t.svb.x, t.svb.y, t.svb.z, t.svb.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) pf[j] = (_Float16)(j < nvalid ? p[j] * sv[j] : 0.0f);
  } else {
    split_bf16x8(p, ph, pl);
  }
#pragma unroll
  for (int c = 0; c < CG; ++c) A.O[c] *= alpha;

  // ---- O^T += V^T P^T: channel 16c+n, tokens 8g..8g+7 of the tile ---------
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    if constexpr (V_I8) {
      uint2 w = t.v8[c];
      w.x &= keep_mask8(0, nvalid);
      w.y &= keep_mask8(1, nvalid);
      A.O[c] = mfma_f16(i8x8_to_f16x8(w), pf, A.O[c]);
    } else {
      uint4 w = t.v16[c];
      w.x &= keep_mask16(0, nvalid);
      w.y &= keep_mask16(1, nvalid);
      w.z &= keep_mask16(2, nvalid);
      w.w &= keep_mask16(3, nvalid);
      const v8bf vb = __builtin_bit_cast(v8bf, w);
      A.O[c] = mfma_bf16(vb, ph, A.O[c]);
      A.O[c] = mfma_bf16(vb, pl, A.O[c]);
    }
  }
}

// Fused decode step: the query rows and the new token's K/V row are
// quantized inside the split kernel ([QK-MMAC] §4: the producer quantizes Q
// once; here every workgroup re-derives its G rows, which is cheaper than a
// separate launch). Job j < G of a workgroup quantizes query head kvh*G + j
// into LDS; in the workgroup whose segment holds the new token (position
// ctx - 1) job G quantizes its K row and job G + 1 its V row, writes them to
// the cache slot and keeps them in LDS, and the wave whose tile holds that
// position substitutes them for what it loaded from the cache. Same
// arithmetic as the producer kernel, so the results are bit-identical.
template <int D, bool V_I8>
struct NewToken {
  int8_t q[16][D];          // query codes, one row per head of the group
  float qs[16];             // query scales
  uint32_t k[D / 4];        // K codes of the new token
  uint16_t v[D];            // its V: bf16 bits, or INT8 codes (low byte)
  float ks, vs;             // its K and V scales
};

// One wave quantizes a row of D 16-bit values, E = D/64 per lane (bits as
// loaded): returns this lane's E codes packed in bytes and the row scale.
// With rope.pos set, the row (16-bit inputs at `row`) is first rotated by the
// table row of position p.
template <int D>
__device__ __forceinline__ uint32_t quant_row_wave(const uint16_t (&bits)[D / 64], bool bf16, float& scale,
                                                   const Rope& rope = Rope{}, const uint16_t* row = nullptr,
                                                   int64_t p = 0) {
  constexpr int E = D / 64;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = bf16 ? bf16_to_f32(bits[e]) : f16_to_f32(bits[e]);
  if (rope.pos != nullptr) {
    const int lane = threadIdx.x & 63;
    const float* cs = rope.cs + p * rope.rot;
    if (bf16) rope_lane<E, true>(row, lane * E, x, cs, rope.rot, rope.neox);
    else rope_lane<E, false>(row, lane * E, x, cs, rope.rot, rope.neox);
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = wave_max(amax);
  scale = quant_scale(amax);
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = amax > 0.0f ? quant_code(x[e], scale) : 0;
    packed |= ((uint32_t)c & 0xFFu) << (8 * e);
  }
  return packed;
}

// MT: several query tokens per sequence (a.tq > 1); the one-token kernels
// are compiled without the per-column bookkeeping. ROPE (fused step only):
// rotate the query rows and the new K row first.
template <int D, bool V_I8, bool EXPORT_QK, bool FUSED, bool MT, bool ROPE = false>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_decode(DecodeArgs a) {
  constexpr int KS = D / 64;   // INT8 K-steps
  constexpr int CG = D / 16;   // 16-channel groups of the output
  extern __shared__ float smem[];

  const int split = blockIdx.x, kvh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Sequences longest first (a.lpt, 2..64 sequences): slot blockIdx.z takes
  // the sequence of that rank by context length, so that the longest
  // segments start first and the short ones fill in at the end (workgroups
  // are dispatched in index order). Every wave ranks its lane's sequence
  // against all the others with lane reads (ties by index, so slots and
  // sequences correspond one to one); no barrier, no extra launch.
  int seq = blockIdx.z;
  int ctx;
  if (a.lpt) {
    const int ns = a.num_seqs;
    const int mine = lane < ns ? a.ctx_lens[lane] : 0;
    int rank = 0;
    for (int s2 = 0; s2 < ns; ++s2) {
      const int c = __builtin_amdgcn_readlane(mine, s2);
      rank += (c > mine || (c == mine && s2 < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < ns && rank == (int)blockIdx.z);
    seq = __builtin_amdgcn_readfirstlane(hit != 0 ? (int)__builtin_ctzll(hit) : (int)blockIdx.z);
    ctx = __builtin_amdgcn_readlane(mine, seq);
  } else {
    ctx = a.ctx_lens[seq];
  }
  const int n = lane & 15, g = lane >> 4;
  const int G = a.G, Hq = a.Hq, Hkv = a.Hkv, S = a.num_splits;

  // Segment of this split: blocks [split*per, (split+1)*per) of the block
  // table, cut at the context length. With seq_split the sequence's own
  // blocks are cut into S equal segments (per = ceil(ceil(ctx/16)/S): every
  // split of a sequence gets the same share, whatever the other sequences'
  // lengths), so the table fetch waits for the context length; otherwise
  // per = ceil(max_blocks/S) depends only on host-known sizes and the
  // block-table entries are fetched together with the context length.
  const int per = a.seq_split ? max(((ctx + 15) / 16 + S - 1) / S, 1) : (a.max_blocks + S - 1) / S;
  const int blk0 = split * per;
  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  // lane j: block (j & 1) of this wave's tile j/2 (tiles k .. k+31)
  int tab = trow[min(blk0 + 2 * (wave + kWaves * (lane >> 1)) + (lane & 1), a.max_blocks - 1)];

  // Query fragments (B operand): column n = token jt, head kvh*G + hn of this
  // KV group, channels 64s+16g..+15.
  const int Tq = MT ? a.tq : 1, ncol = G * Tq;
  const int jt = MT ? n / G : 0, hn = n - jt * G;
  const int h = kvh * G + hn;
  const int qrow = seq * Tq + jt;                  // query row (sequence, token)
  const bool live_col = n < ncol;
  v4i qf[KS];
  float qsc = 0.0f;
  if constexpr (!FUSED) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (live_col)
        qf[s] = *reinterpret_cast<const v4i*>(a.q + ((int64_t)qrow * Hq + h) * D + 64 * s + 16 * g);
      else
        qf[s] = v4i{0, 0, 0, 0};
    }
    qsc = live_col ? a.q_scale[(int64_t)qrow * Hq + h] * a.scale_log2 : 0.0f;
  }
  const int t0 = min(blk0 * 16, ctx);
  const int t1 = min(t0 + per * 16, ctx);
  const int ntiles = (t1 - t0 + 31) >> 5;
  // token jt of a tq-token step sits at position ctx - tq + jt and sees the
  // keys up to it
  const int t1c = MT ? min(t1, ctx - Tq + jt + 1) : t1;
  const int ntw = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;   // this wave's tiles

  int32_t* qk_dst = nullptr;
  if constexpr (EXPORT_QK)
    if (live_col) qk_dst = a.acc_out + ((int64_t)seq * Hq + h) * (int64_t)a.max_blocks * 16;

  Acc<D> A;
  A.m = kNegInf;
  A.l = 0.0f;
#pragma unroll
  for (int c = 0; c < CG; ++c) A.O[c] = v4f{0.f, 0.f, 0.f, 0.f};
  const DecodeLane L{n, g, kvh, Hkv, 8 * (n >> 2) + (n & 3)};

  // Issue every load of this wave's tile k (tiles go round-robin over the
  // waves); the block-table entries come 32 tiles at a time.
  auto issue_k = [&](Tile<D, V_I8>& T, int k) {
    if (k > 0 && (k & 31) == 0)
      tab = trow[min(blk0 + 2 * (wave + kWaves * (k + (lane >> 1))) + (lane & 1), a.max_blocks - 1)];
    const int ki = k & 31;
    const int tb = t0 + 32 * (wave + kWaves * k);
    const int p0 = __builtin_amdgcn_readlane(tab, 2 * ki);
    // The second block exists only if the tile has tokens in it; table
    // entries past the sequence are never used as addresses.
    const int p1 = tb + 16 < t1 ? __builtin_amdgcn_readlane(tab, 2 * ki + 1) : p0;
    issue_tile<D, V_I8, EXPORT_QK>(T, a, L, p0, p1);
  };

  // ---- fused step: which rows this workgroup quantizes --------------------
  const int pnew = ctx - 1;                                   // position of the new token
  const bool writer = ctx > 0 ? (pnew >> 4) >= blk0 && (pnew >> 4) < blk0 + per : split == 0;
  const int jobs = FUSED ? G + (writer ? 2 : 0) : 0;
  auto job_row = [&](int j) -> const uint16_t* {
    if (j < G) return a.q_in + seq * a.q_st + (int64_t)(kvh * G + j) * a.q_sh;
    return (j == G ? a.k_new : a.v_new) + seq * a.kv_st + (int64_t)kvh * a.kv_sh;
  };
  // the first job's row is loaded before the first tile, so waiting for it
  // does not wait for the tile
  uint16_t pre[KS];
  if (FUSED && (wave < G || wave < jobs)) {   // (wave < G needs no context length)
    const uint16_t* row = job_row(wave);
#pragma unroll
    for (int e = 0; e < KS; ++e) pre[e] = row[lane * KS + e];
  }

  Tile<D, V_I8> T;
  if (ntw > 0) issue_k(T, 0);
  // keep the loads of the first tile ahead of the query work below
  __builtin_amdgcn_sched_barrier(0);

  int64_t slot = -1;
  if constexpr (FUSED) {
    __shared__ NewToken<D, V_I8> nt;
    slot = a.slots[seq];
    for (int j = wave; j < jobs; j += kWaves) {
      uint16_t bits[KS];
      if (j == wave) {
#pragma unroll
        for (int e = 0; e < KS; ++e) bits[e] = pre[e];
      } else {
        const uint16_t* row = job_row(j);
#pragma unroll
        for (int e = 0; e < KS; ++e) bits[e] = row[lane * KS + e];
      }
      float sc;
      const Rope rope = ROPE ? a.rope : Rope{};
      const int64_t rpos = ROPE ? a.rope.pos[seq] : 0;
      if (j < G) {
        const uint32_t codes = quant_row_wave<D>(bits, a.in_bf16, sc, rope, job_row(j), rpos);
#pragma unroll
        for (int e = 0; e < KS; ++e) nt.q[j][lane * KS + e] = (int8_t)(codes >> (8 * e));
        if (lane == 0) nt.qs[j] = sc;
      } else if (j == G) {
        const uint32_t codes = quant_row_wave<D>(bits, a.in_bf16, sc, rope, job_row(j), rpos);
#pragma unroll
        for (int e = 0; e < KS; ++e) reinterpret_cast<int8_t*>(nt.k)[lane * KS + e] = (int8_t)(codes >> (8 * e));
        if (lane == 0) nt.ks = sc;
        if (slot >= 0) {
          const int64_t bh = (slot >> 4) * Hkv + kvh;
          const int off = (int)(slot & 15), ch = lane * KS;
          int8_t* dst = a.kc_w + (bh * (D / 16) + ch / 16) * 256 + off * 16 + (ch % 16);
          if constexpr (KS == 4) *reinterpret_cast<uint32_t*>(dst) = codes;
          else if constexpr (KS == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)codes;
          else *dst = (int8_t)codes;
          if (lane == 0) a.ks_w[bh * 16 + off] = sc;
        }
      } else {
        const int64_t bh = (slot >> 4) * Hkv + kvh;
        const int off = (int)(slot & 15);
        if constexpr (V_I8) {
          const uint32_t codes = quant_row_wave<D>(bits, a.in_bf16, sc);
#pragma unroll
          for (int e = 0; e < KS; ++e) nt.v[lane * KS + e] = (uint16_t)((codes >> (8 * e)) & 0xFFu);
          if (lane == 0) nt.vs = sc;
          if (slot >= 0) {
#pragma unroll
            for (int e = 0; e < KS; ++e)
              reinterpret_cast<int8_t*>(a.vc_w)[(bh * D + lane * KS + e) * 16 + off] = (int8_t)(codes >> (8 * e));
            if (lane == 0) a.vs_w[bh * 16 + off] = sc;
          }
        } else {
#pragma unroll
          for (int e = 0; e < KS; ++e) {
            nt.v[lane * KS + e] = bits[e];
            if (slot >= 0) reinterpret_cast<uint16_t*>(a.vc_w)[(bh * D + lane * KS + e) * 16 + off] = bits[e];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = live_col ? *reinterpret_cast<const v4i*>(&nt.q[n][64 * s + 16 * g]) : v4i{0, 0, 0, 0};
    qsc = live_col ? nt.qs[n] * a.scale_log2 : 0.0f;

    // ---- main loop, with the new token substituted in its tile ----------
    for (int k = 0; k < ntw; ++k) {
      const int tb = t0 + 32 * (wave + kWaves * k);
      if (writer && slot >= 0 && pnew >= tb && pnew < tb + 32) {
        const int i = pnew - tb;       // the new token's row in this tile
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (L.tau0 + 4 * u == i) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
              T.kr[u][s] = *reinterpret_cast<const v4i*>(reinterpret_cast<const int8_t*>(nt.k) + 64 * s + 16 * g);
          }
        const int j = i - 8 * g;       // its slot among this lane's 8 tokens, if any
        if (j >= 0 && j < 8) {
          float* ska = reinterpret_cast<float*>(&T.ska);
          float* skb = reinterpret_cast<float*>(&T.skb);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (j == e) ska[e] = nt.ks;
            if (j == 4 + e) skb[e] = nt.ks;
          }
          if constexpr (V_I8) {
            float* sva = reinterpret_cast<float*>(&T.sva);
            float* svb = reinterpret_cast<float*>(&T.svb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (j == e) sva[e] = nt.vs;
              if (j == 4 + e) svb[e] = nt.vs;
            }
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const uint32_t code = nt.v[16 * c + n] & 0xFFu;
              uint32_t* w = reinterpret_cast<uint32_t*>(&T.v8[c]);
              const int wi = j >> 2, sh = 8 * (j & 3);
#pragma unroll
              for (int q = 0; q < 2; ++q)
                if (q == wi) w[q] = (w[q] & ~(0xFFu << sh)) | (code << sh);
            }
          } else {
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const uint32_t bits = nt.v[16 * c + n];
              uint32_t* w = reinterpret_cast<uint32_t*>(&T.v16[c]);
              const int wi = j >> 1, sh = 16 * (j & 1);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (q == wi) w[q] = (w[q] & ~(0xFFFFu << sh)) | (bits << sh);
            }
          }
        }
      }
      consume_tile<D, V_I8, EXPORT_QK>(T, A, qf, qsc, tb + 8 * g, t1, t1c, qk_dst);
      if (k + 1 < ntw) {
        issue_k(T, k + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    for (int k = 0; k < ntw; ++k) {
      const int tb = t0 + 32 * (wave + kWaves * k);
      consume_tile<D, V_I8, EXPORT_QK>(T, A, qf, qsc, tb + 8 * g, t1, t1c, qk_dst);
      if (k + 1 < ntw) {
        issue_k(T, k + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (EXPORT_QK) return;

  // ---- merge the waves of this workgroup ----------------------------------
  const float l_run = group4_sum(A.l);
  float* sm_ml = smem;                       // [kWaves][16][2]
  float* sm_o = smem + kWaves * 32;          // [kWaves][G*tq][D]
  if (g == 0) {
    sm_ml[(wave * 16 + n) * 2] = A.m;
    sm_ml[(wave * 16 + n) * 2 + 1] = l_run;
  }
  if (live_col) {
#pragma unroll
    for (int c = 0; c < CG; ++c)
      *reinterpret_cast<float4*>(sm_o + ((int64_t)wave * ncol + n) * D + 16 * c + 4 * g) =
          make_float4(A.O[c][0], A.O[c][1], A.O[c][2], A.O[c][3]);
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < ncol * D; idx += kWaves * 64) {
    const int cn = idx / D, ch = idx - cn * D;     // column cn = token cn / G, head cn % G
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[(w * 16 + cn) * 2]);
    float lsum = 0.0f, o = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(sm_ml[(w * 16 + cn) * 2] - M);
        lsum += wt * sm_ml[(w * 16 + cn) * 2 + 1];
        o += wt * sm_o[((int64_t)w * ncol + cn) * D + ch];
      }
    }
    const int ct = MT ? cn / G : 0;
    const int hh = kvh * G + (cn - ct * G);
    const int row = seq * Tq + ct;
    if (S == 1) {
      const float r = lsum > 0.0f ? o / lsum : 0.0f;
      const int64_t oi = ((int64_t)row * Hq + hh) * D + ch;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(r);
      else reinterpret_cast<float*>(a.out)[oi] = r;
    } else {
      const int64_t pi = ((int64_t)row * Hq + hh) * S + split;
      a.ws_o[pi * D + ch] = o;
      if (ch == 0) {
        a.ws_ml[pi * 2] = M;
        a.ws_ml[pi * 2 + 1] = lsum;
      }
    }
  }
}

// Merge the S partials of each (query head, sequence):
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
// Many splits: one wave per (query row, head, 4 channels). Lane s reads
// split s (and s + 64, ... when S > 64); the wave reduces the maximum, then
// the weighted sums, with lane exchanges inside the registers (DPP and
// permlane: a fixed order, so results do not vary from run to run): one
// round of loads, no LDS, no barrier.
template <int D>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                 int32_t Hq, int32_t S, int32_t rows, bool out_bf16, void* out) {
  constexpr int C4 = D / 4;
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (row * Hq + head) * C4 + c4
  if (wv >= (int64_t)rows * Hq * C4) return;                        // the whole wave
  const int c4 = (int)(wv % C4);
  const int64_t rh = wv / C4;
  const int64_t base = rh * S;
  // the first split of this lane stays in registers between the two passes
  const bool has = lane < S;
  const float2 ml0 = has ? *reinterpret_cast<const float2*>(ws_ml + (base + lane) * 2) : make_float2(kNegInf, 0.f);
  const float4 o0 = has ? *reinterpret_cast<const float4*>(ws_o + (base + lane) * D + 4 * c4)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
  float m = ml0.x;
  for (int s = lane + 64; s < S; s += 64) m = fmaxf(m, ws_ml[(base + s) * 2]);
  const float M = wave_max(m);
  float l = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != kNegInf) {
    if (ml0.x != kNegInf) {
      const float w = fast_exp2(ml0.x - M);
      l = w * ml0.y;
      acc = make_float4(w * o0.x, w * o0.y, w * o0.z, w * o0.w);
    }
    for (int s = lane + 64; s < S; s += 64) {
      const float2 ml = *reinterpret_cast<const float2*>(ws_ml + (base + s) * 2);
      if (ml.x == kNegInf) continue;
      const float4 o = *reinterpret_cast<const float4*>(ws_o + (base + s) * D + 4 * c4);
      const float w = fast_exp2(ml.x - M);
      l += w * ml.y;
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
  }
  l = wave_sum(l);
  acc.x = wave_sum(acc.x);
  acc.y = wave_sum(acc.y);
  acc.z = wave_sum(acc.z);
  acc.w = wave_sum(acc.w);
  if (lane != 0) return;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const int64_t oi = rh * D + 4 * c4;
  if (out_bf16) {
    uint2 w;
    w.x = f32_to_bf16_bits(acc.x * inv) | (f32_to_bf16_bits(acc.y * inv) << 16);
    w.y = f32_to_bf16_bits(acc.z * inv) | (f32_to_bf16_bits(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oi) = w;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oi) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

// The merge for few splits (S <= kFewSplits): one thread per (query row,
// head, 4 channels) walks the S partials with every load of a batch of 8
// issued before the merge; many sequences fill the grid.
constexpr int kFewSplits = 16;

template <int D>
__global__ __launch_bounds__(256) void k_combine_few(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                     int32_t Hq, int32_t S, int32_t rows, bool out_bf16,
                                                     void* out) {
  constexpr int C4 = D / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)rows * Hq * C4) return;
  const int c4 = (int)(t % C4);
  const int64_t rh = t / C4;                  // row * Hq + head
  const int64_t base = rh * S;
  float m = kNegInf, lsum = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += 8) {
    float2 ml[8];
    float4 o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sp = min(s0 + i, S - 1);
      ml[i] = *reinterpret_cast<const float2*>(ws_ml + (base + sp) * 2);
      o[i] = *reinterpret_cast<const float4*>(ws_o + (base + sp) * D + 4 * c4);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i >= S || ml[i].x == kNegInf) continue;
      const float mn = fmaxf(m, ml[i].x);
      const float a0 = fast_exp2(m - mn), a1 = fast_exp2(ml[i].x - mn);
      acc.x = acc.x * a0 + a1 * o[i].x; acc.y = acc.y * a0 + a1 * o[i].y;
      acc.z = acc.z * a0 + a1 * o[i].z; acc.w = acc.w * a0 + a1 * o[i].w;
      lsum = lsum * a0 + a1 * ml[i].y;
      m = mn;
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  const int64_t oi = rh * D + 4 * c4;
  if (out_bf16) {
    uint2 w;
    w.x = f32_to_bf16_bits(acc.x * inv) | (f32_to_bf16_bits(acc.y * inv) << 16);
    w.y = f32_to_bf16_bits(acc.z * inv) | (f32_to_bf16_bits(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oi) = w;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oi) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

template <int D>
hipError_t launch_combine(const DecodeArgs& a, hipStream_t st) {
  const int rows = a.num_seqs * a.tq;
  if (a.num_splits <= kFewSplits) {
    const int64_t threads = (int64_t)rows * a.Hq * (D / 4);
    k_combine_few<D><<<dim3((unsigned)((threads + 255) / 256)), 256, 0, st>>>(a.ws_o, a.ws_ml, a.Hq, a.num_splits,
                                                                             rows, a.out_bf16, a.out);
  } else {
    const int64_t waves = (int64_t)rows * a.Hq * (D / 4);
    k_combine<D><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, st>>>(a.ws_o, a.ws_ml, a.Hq, a.num_splits, rows,
                                                                    a.out_bf16, a.out);
  }
  return hipGetLastError();
}

template <int D, bool V_I8, bool EXPORT_QK, bool FUSED, bool MT, bool ROPE = false>
hipError_t run_decode(const DecodeArgs& a, DecodePhase phase, hipStream_t st) {
  if (phase == DecodePhase::kCombine) {
    if (a.num_splits > 1) return launch_combine<D>(a, st);
    return hipSuccess;
  }
  const dim3 grid(a.num_splits, a.Hkv, a.num_seqs);
  // LDS: per-wave partials [kWaves][G][D] plus (max, sum) pairs.
  const size_t lds = EXPORT_QK ? 0 : (size_t)(kWaves * 32 + kWaves * a.G * a.tq * D) * sizeof(float);
  auto kern = k_decode<D, V_I8, EXPORT_QK, FUSED, MT, ROPE>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<grid, kWaves * 64, lds, st>>>(a);
  if (!EXPORT_QK && a.num_splits > 1 && phase == DecodePhase::kBoth) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine<D>(a, st);
  }
  return hipGetLastError();
}

template <bool EXPORT_QK>
hipError_t dispatch(const DecodeArgs& a, DecodePhase phase, hipStream_t st) {
#define QA_DEC(DD)                                                                                  \
  if (a.q_in != nullptr && a.rope.pos != nullptr)                                                   \
    return a.v_int8 ? run_decode<DD, true, false, true, false, true>(a, phase, st)                  \
                    : run_decode<DD, false, false, true, false, true>(a, phase, st);                \
  if (a.q_in != nullptr)                                                                            \
    return a.v_int8 ? run_decode<DD, true, false, true, false>(a, phase, st)                        \
                    : run_decode<DD, false, false, true, false>(a, phase, st);                      \
  if (!EXPORT_QK && a.tq > 1)                                                                       \
    return a.v_int8 ? run_decode<DD, true, false, false, true>(a, phase, st)                        \
                    : run_decode<DD, false, false, false, true>(a, phase, st);                      \
  return a.v_int8 ? run_decode<DD, true, EXPORT_QK, false, false>(a, phase, st)                     \
                  : run_decode<DD, false, EXPORT_QK, false, false>(a, phase, st)
  switch (a.D) {
    case 64: QA_DEC(64);
    case 128: QA_DEC(128);
    default: QA_DEC(256);
  }
#undef QA_DEC
}

}  // namespace

int32_t choose_decode_splits(int32_t num_seqs, int32_t Hkv, int32_t max_blocks) {
  // Aim for one workgroup per compute unit (256 CUs) for one sequence (its
  // segments are equal) and two for several (segments of unequal length,
  // run longest first, balance better two to a unit), but keep at least 16
  // blocks (256 tokens) per segment.
  const int64_t units = (int64_t)num_seqs * Hkv;
  const int64_t target = num_seqs > 1 ? 512 : 256;
  int64_t s = (target + units - 1) / units;
  const int64_t cap = max_blocks / 16 > 0 ? max_blocks / 16 : 1;
  if (s > cap) s = cap;
  if (s > 256) s = 256;
  return (int32_t)(s < 1 ? 1 : s);
}

hipError_t decode_scratch(void** ptr) {
  // Device addresses of `scratch`, one per device, looked up on the first
  // call made with that device current.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, DecodePhase phase, hipStream_t st) {
  return dispatch<false>(a, phase, st);
}

hipError_t launch_debug_qk(const DecodeArgs& a, hipStream_t st) {
  DecodeArgs b = a;
  b.num_splits = 1;
  return dispatch<true>(b, DecodePhase::kPartials, st);
}

}  // namespace qa
