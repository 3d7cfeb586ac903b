// Chunked prefill with the P.V product in FP8 (E4M3) ([QK-MMAC] §5.2 for the
// paged rows; [SAGE-MACA] names the FP8 P.V product of later SageAttention
// versions among the features its hardware cannot run, and gfx950 has E4M3
// matrix instructions).
//
// Two passes over V, then the attention:
//   k_v8_amax   per (sequence, KV head, channel) partial maxima of |V| over
//               32 slices of the cached tokens (INT8 V as fl32(code * scale))
//   k_v8_tiles  the channel scales s_c = fl32(max|V| / 448) and the E4M3
//               codes E4M3(fl32(V / s_c)) of every 128-key tile, written in
//               the attention kernel's LDS layout (zero past the context)
//   k_prefill8  the attention: per 128-key tile, S^T = K Q^T on
//               v_mfma_i32_16x16x64_i8 (K straight from the paged cache into
//               LDS), the online softmax, and O^T += V8^T P8^T on
//               v_mfma_scale_f32_16x16x128_f8f6f4 (V8 straight from the
//               workspace into LDS); row sums against an all-ones E4M3 block.
//
// P8 = E4M3(448 * 2^-3 * 2^(s - m_ref)) with a reference m_ref moved only when
// a tile's maximum exceeds it by more than 3 (base 2), so P <= 448 (the
// largest E4M3 value) and the accumulators are rescaled rarely.
//
// Rows as in the 16-bit prefill kernel: row r of a (sequence, KV head) is
// query token r / G of query head kvh*G + r % G; 12 waves of 16 rows.
//
// Lane layout of the products (lane l: n = l % 16, g = l / 16):
//   S^T block b (16 keys) row 4g + i holds key 32*g + 4*b + i of the tile
//   (K rows are read in that order), so lane l ends up owning the 32
//   consecutive keys 32g .. 32g+31 of its query n, byte k of its P8 operand
//   being key 32g + k. The V8 operand of lane l is channel 16c + n, the same
//   32 keys: the reduction pairs A and B bytes of one lane group.
//   LDS V8 tile: [key group 4][channel D][32 bytes]; the two 16-key halves of
//   a channel's 32 bytes are swapped when bit 3 of the channel is set, so the
//   16 lanes of each ds_read_b128 pass (lane bits 2..4 of equal parity) read
//   16 distinct 16-byte bank slots.
//   LDS K tile: 8 blocks of D*16 bytes, each padded by 32 bytes: the 16 lanes
//   of a pass then read 16 distinct slots in every S^T step.
#include "common.h"
#include "internal.h"

namespace qa {
namespace {

constexpr int KT8 = 128;                           // keys per tile
constexpr int kBlk8 = KT8 / 16;                    // cache blocks per tile
constexpr int kNW8 = 12;                           // waves per workgroup
constexpr int kParts = kV8Parts;                   // slices of the max pass
constexpr float kSlack8 = 3.0f;                    // reference threshold (base 2)
constexpr float kLog2Top8 = 5.807354922057604f;    // log2(448) - 3
constexpr float kMRun8 = -1.0e30f;                 // finite start: no empty-row test needed

typedef int v8i_t __attribute__((ext_vector_type(8)));

// O^T (16 channels x 16 queries) += V8^T P8^T over 128 keys, E4M3 operands
// (zero scale operands: the unscaled product).
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i_t a, v8i_t b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// fp32 values of 8 consecutive tokens (8*h8 .. 8*h8+7) of one channel row of
// a cache block (bh = block * Hkv + KV head): bf16 exactly, INT8 codes as
// fl32(code * scale of the token)
template <int D, bool VI8>
__device__ __forceinline__ void v_row8(const PrefillFp8Args& a, int64_t bh, int ch, int h8, float (&v)[8]) {
  if constexpr (VI8) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(a.v_cache) + (bh * D + ch) * 16 + 8 * h8);
    const float4 s0 = *reinterpret_cast<const float4*>(a.v_scale + bh * 16 + 8 * h8);
    const float4 s1 = *reinterpret_cast<const float4*>(a.v_scale + bh * 16 + 8 * h8 + 4);
    const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t word = e < 4 ? w.x : w.y;
      v[e] = (float)(int8_t)(word >> (8 * (e & 3))) * sc[e];
    }
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_cache) + (bh * D + ch) * 16 + 8 * h8);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(ws[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(ws[i] >> 16);
    }
  }
}

// Partial maxima: workgroup (slice, KV head, sequence). A unit is one half
// row (8 tokens of one channel) of one cache block; the 2*D units of a block
// fill 256 threads for D = 128, and the threads of one (channel, half) walk
// the slice's blocks (2*D / 256 ... 256 / (2*D) blocks per pass). Threads of
// one channel combine through LDS. Tokens past the context are skipped.
template <int D, bool VI8>
__global__ __launch_bounds__(256) void k_v8_amax(PrefillFp8Args a) {
  constexpr int U = 2 * D;                         // units per block
  constexpr int BPP = U >= 256 ? 1 : 256 / U;      // blocks per pass
  constexpr int UPT = U >= 256 ? U / 256 : 1;      // units per thread and block
  __shared__ float red[256 * UPT];
  const int part = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int ctx = a.ctx_lens[seq];
  const int nblk = min((ctx + 15) / 16, a.max_blocks);
  const int per = (nblk + kParts - 1) / kParts;
  const int b0 = part * per, b1 = min(b0 + per, nblk);
  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  const int bo = (int)threadIdx.x / (U / UPT);     // block offset within a pass (BPP > 1)
  float m[UPT];
#pragma unroll
  for (int k = 0; k < UPT; ++k) m[k] = 0.0f;
#pragma unroll 4
  for (int b = b0 + bo; b < b1; b += BPP) {
    const int64_t bh = (int64_t)trow[b] * a.Hkv + kvh;
    const int nt = ctx - b * 16;                   // tokens of this block in the context (>= 1)
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = ((int)threadIdx.x % (U / UPT)) + k * 256;   // unit: channel u / 2, half u % 2
      float v[8];
      v_row8<D, VI8>(a, bh, u >> 1, u & 1, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) m[k] = 8 * (u & 1) + e < nt ? fmaxf(m[k], fabsf(v[e])) : m[k];
    }
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) red[threadIdx.x + 256 * k] = m[k];
  __syncthreads();
  for (int ch = threadIdx.x; ch < D; ch += 256) {
    float r = 0.0f;
    // unit u of pass slot bo sits at red[bo * U + u] (UPT == 1) or red[u] (UPT > 1)
#pragma unroll
    for (int q = 0; q < BPP; ++q) r = fmaxf(r, fmaxf(red[q * (U / UPT) * UPT + 2 * ch], red[q * (U / UPT) * UPT + 2 * ch + 1]));
    a.partial[(((int64_t)seq * a.Hkv + kvh) * kParts + part) * D + ch] = r;
  }
}

// E4M3 tiles: workgroup (tile, KV head, sequence). It first reduces the
// partial maxima to the channel scales (tile 0 stores them), then converts
// units of 8 tokens (block j of the tile, channel ch, half h8): the 8 codes
// land at [j/2][ch][16 * ((j%2) ^ bit 3 of ch) + 8 * h8]. Blocks and tokens
// past the context give zeros.
template <int D, bool VI8>
__global__ __launch_bounds__(256) void k_v8_tiles(PrefillFp8Args a) {
  __shared__ float s_sv[D];
  const int tile = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int ctx = a.ctx_lens[seq];
  if (tile * KT8 >= ctx) return;
  const int64_t sk = (int64_t)seq * a.Hkv + kvh;
  for (int ch = threadIdx.x; ch < D; ch += 256) {
    const float* p = a.partial + sk * kParts * D + ch;
    float m = 0.0f;
#pragma unroll 8
    for (int i = 0; i < kParts; ++i) m = fmaxf(m, p[i * D]);
    const float sc = __fdiv_rn(m, 448.0f);
    s_sv[ch] = sc;
    if (tile == 0) a.v8_scale[sk * D + ch] = sc;
  }
  __syncthreads();
  const int nblk = min((ctx + 15) / 16, a.max_blocks);
  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  uint8_t* dst = a.v8 + (((int64_t)seq * a.v8_seq_tiles + tile) * a.Hkv + kvh) * (int64_t)(KT8 * D);
  // units u = threadIdx.x + 256 i; each thread loads a batch of units before
  // converting any (blocks past the sequence read its last block, masked)
  constexpr int PER = kBlk8 * D * 2 / 256;          // units per thread
  constexpr int BATCH = PER < 4 ? PER : 4;
  static_assert(PER % BATCH == 0, "whole batches");
  for (int i0 = 0; i0 < PER; i0 += BATCH) {
    float v[BATCH][8];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = (int)threadIdx.x + 256 * (i0 + k);
      const int h8 = u & 1, ch = (u >> 1) % D, j = (u >> 1) / D;
      const int b = min(tile * kBlk8 + j, nblk - 1);
      v_row8<D, VI8>(a, (int64_t)trow[b] * a.Hkv + kvh, ch, h8, v[k]);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = (int)threadIdx.x + 256 * (i0 + k);
      const int h8 = u & 1, ch = (u >> 1) % D, j = (u >> 1) / D;
      const int b = tile * kBlk8 + j;
      const float sc = s_sv[ch];
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = b < nblk && sc > 0.0f && b * 16 + 8 * h8 + e < ctx ? __fdiv_rn(v[k][e], sc) : 0.0f;
      uint32_t w[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q], x[4 * q + 1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q + 2], x[4 * q + 3], word, true);
        w[q] = (uint32_t)word;
      }
      const int off = (j >> 1) * D * 32 + ch * 32 + 16 * ((j & 1) ^ ((ch >> 3) & 1)) + 8 * h8;
      *reinterpret_cast<uint2*>(dst + off) = make_uint2(w[0], w[1]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kNW8 * 64) __attribute__((amdgpu_waves_per_eu(kNW8 / 4))) void k_prefill8(
    PrefillFp8Args a) {
  constexpr int NW = kNW8;
  constexpr int KS = D / 64;                       // S^T steps of 64 channels
  constexpr int CG = D / 16;                       // 16-channel output blocks
  constexpr int QT = NW * 16;                      // rows per workgroup
  constexpr int KBS = D * 16 + 32;                 // padded K block in LDS
  constexpr int KC = D / 64;                       // 1 KB chunks per K block
  constexpr int VC = KT8 * D / 1024;               // 1 KB chunks per V8 tile
  __shared__ __attribute__((aligned(16))) int8_t s_k[2][kBlk8 * KBS];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][KT8 * D];
  __shared__ __attribute__((aligned(16))) float s_ks[2][KT8];

  // ---- work item: (row tile, KV head, sequence), XCD-aware, long rows first
  const int G = a.G;
  const int nqt = (a.max_seqlen_q * G + QT - 1) / QT;
  const int total = (int)gridDim.x;
  int wid = blockIdx.x;
  if ((total & 7) == 0) wid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  // (uniform: readfirstlane keeps the divisions' results, and all that is
  // derived from them, in scalar registers)
  const int qtile = __builtin_amdgcn_readfirstlane(nqt - 1 - wid % nqt);
  const int kvh = __builtin_amdgcn_readfirstlane((wid / nqt) % a.Hkv);
  const int z = __builtin_amdgcn_readfirstlane(wid / (nqt * a.Hkv));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int Hq = a.Hq, Hkv = a.Hkv;
  const int64_t q_row0 = a.cu_q[z];
  const int Tq = a.cu_q[z + 1] - (int)q_row0;
  const int kv_len = a.ctx_lens[z];
  const int32_t* trow = a.tables + (int64_t)z * a.max_blocks;
  const int r0 = qtile * QT;
  if (r0 >= Tq * G) return;
  const int offset = kv_len - Tq;                  // bottom-right causal alignment
  const int last_blk = (kv_len + 15) / 16 - 1;

  // ---- this lane's query row: fragments and scale
  const int r = r0 + wave * 16 + n;
  const int qi = r / G, qh = kvh * G + (r - qi * G);
  const bool row_ok = qi < Tq;
  v4i qf[KS];
  {
    const int8_t* qp = a.q + ((q_row0 + qi) * Hq + qh) * D + 16 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = row_ok ? *reinterpret_cast<const v4i*>(qp + 64 * s) : v4i{0, 0, 0, 0};
  }
  // score = x * f in base 2. f is kept >= the smallest normal float, so that
  // a hidden key's x = -inf gives -inf, never NaN: only a query row with
  // q_scale * scale below 1.2e-38 is affected, whose codes and hence x are 0
  // when its scale is 0 (a zero row), and whose scores are 0 to fp32
  // precision otherwise, unless K is of order 1e30
  const float f = fmaxf(row_ok ? a.q_scale[(q_row0 + qi) * Hq + qh] * a.scale_log2 : 0.0f, 1.17549435e-38f);
  const int pos = qi + offset;                     // the row sees keys <= pos
  const int wq_first = (r0 + wave * 16) / G;       // first query token of this wave

  float m_run = kMRun8;
  v4f O[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) O[c] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = v4f{0.f, 0.f, 0.f, 0.f};
  const v8i_t ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0

  const int kv_end = min(kv_len, (min(r0 + QT, Tq * G) - 1) / G + offset + 1);
  const int ntiles = kv_end > 0 ? (kv_end + KT8 - 1) / KT8 : 0;
  // tiles of this sequence in the workspace (bounded by its region, whatever the context length)
  const int ntiles_ws = max(min((kv_len + KT8 - 1) / KT8, a.v8_seq_tiles), 1);

  // ---- tile copies ---------------------------------------------------------
  const int64_t k_head = (int64_t)kvh * D * 16;
  const uint32_t kblk32 = (uint32_t)((int64_t)Hkv * D * 16);   // < 2^32: Hkv <= 65535, D <= 256
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lane16 = (uint32_t)lane * 16u;
  const uint32_t sk_lds = lds_addr(&s_k[0][0]), sv_lds = lds_addr(&s_v[0][0]);
  const uint8_t* v8seq = a.v8 + ((int64_t)z * a.v8_seq_tiles * Hkv + kvh) * (int64_t)(KT8 * D);
  const int64_t v8_tile_stride = (int64_t)Hkv * KT8 * D;
  // Block-table entries of a tile: lanes 0..7 read them with one vector load,
  // one tile ahead; readlane turns them into scalars. The logical block is
  // clamped to the sequence's last block and to the table row.
  const int blk_hi = max(min(last_blk, a.max_blocks - 1), 0);
  auto load_blocks = [&](int t) -> int { return trow[min(t * kBlk8 + (lane & 7), blk_hi)]; };
  using Blocks = v8i_t;                           // the 8 physical blocks of a tile (scalars)
  auto unpack = [](int v) {
    Blocks pb;
#pragma unroll
    for (int j = 0; j < kBlk8; ++j) pb[j] = __builtin_amdgcn_readlane(v, j);
    return pb;
  };
  auto pick = [](Blocks pb, int j) {
    int blk = pb[0];
#pragma unroll
    for (int jj = 1; jj < kBlk8; ++jj) blk = j == jj ? pb[jj] : blk;
    return blk;
  };
  auto dma = [&](int buf, int t, Blocks pb) {
#pragma unroll
    for (int i = 0; i < (kBlk8 * KC + NW - 1) / NW; ++i) {
      const int c = wave_s + NW * i, j = c / KC, part = c % KC;
      if ((kBlk8 * KC) % NW != 0 && c >= kBlk8 * KC) break;   // wave-uniform
      const int blk = __builtin_amdgcn_readfirstlane(pick(pb, j));   // uniform: keep it scalar
      copy16_to_lds(a.k_blocks + (uint64_t)(uint32_t)blk * kblk32 + k_head + part * 1024, lane16,
                    sk_lds + (uint32_t)(buf * kBlk8 * KBS + j * KBS + part * 1024));
    }
    const uint8_t* vsrc = v8seq + (int64_t)min(t, ntiles_ws - 1) * v8_tile_stride;
#pragma unroll
    for (int i = 0; i < (VC + NW - 1) / NW; ++i) {
      const int c = wave_s + NW * i;
      if (VC % NW != 0 && c >= VC) break;                     // wave-uniform
      copy16_to_lds(vsrc + c * 1024, lane16, sv_lds + (uint32_t)(buf * KT8 * D + c * 1024));
    }
  };
  // K scales of a tile: thread t < 128 reads key t's scale (0 past the context)
  auto scale_of = [&](int t, Blocks pb) -> float {
    if (tid >= KT8) return 0.0f;
    const int blk = pick(pb, tid >> 4);
    return t * KT8 + tid < kv_len ? a.k_scale[((int64_t)blk * Hkv + kvh) * 16 + (tid & 15)] : 0.0f;
  };

  if (ntiles > 0) {
    const Blocks pb0 = unpack(load_blocks(0));
    dma(0, 0, pb0);
    const float ks0 = scale_of(0, pb0);
    if (tid < KT8) s_ks[0][tid] = ks0;
  }
  int pb_next = ntiles > 0 ? load_blocks(1) : 0;
  wait_vmem_all();
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int kbase = tile * KT8;
    const Blocks pb = unpack(pb_next);            // the next tile's physical blocks

    // ---- S^T = K Q^T: block b, row 4g + i = key 32g + 4b + i ------------------
    // K fragments stream through a ring of 4 registers, read 3 products
    // ahead (a fence per product keeps the compiler from hoisting more)
    v4i acc[kBlk8];
    auto kfrag = [&](int i) {                      // fragment i = KS*b + s
      const int b = i / KS, s = i % KS;
      const int tau = 32 * (n >> 2) + 4 * b + (n & 3);          // key of A row n
      return *reinterpret_cast<const v4i*>(&s_k[buf][(tau >> 4) * KBS + (tau & 15) * 16 + g * 256 + s * 1024]);
    };
    constexpr int NF = kBlk8 * KS, AHEAD = 3;
    v4i kf[4];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) kf[i] = kfrag(i);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      if (i + AHEAD < NF) kf[(i + AHEAD) & 3] = kfrag(i + AHEAD);
      const int b = i / KS, s = i % KS;
      if (s == 0) acc[b] = v4i{0, 0, 0, 0};
      acc[b] = mfma_i8(kf[i & 3], qf[s], acc[b]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // next tile: copies, its block entries one further ahead, its key scales
    // (issued after this tile's S^T products: issued before them, the copies
    // of all waves sit in front of every wave's first products; measured 3%
    // slower)
    dma(buf ^ 1, tile + 1, pb);
    pb_next = load_blocks(tile + 2);
    const float ks_next = scale_of(tile + 1, pb);

    // ---- scores of keys 32g + k, k = 4b + i ------------------------------------
    float x[32];
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
      const v4f sk = *reinterpret_cast<const v4f*>(&s_ks[buf][32 * g + 4 * q4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * q4 + i] = (float)acc[q4][i] * sk[i];
    }
    // masks only on tiles that cross the context end or the causal diagonal:
    // key 32g + k of this lane is visible when k < vis_end; hidden keys get
    // x = -inf, so that their P is exp2(-inf) = 0 (f > 0, see above)
    const bool need_mask = kbase + KT8 > kv_len || kbase + KT8 - 1 > wq_first + offset;
    if (need_mask) {
      const int vis_end = min(kv_len, pos + 1) - kbase - 32 * g;
#pragma unroll
      for (int k = 0; k < 32; ++k) x[k] = k < vis_end ? x[k] : kNegInf;
    }
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int k = 2; k < 32; k += 2) mx = fmaxf(mx, fmaxf(x[k], x[k + 1]));
    // lazy reference: moved only when exceeded by more than the slack. Some
    // lane of the row then holds such a score, so the test takes each lane's
    // own maximum; the maximum across the lane groups is formed only when the
    // reference moves (-inf when every key of the row is hidden).
    const float ml = mx * f;
    if (__any(ml > m_run + kSlack8)) {
      const float m_new = fmaxf(m_run, group4_max(ml));
      const float alpha = fast_exp2(m_run - m_new);
      L *= alpha;
#pragma unroll
      for (int c = 0; c < CG; ++c) O[c] *= alpha;
      m_run = m_new;
    }
    const float cterm = kLog2Top8 - m_run;
    v8i_t bop;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(x[4 * w + i], f, cterm));
      // the first conversion fills bytes 0-1 and keeps the rest of its third
      // operand, which the second one overwrites: any live value serves
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[2]), false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
      bop[w] = word;
    }

    // ---- O^T += V8^T P8^T, row sums against ones -----------------------------
    __builtin_amdgcn_sched_barrier(0);             // no V8 reads hoisted into the softmax
    // V8 fragments two channel blocks ahead (one ahead measured 5% slower)
    const uint8_t* vt = s_v[buf] + g * (D * 32) + n * 32;
    const int sw = (n >> 3) & 1;                   // bit 3 of the channel 16c + n
    auto vfrag = [&](int c) {
      const v4i lo = *reinterpret_cast<const v4i*>(vt + c * 512 + 16 * sw);
      const v4i hi = *reinterpret_cast<const v4i*>(vt + c * 512 + 16 * (sw ^ 1));
      return v8i_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    v8i_t aop[4];
    aop[0] = vfrag(0);
    aop[1] = vfrag(1);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      if (c + 2 < CG) aop[(c + 2) & 3] = vfrag(c + 2);
      O[c] = mfma_fp8_16x16x128(aop[c & 3], bop, O[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    L = mfma_fp8_16x16x128(ones8, bop, L);
    __builtin_amdgcn_sched_barrier(0);

    wait_vmem_all();                               // the next tile has landed
    if (tid < KT8) s_ks[buf ^ 1][tid] = ks_next;
    __syncthreads();
  }

  // ---- normalize, scale by the channel scales, store --------------------------
  if (!row_ok) return;
  const float l = L[0];
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  // a row that sees no key gives zeros (its sequence's scales may be unset)
  const float* svc = a.v8_scale + ((int64_t)z * Hkv + kvh) * D + 4 * g;
  const int64_t ob = ((q_row0 + qi) * Hq + qh) * D + 4 * g;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const float4 sc4 = l > 0.0f ? *reinterpret_cast<const float4*>(svc + 16 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    const v4f o = {O[c][0] * inv * sc4.x, O[c][1] * inv * sc4.y, O[c][2] * inv * sc4.z, O[c][3] * inv * sc4.w};
    const int64_t oi = ob + 16 * c;
    if (a.out_bf16) {
      uint2 w;
      w.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
      w.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = w;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <int D>
hipError_t prefill_fp8_d(const PrefillFp8Args& a, hipStream_t st) {
  const dim3 gv((unsigned)kParts, (unsigned)a.Hkv, (unsigned)a.num_seqs);
  const dim3 gt((unsigned)a.v8_seq_tiles, (unsigned)a.Hkv, (unsigned)a.num_seqs);
  if (a.v_int8) {
    k_v8_amax<D, true><<<gv, 256, 0, st>>>(a);
    k_v8_tiles<D, true><<<gt, 256, 0, st>>>(a);
  } else {
    k_v8_amax<D, false><<<gv, 256, 0, st>>>(a);
    k_v8_tiles<D, false><<<gt, 256, 0, st>>>(a);
  }
  constexpr int QT = kNW8 * 16;
  const int64_t qtiles = ((int64_t)a.max_seqlen_q * a.G + QT - 1) / QT;
  const int64_t total = qtiles * a.Hkv * a.num_seqs;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (total > 0) k_prefill8<D><<<dim3((unsigned)total), kNW8 * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp8(const PrefillFp8Args& a, hipStream_t st) {
  switch (a.D) {
    case 64: return prefill_fp8_d<64>(a, st);
    case 128: return prefill_fp8_d<128>(a, st);
    default: return prefill_fp8_d<256>(a, st);
  }
}

}  // namespace qa
