// Chunked prefill over a paged history ([QK-MMAC] §5.2) and dense
// SageAttention-style forward ([SAGE-MACA] attention-kernel pipeline), one
// kernel template.
//
// Workgroup = NW waves x (16*QG) query rows (dense: of one query head;
// paged: (token, head) rows of one KV head, see k_flash). 64-token KV
// tiles are double-buffered in LDS. Paged tiles are staged through
// registers: while the waves compute on one buffer, every thread holds its
// share of the next tile and writes it to the other buffer afterwards,
// converting V to fp16 (bf16 rounded to fp16, INT8 codes exact). Dense tiles
// come from this library's own preprocessing, already in the LDS layout with
// fp16 V, and are copied global -> LDS directly (global_load_lds_dwordx4),
// which frees the staging registers for a third wave per SIMD. One barrier
// per tile. A dense workgroup's 128 query rows are one query block of the
// per-block quantization ([SAGE-MACA]): the kernel quantizes it from the
// 16-bit queries in its prologue (the preprocessing then skips the query
// pass), with the block quantizer's arithmetic. With fp16 V (no smooth_v,
// whole 64-key tiles) the dense kernel copies V tiles in token order from
// the input itself and forms its P.V operands with transposing LDS reads,
// so the preprocessing has no V pass either.
//
// Matrix products are computed transposed, as in the decode kernel:
//   S^T = K Q^T   (v_mfma_i32_16x16x64_i8; A = 16 keys from LDS, B = 16 queries
//                  held in registers for the whole KV loop)
//   O^T += V^T P^T (v_mfma_f32_16x16x32_f16; A = 16 channels x 32 keys from LDS,
//                  B = P straight from the score registers)
// Key rows are permuted within each 32-token half so that every lane owns 8
// consecutive keys of one query. The softmax row sums run on the matrix
// units as well: a product of P with an all-ones block sums exactly the fp16
// P that multiplies V.
//
// Online softmax in base 2 with lazy rescaling: the running maximum (and the
// O/l rescale) is only moved when a tile's maximum exceeds it by more than
// 2^8, so P stays below 256 (well inside fp16) and most tiles skip the
// rescale. Masks are applied only on tiles that cross the end of the context
// or the causal diagonal ([SAGE-MACA]: the causal mask is needed on the
// diagonal tiles only; tiles above it are skipped).
//
// Tile staging is branch-free: the four physical blocks of a tile are
// wave-uniform (scalar) loads, issued one tile ahead, with the logical block
// clamped to the last one of the sequence; keys past the context are masked in the scores and
// their V rows cleared when the tile is written to LDS.
//
// Workgroup order is XCD-aware: the 8 XCDs receive workgroups round-robin,
// so consecutive work items (the query tiles of one head, which read the
// same K/V) are assigned to the same XCD and share its L2.
#include "common.h"
#include "internal.h"
#include "quant.h"

namespace qa {
namespace {

constexpr int KT = 64;      // keys per LDS tile
constexpr float kRescaleSlack = 8.0f;   // lazy-rescale threshold (base-2 units)
// FP8 P.V: threshold 3 and P scaled by 448 * 2^-3, so the largest P (the
// reference exceeded by 3) is the largest E4M3 value, 448
constexpr float kFp8Slack = 3.0f;
constexpr float kFp8Log2Top = 5.807354922057604f;   // log2(448) - 3

enum VKind { kVBf16 = 0, kVF16 = 1, kVI8 = 2 };

// Fixed tuning choices (each measured against its alternatives on MI355X):
constexpr int kQG = 2;            // query groups of 16 rows per wave (d <= 128)
constexpr int kWpe = 2;           // waves per SIMD, paged prefill d <= 128
constexpr int kWpeDense = 3;      // waves per SIMD, dense d <= 128
constexpr int kSetprio = 3;       // dense: bit 0 raises wave priority over QK, bit 1 over P.V
constexpr int kNW = 4;            // waves per workgroup, d <= 128
constexpr int kNWD256Dense = 8;   // waves per workgroup, dense d = 256
constexpr int kNWD256Paged = 12;  // waves per workgroup, paged prefill d = 256 (192-row workgroups)

// 8 fp32 -> 8 fp16 through four packed conversions (nearest even)
__device__ __forceinline__ v8h pack8(const float (&p)[8]) {
  v8h r;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const v2h h = cvt2_f16(p[j], p[j + 1]);
    r[j] = h[0];
    r[j + 1] = h[1];
  }
  return r;
}

// Initial softmax reference: finite, so that no step needs a test for an
// empty row (exp2 of anything minus it is 0, and a row's first visible key
// always moves it).
constexpr float kMRunInit = -1.0e30f;

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// O^T (32 channels x 32 queries) += V^T P^T over 64 keys, E4M3 operands,
// fp32 accumulation. Lane l holds A row l % 32 and B column l % 32, keys
// 32 * (l / 32) .. +31 as bytes (layout checked on gfx950). Zero scale
// operands select the unscaled instruction (checked equal to unit scales).
__device__ __forceinline__ v16f mfma_fp8_32x32x64(v8i_t a, v8i_t b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, int VK, int NT, bool KDMA, bool VWS>
struct Staged {
  static constexpr int VB = VK == kVI8 ? 1 : 2;    // bytes per cached V element
  static constexpr int KUB = D;                    // 16-byte K units per block
  static constexpr int VUB = D * VB;               // 16-byte V units per block
  static constexpr int KU = (4 * KUB + NT - 1) / NT;   // K units per thread (the last one
  static constexpr int VU = (4 * VUB + NT - 1) / NT;   // may cover only some waves)
  static constexpr int VUS = VWS ? 0 : VU;         // V units staged (none when V is copied from the workspace)
  v4i k[KDMA ? 1 : KU];   // (unused when K goes straight to LDS) plain vector types: a uint4 struct copy under the
  v4i v[VWS ? 1 : VU];    // partial-round guards left an array in memory
  float ks, vs;
};

// V tiles in token order (dense, 16-bit V input without a transpose pass):
// a 64-key tile of D channels is D/8 copies of 1 KB (chunks), each of 512/D
// token rows of D*2 bytes. A P.V operand comes from transposing reads
// (ds_read_b64_tr_b16: lane i of a 16-lane group receives element i%4 of the
// 8-byte reads of lanes 4j + i/4, j = 0..3), four token rows x 16 channels
// per group; the two groups of a half-wave read rows R + j and R + 8 + j
// (j = 0..3, R = 32h + 16p + t0). Row r = 32h + 16p + 8b + 4c + j has the
// level L = 4b + j, and chunk q = L*D/64 + k starts at q*1024 + 32*L bytes:
// the eight rows of a read pass sit on eight levels (disjoint 32-byte bank
// spans) and the chunks, whose offsets never decrease, do not overlap.
template <int D>
constexpr int kVtokChunks = D / 8;
template <int D>
__device__ __forceinline__ uint32_t vtok_chunk(int q) {
  return (uint32_t)q * 1024u + 32u * (uint32_t)(q / (D / 64));
}
// byte offset of token row r in a tile buffer
template <int D>
__device__ __forceinline__ uint32_t vtok_row_off(int r) {
  constexpr int CPL = D / 64, RPC = 512 / D;   // chunks per level, rows per chunk
  const int L = 4 * ((r >> 3) & 1) + (r & 3);
  const int idx = 4 * (r >> 5) + 2 * ((r >> 4) & 1) + ((r >> 2) & 1);
  return vtok_chunk<D>(L * CPL + idx / RPC) + (uint32_t)((idx % RPC) * D * 2);
}
// the token row that lane lam of chunk q's copy takes (D/8 lanes per row)
template <int D>
__device__ __forceinline__ int vtok_dma_row(int q, int lam) {
  constexpr int CPL = D / 64, RPC = 512 / D, LPR = D / 8;
  const int L = q / CPL, idx = (q % CPL) * RPC + lam / LPR;
  return 32 * (idx >> 2) + 16 * ((idx >> 1) & 1) + 8 * (L >> 2) + 4 * (idx & 1) + (L & 3);
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));

// A dense workgroup's query block (128 rows of head h from row r0 of its
// sequence; rows past the sequence count as zeros), quantized in the kernel
// as the block quantizer does it: one scale over the block, quant_scale of
// its largest |x|, and the codes of quant_bytes. Lane (n, g) of a wave
// loads the 16-bit values of its fragments (row qi[qg], channels 64s + 16g
// .. +15) and receives their codes; the block maximum meets in s_red (one
// float per wave). Returns the block's scale.
template <int D, int QG, int NW, bool BF16>
__device__ __forceinline__ float quant_q_block(const FlashArgs& a, int64_t qseq, int h, int Tq,
                                               const int (&qi)[QG], v4i (&qf)[QG][D / 64], float* s_red) {
  constexpr int KS = D / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
  uint4 raw[QG][KS][2];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const bool ok = qi[qg] < Tq;
    const uint16_t* src = a.q_in + qseq + (int64_t)min(qi[qg], Tq - 1) * a.q_st + (int64_t)h * a.q_sh + 16 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      raw[qg][s][0] = ok ? *reinterpret_cast<const uint4*>(src + 64 * s) : make_uint4(0, 0, 0, 0);
      raw[qg][s][1] = ok ? *reinterpret_cast<const uint4*>(src + 64 * s + 8) : make_uint4(0, 0, 0, 0);
    }
  }
  auto vals = [&](int qg, int s, float (&v)[16]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t ws[4] = {raw[qg][s][q].x, raw[qg][s][q].y, raw[qg][s][q].z, raw[qg][s][q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = half_to_f32<BF16>(ws[i] & 0xFFFFu);
        v[8 * q + 2 * i + 1] = half_to_f32<BF16>(ws[i] >> 16);
      }
    }
  };
  float am = 0.0f;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float v[16];
      vals(qg, s, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    }
  am = wave_max(am);
  if (lane == 0) s_red[wave] = am;
  __syncthreads();
  am = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) am = fmaxf(am, s_red[w]);
  const float sc = quant_scale(am);
  const float rs = __fdiv_rn(1.0f, sc);
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float v[16];
      vals(qg, s, v);
      uint32_t w[4];
      quant_bytes<16>(v, am, sc, rs, w);
      qf[qg][s] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  return sc;
}

// NW waves per workgroup, each with QG groups of 16 query rows. Paged
// prefill packs the G query heads of one KV head into the rows ([QK-MMAC]
// §5.2 packs tokens; here tokens and heads): row r of a (sequence, KV head)
// is query token r / G of query head kvh*G + r % G, so one workgroup's K/V
// tiles serve all G heads and the row space G*Tq is cut into equal
// workgroups.
// PV8 (dense, two query groups per wave): P and V in FP8 (E4M3) for the
// second product, a 32x32x64 matrix instruction per 32 channels and tile.
// VWS (paged): V tiles come as fp16 blocks from the per-call workspace that
// k_v16_blocks fills (the LDS layout already), copied straight into LDS
// instead of staged and converted by every workgroup.
template <int D, int QG, int NW, int VK, bool DENSE, bool CAUSAL, bool PV8 = false, bool VWS = false,
          bool VTOK = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D <= 128 ? (DENSE ? kWpeDense : kWpe) : NW / 4))) void k_flash(
    FlashArgs a) {
  constexpr int NT = NW * 64;
  // At 12 waves the register file has no room to stage K as well: paged K
  // tiles (INT8, already in the LDS layout) are copied straight into LDS.
  constexpr bool KDMA = !DENSE && NW == 12;
  constexpr bool VWS_ = VWS && !DENSE;
  using St = Staged<D, VK, NT, KDMA, VWS_>;
  static_assert(!PV8 || (DENSE && QG == 2 && D <= 128), "FP8 P.V: dense, 32 queries per wave");
  constexpr int KS = D / 64;
  constexpr int CG = D / 16;
  constexpr int QT = NW * 16 * QG;                 // query rows per workgroup
  constexpr int VB = St::VB, KUB = St::KUB, VUB = St::VUB, KU = St::KU, VU = St::VU;
  // ds_read_b128 serves a half-wave in two passes of 16 lanes, chosen by the
  // parity of lane bits 2..4 (quads 0,3,5,6 and quads 1,2,4,7); a pass with
  // 16 distinct 16-byte bank slots (of 64 four-byte banks) is conflict-free.
  // K: 4 blocks of D*16 bytes, each padded by 64 bytes, so the blocks that
  // one pass reads fall on complementary banks. V: channel rows of 32 bytes
  // in plain order; a pass reads 8 channels at one key half and 8 at the
  // other, which covers all 16 slots.
  constexpr int KBS = D * 16 + 64;
  constexpr bool kRowSumMfma = VK != kVI8;         // INT8 V folds sV into P: sum P on the VALU
  constexpr bool kMagic = DENSE;                          // dense scores read as floats, see QK
  constexpr int kAcc0 = kMagic ? 0x4B400000 : 0;                            // bit pattern of 1.5 * 2^23
  constexpr float kOffset = 12582912.0f;                                     // 1.5 * 2^23
  __shared__ __attribute__((aligned(16))) int8_t s_k[2][4 * KBS];
  // VTOK: V tiles in token order (see vtok_chunk), 256 bytes of bank offsets more
  __shared__ __attribute__((aligned(16))) _Float16 s_v[2][KT * D + (VTOK ? 128 : 0)];
  __shared__ float s_ks[DENSE ? 1 : 2][KT];
  __shared__ float s_vs[DENSE ? 1 : 2][KT];
  // With 12 waves the query fragments are parked in LDS (each lane re-reads
  // its 16 bytes per K step of every tile) to free registers.
  constexpr bool QLDS = KDMA;
  __shared__ __attribute__((aligned(16))) v4i s_q[QLDS ? NW * QG * KS : 1][64];

  // ---- work item (XCD-aware order) ----------------------------------------
  // Consecutive work items go to one XCD (they share K/V in its L2); each
  // XCD takes one contiguous eighth of the items. Paged: (row tile, KV head,
  // sequence), row tile fastest. Dense: (query tile, sequence, query head):
  // head-major, so every eighth holds heads of all sequences and a long
  // sequence of a varlen batch is spread over all XCDs.
  const int G = DENSE ? 1 : a.G;
  const int nunits = DENSE ? a.Hq : a.Hkv;
  const int nqt = ((DENSE ? a.Nq : a.max_seqlen_q) * G + QT - 1) / QT;
  const int total = (int)gridDim.x;
  int wid = blockIdx.x;
  if ((total & 7) == 0) wid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  // causal: the longest rows (last tiles) start first, the short ones fill the tail
  int qtile = CAUSAL ? nqt - 1 - wid % nqt : wid % nqt;
  int hu_ = DENSE ? wid / (nqt * a.num_seqs) : (wid / nqt) % nunits;
  int z = DENSE ? (wid / nqt) % a.num_seqs : wid / (nqt * nunits);
  if (DENSE && CAUSAL && !a.q_rows.packed && (total & 7) == 0 && ((a.num_seqs * nunits) & 7) == 0) {
    // causal, batched: each XCD keeps its eighth of the (query head,
    // sequence) units and takes their query tiles longest first across all
    // of them (per unit, the long tiles of its last units would start late)
    const int per = (a.num_seqs * nunits) >> 3;
    const int li = (int)(blockIdx.x >> 3);
    const int u = (int)(blockIdx.x & 7) * per + li % per;
    qtile = nqt - 1 - li / per;
    hu_ = u / a.num_seqs;
    z = u % a.num_seqs;
  }
  if (DENSE && a.q_rows.packed) {
    // varlen: (packed 128-row block, query head), the block's sequence from the map

    const int nblk = (int)a.q_rows.nblocks(QT);
    const int j = CAUSAL ? nblk - 1 - wid % nblk : wid % nblk;
    hu_ = wid / nblk;
    z = a.q_map[j];
    if (z < 0 || z >= a.num_seqs) return;
    qtile = j - (int)a.q_rows.block0(z, QT);
  }
  // uniform values: readfirstlane keeps the divisions' results, and all the
  // addresses derived from them, in scalar registers
  qtile = __builtin_amdgcn_readfirstlane(qtile);
  hu_ = __builtin_amdgcn_readfirstlane(hu_);
  z = __builtin_amdgcn_readfirstlane(z);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int Hq = a.Hq, Hkv = a.Hkv;
  const int kvh = DENSE ? hu_ / a.G : hu_;

  int64_t q_row0;
  int Tq, kv_len;
  const int32_t* trow = nullptr;
  int64_t blk_base = 0;
  if constexpr (DENSE) {
    // batched: every sequence has Nq queries and Nk keys; varlen: packed rows
    q_row0 = a.q_rows.start(z);
    Tq = a.q_rows.len(z);
    kv_len = a.k_rows.len(z);
    blk_base = a.k_rows.block0(z, 16);
  } else {
    q_row0 = a.cu_q[z];
    Tq = a.cu_q[z + 1] - (int)q_row0;
    kv_len = a.ctx_lens[z];
    trow = a.tables + (int64_t)z * a.max_blocks;
  }
  const int r0 = qtile * QT;        // first row of the workgroup
  if (r0 >= Tq * G) return;
  const int offset = kv_len - Tq;   // bottom-right causal alignment
  const int last_blk = (kv_len + 15) / 16 - 1;

  // ---- query fragments and scales -------------------------------------------
  v4i qf[QG][KS];
  float qsc[QG];
  int qi[QG], qh[QG];               // query token and query head of this lane's row
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int r = r0 + wave * 16 * QG + 16 * qg + n;
    qi[qg] = DENSE ? r : r / G;
    qh[qg] = DENSE ? hu_ : kvh * G + (r - qi[qg] * G);
    const bool ok = qi[qg] < Tq;
    if (DENSE && a.q_in != nullptr) continue;   // quantized below
    const int8_t* qp = a.q + ((q_row0 + qi[qg]) * Hq + qh[qg]) * D + 16 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qg][s] = ok ? *reinterpret_cast<const v4i*>(qp + 64 * s) : v4i{0, 0, 0, 0};
    if constexpr (DENSE) {
      const int nqb = (Tq + 127) / 128;   // >= 1: the workgroup holds a row of the sequence
      qsc[qg] = a.q_scale[a.q_rows.scale_at(z, qh[qg], Hq, min(qi[qg] / 128, nqb - 1), 128)] * a.scale_log2;
    } else {
      qsc[qg] = ok ? a.q_scale[(q_row0 + qi[qg]) * Hq + qh[qg]] * a.scale_log2 : 0.0f;
    }
  }
  if constexpr (DENSE) {
    if (a.q_in != nullptr) {
      // the workgroup's rows are one 128-row query block of head hu_
      static_assert(QT == 128, "a dense workgroup holds one query block");
      __shared__ float s_qred[NW];
      const int64_t qseq = a.q_rows.packed ? (int64_t)a.q_rows.start(z) * a.q_st : (int64_t)z * a.q_sb;
      const float sq = a.q_in_bf16 ? quant_q_block<D, QG, NW, true>(a, qseq, hu_, Tq, qi, qf, s_qred)
                                   : quant_q_block<D, QG, NW, false>(a, qseq, hu_, Tq, qi, qf, s_qred);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) qsc[qg] = sq * a.scale_log2;
    }
  }
  const int wq_first = (r0 + wave * 16 * QG) / G;   // first query token of this wave
  if constexpr (QLDS) {
#pragma unroll
    for (int qg = 0; qg < QG; ++qg)
#pragma unroll
      for (int s = 0; s < KS; ++s) s_q[(wave * QG + qg) * KS + s][lane] = qf[qg][s];
  }

  float m_run[QG], l_run[QG];
  v4f O[QG][CG];
  v16f O8[PV8 ? D / 32 : 1];                   // FP8 P.V: 32 channels x the wave's 32 queries
  v16f L8;                                     // row sums of the FP8 P (every element of lane l: query l % 32)
#pragma unroll
  for (int c = 0; c < (PV8 ? D / 32 : 1); ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) O8[c][e] = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) L8[e] = 0.0f;
  v4f Ls[QG];                                  // row sums from the matrix units
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    m_run[qg] = kMRunInit;
    l_run[qg] = 0.0f;
    Ls[qg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CG; ++c) O[qg][c] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  v8h ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (_Float16)1.0f;

  int kv_end = kv_len;   // keys past kv_end are hidden from every query of the workgroup
  if constexpr (CAUSAL) kv_end = min(kv_len, (min(r0 + QT, Tq * G) - 1) / G + offset + 1);
  const int ntiles = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;

  // ---- tile staging: global -> registers -> LDS ---------------------------
  const int64_t k_head = (int64_t)kvh * D * 16;    // K bytes before this KV head in a block
  const int64_t k_blk = (int64_t)Hkv * D * 16;     // K bytes per physical block
  const uint32_t kblk32 = (uint32_t)k_blk;         // (< 2^32: Hkv <= 65535, D <= 256)
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // the same value, held in a scalar
  const uint32_t lane16 = (uint32_t)lane * 16u;                // each lane's 16 bytes of a 1 KB copy
  const uint32_t sk_lds = lds_addr(&s_k[0][0]), sv_lds = lds_addr(&s_v[0][0]);
  // VWS: this (sequence, KV head)'s fp16 V blocks in the workspace
  // [seq][logical block][Hkv][D][16]
  const uint8_t* vws_seq = VWS_ ? reinterpret_cast<const uint8_t*>(a.v_ws) + ((int64_t)z * a.max_blocks * Hkv + kvh) * D * 32
                                : nullptr;
  const uint32_t vblk32 = (uint32_t)(Hkv * D * 32);   // bytes per logical block (< 2^32)
  // Physical blocks of a paged tile: lanes 0..3 read the four block-table
  // entries with one vector load, issued one tile ahead of the fetch that
  // uses them (a vector load, so that waiting for LDS reads - lgkmcnt - never
  // waits for it), and the fetch reads them out with readlane.
  // The logical block is clamped to the sequence's last block and to the
  // table row, so no entry outside the row is read (context_lens beyond
  // max_blocks_per_seq * 16 breaks a documented precondition, but still reads
  // inside the row).
  const int blk_hi = DENSE ? 0 : min(last_blk, a.max_blocks - 1);
  auto load_blocks = [&](int tile) -> int {
    if constexpr (DENSE) return 0;
    else return trow[max(min(tile * 4 + (lane & 3), blk_hi), 0)];
  };
  using Blocks = v4i;
  auto unpack = [](int v) -> Blocks {
    return Blocks{__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 1),
                  __builtin_amdgcn_readlane(v, 2), __builtin_amdgcn_readlane(v, 3)};
  };
  auto pick = [](Blocks pb, int b) { return (b & 2) ? ((b & 1) ? pb[3] : pb[2]) : ((b & 1) ? pb[1] : pb[0]); };
  auto fetch = [&](St& st, int tile, Blocks pb, int kbuf) {
    // unit i of this thread lies in block (i*NT + 64*wave) / units-per-block of
    // the tile: wave-uniform, so its physical block is a scalar
    auto phys = [&](int b) -> int64_t {
      return DENSE ? blk_base + min(tile * 4 + b, last_blk) : (int64_t)pick(pb, b);
    };
    if constexpr (KDMA) {
      constexpr int KC = D / 64;                   // 1 KB chunks per K block (per head)
#pragma unroll
      for (int i = 0; i < (4 * KC + NW - 1) / NW; ++i) {
        const int c = wave_s + NW * i, b = c / KC, part = c % KC;
        if (4 * KC % NW != 0 && c >= 4 * KC) break;   // wave-uniform
        copy16_to_lds(a.k_blocks + (uint64_t)(uint32_t)pick(pb, b) * kblk32 + k_head + part * 1024, lane16,
                      sk_lds + (uint32_t)(kbuf * 4 * KBS + b * KBS + part * 1024));
      }
    }
#pragma unroll
    for (int i = 0; i < (KDMA ? 0 : KU); ++i) {
      if ((4 * KUB) % NT != 0 && i * NT + 64 * wave_s >= 4 * KUB) break;   // wave-uniform
      const int b = (i * NT + 64 * wave_s) / KUB;
      const int8_t* base = a.k_blocks + (uint64_t)(uint32_t)phys(b) * kblk32 + k_head;
      st.k[i] = *reinterpret_cast<const v4i*>(base + (uint32_t)((tid + i * NT) % KUB) * 16u);
    }
    if constexpr (VWS_) {
      // fp16 V blocks of this sequence from the workspace: block b of the
      // tile is logical block tile*4 + b, clamped like the block-table reads
      constexpr int VC = D / 32;                   // 1 KB chunks per V block (per head)
#pragma unroll
      for (int i = 0; i < (4 * VC + NW - 1) / NW; ++i) {
        const int c = wave_s + NW * i, b = c / VC, part = c % VC;
        if (4 * VC % NW != 0 && c >= 4 * VC) break;   // wave-uniform
        const int lb = max(min(tile * 4 + b, blk_hi), 0);
        copy16_to_lds(vws_seq + (uint64_t)(uint32_t)lb * vblk32 + part * 1024, lane16,
                      sv_lds + (uint32_t)(kbuf * KT * D * 2 + b * D * 32 + part * 1024));
      }
    }
#pragma unroll
    for (int i = 0; i < St::VUS; ++i) {
      if ((4 * VUB) % NT != 0 && i * NT + 64 * wave_s >= 4 * VUB) break;   // wave-uniform
      const int b = (i * NT + 64 * wave_s) / VUB;
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.v_blocks) + ((uint64_t)(uint32_t)phys(b) * kblk32 + k_head) * VB;
      st.v[i] = *reinterpret_cast<const v4i*>(base + (uint32_t)((tid + i * NT) % VUB) * 16u);
    }
    if constexpr (!DENSE) {
      if (tid < KT) {
        const int64_t si = ((int64_t)pick(pb, tid >> 4) * Hkv + kvh) * 16 + (tid & 15);
        st.ks = a.k_scale[si];
        st.vs = VK == kVI8 ? a.v_scale[si] : 0.0f;
      }
    }
  };
  auto commit = [&](const St& st, int buf, int tile) {
    const int kbase = tile * KT;
    const bool tail = kbase + KT > kv_len;       // the tile reaches past the context
#pragma unroll
    for (int i = 0; i < (KDMA ? 0 : KU); ++i) {
      if ((4 * KUB) % NT != 0 && i * NT + 64 * wave_s >= 4 * KUB) break;   // wave-uniform
      const int u = tid + i * NT;
      const int b = (i * NT + 64 * wave_s) / KUB;
      *reinterpret_cast<v4i*>(&s_k[buf][b * KBS + (u % KUB) * 16]) = st.k[i];
    }
    // V rows of keys past the context are cleared (the cache may hold anything there)
#pragma unroll
    for (int i = 0; i < St::VUS; ++i) {
      if ((4 * VUB) % NT != 0 && i * NT + 64 * wave_s >= 4 * VUB) break;   // wave-uniform
      const int u = tid + i * NT;
      const int b = (i * NT + 64 * wave_s) / VUB, r = u % VUB;
      const int ch = VB == 2 ? r >> 1 : r;          // channel of this unit
      const int row = (b * D + ch) * 16;            // fp16 element index of the channel row
      if constexpr (VB == 2) {
        const uint4 w = make_uint4(st.v[i][0], st.v[i][1], st.v[i][2], st.v[i][3]);
        v8h f = VK == kVF16 ? f16x8_from_u4(w) : bf16x8_to_f16x8(w);
        if (tail) {
          const int t_first = kbase + b * 16 + (r & 1) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t_first + e >= kv_len) f[e] = (_Float16)0.0f;
        }
        *reinterpret_cast<v8h*>(&s_v[buf][row + ((r & 1) << 3)]) = f;
      } else {
        const uint4 w = make_uint4(st.v[i][0], st.v[i][1], st.v[i][2], st.v[i][3]);
        v8h f0 = i8x8_to_f16x8(make_uint2(w.x, w.y));
        v8h f1 = i8x8_to_f16x8(make_uint2(w.z, w.w));
        if (tail) {
          const int t_first = kbase + b * 16;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (t_first + e >= kv_len) f0[e] = (_Float16)0.0f;
            if (t_first + 8 + e >= kv_len) f1[e] = (_Float16)0.0f;
          }
        }
        *reinterpret_cast<v8h*>(&s_v[buf][row]) = f0;
        *reinterpret_cast<v8h*>(&s_v[buf][row + 8]) = f1;
      }
    }
    if constexpr (!DENSE) {
      if (tid < KT) {
        const bool in = kbase + tid < kv_len;
        s_ks[buf][tid] = in ? st.ks : 0.0f;
        s_vs[buf][tid] = in ? st.vs : 0.0f;
      }
    }
  };

  // Dense inputs come from this library's own preprocessing, whose K and V
  // block layouts equal the LDS layouts, so
  // their tiles are copied straight from global memory into LDS by
  // global_load_lds_dwordx4: each wave moves 1 KB chunks (lane l's 16 bytes
  // land at chunk base + 16*l), with no staging registers and no LDS writes.
  // Blocks past the last one are clamped to it, as in fetch(). The copies go
  // through copy16_to_lds (inline assembly): issued with the builtin, the
  // compiler cannot tell the two LDS buffers apart and waits for the next
  // tile's copies before the first LDS read of the current one. The wait
  // before the end-of-tile barrier covers them.
  // Block b of tile t is the sequence's block min(4t + b, last_blk): a 32-bit
  // index times the per-block stride, added to the sequence's first block
  // (scalar arithmetic, no 64 x 64-bit products per copy).
  const int8_t* kseq = a.k_blocks + blk_base * k_blk + k_head;
  const uint8_t* vseq = reinterpret_cast<const uint8_t*>(a.v_blocks) + (blk_base * k_blk + k_head) * 2;
  // VTOK: this (sequence, KV head)'s 16-bit V rows; lane l of chunk q's copy
  // takes 16 bytes of token row vtok_dma_row(q, l) of the tile
  const uint8_t* vtok_seq = nullptr;
  uint32_t vtok_row = 0;
  uint32_t vtok_off[VTOK ? (kVtokChunks<D> + NW - 1) / NW : 1];
  if constexpr (VTOK) {
    const int64_t vrow0 = a.k_rows.packed ? (int64_t)a.k_rows.start(z) * a.v_st : (int64_t)z * a.v_sb;
    vtok_seq = reinterpret_cast<const uint8_t*>(a.v_tok) + (vrow0 + (int64_t)kvh * a.v_sh) * 2;
    vtok_row = (uint32_t)(a.v_st * 2);
    constexpr int LPR = D / 8;                     // lanes per token row
#pragma unroll
    for (int i = 0; i < (kVtokChunks<D> + NW - 1) / NW; ++i) {
      const int q = wave_s + NW * i;
      vtok_off[i] = (uint32_t)vtok_dma_row<D>(min(q, kVtokChunks<D> - 1), lane) * vtok_row + (uint32_t)(lane % LPR) * 16u;
    }
  }
  auto dma = [&](int buf, int tile) {
    constexpr int KC = D / 64;                     // 1 KB chunks per K block (per head)
    constexpr int VC = D / 32;                     // 1 KB chunks per V block (per head)
    auto blk = [&](int b) -> uint64_t { return (uint64_t)(uint32_t)min(tile * 4 + b, last_blk) * kblk32; };
#pragma unroll
    for (int i = 0; i < (4 * KC + NW - 1) / NW; ++i) {
      const int c = wave_s + NW * i, b = c / KC, part = c % KC;
      if (4 * KC % NW != 0 && c >= 4 * KC) break;   // wave-uniform
      copy16_to_lds(kseq + blk(b) + part * 1024, lane16, sk_lds + (uint32_t)(buf * 4 * KBS + b * KBS + part * 1024));
    }
    if constexpr (PV8) {
      // one E4M3 block of 64 keys: D rows of 64 bytes, D/16 chunks of 1 KB
      constexpr int V8C = D / 16;
      // The sequence's first block (Rows::block0 with 64-token blocks) is
      // derived here, per tile: a value kept across the loop costs the causal
      // d = 128 kernel spill reloads in it. The varlen offset is a scalar
      // (constant-memory) load, so that waiting for it waits for no copy.
      typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
      const int64_t seq0 = a.k_rows.packed ? (int64_t)(((const_i32_ptr)a.k_rows.cu)[z] / KT) + z
                                           : (int64_t)z * ((a.k_rows.N + KT - 1) / KT);
      const int64_t vb8 = seq0 + min(tile, (kv_len + KT - 1) / KT - 1);
      const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(a.v_blocks) + (vb8 * Hkv + kvh) * (int64_t)D * 64;
#pragma unroll
      for (int i = 0; i < (V8C + NW - 1) / NW; ++i) {
        const int c = wave_s + NW * i;
        if (V8C % NW != 0 && c >= V8C) break;   // wave-uniform
        copy16_to_lds(vsrc + c * 1024, lane16, sv_lds + (uint32_t)(buf * KT * D * 2 + c * 1024));
      }
    }
#pragma unroll
    for (int i = 0; i < (PV8 || VTOK ? 0 : (4 * VC + NW - 1) / NW); ++i) {
      const int c = wave_s + NW * i, b = c / VC, part = c % VC;
      if (4 * VC % NW != 0 && c >= 4 * VC) break;   // wave-uniform
      copy16_to_lds(vseq + 2 * blk(b) + part * 1024, lane16, sv_lds + (uint32_t)(buf * KT * D * 2 + b * D * 32 + part * 1024));
    }
    if constexpr (VTOK) {
      // chunk q of the tile's 16-bit V rows (the tile is clamped to the last
      // one, as the K blocks are)
      const int t = min(tile, (kv_len + KT - 1) / KT - 1);
      const uint8_t* src = vtok_seq + (uint64_t)(uint32_t)(t * KT) * vtok_row;
      const int vis = kv_len - t * KT;   // rows of the tile inside the sequence (>= 1)
      if (vis >= KT) {   // wave-uniform
#pragma unroll
        for (int i = 0; i < (kVtokChunks<D> + NW - 1) / NW; ++i) {
          const int q = wave_s + NW * i;
          if (kVtokChunks<D> % NW != 0 && q >= kVtokChunks<D>) break;   // wave-uniform
          copy16_to_lds(src, vtok_off[i], sv_lds + (uint32_t)(buf * (KT * D * 2 + 256)) + vtok_chunk<D>(q));
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < (kVtokChunks<D> + NW - 1) / NW; ++i) {
        const int q = wave_s + NW * i;
        if (kVtokChunks<D> % NW != 0 && q >= kVtokChunks<D>) break;   // wave-uniform
        // a partial last tile re-reads the sequence's last row for the rows
        // past the sequence: P is exactly 0 at those keys, so with finite V
        // they add 0 (a zero fill of LDS would make the compiler wait for
        // the copies in flight)
        const uint32_t off = (uint32_t)min(vtok_dma_row<D>(q, lane), vis - 1) * vtok_row + (uint32_t)(lane % (D / 8)) * 16u;
        copy16_to_lds(src, off, sv_lds + (uint32_t)(buf * (KT * D * 2 + 256)) + vtok_chunk<D>(q));
      }
    }
  };
  constexpr bool kDma = DENSE;
  // Raised wave priority (s_setprio) while a wave issues its matrix
  // products: measured faster for the dense kernels, slower for the paged
  // prefill, so dense only.
  constexpr int kPrio = DENSE ? kSetprio : 0;

  if (ntiles > 0) {
    if constexpr (kDma) {
      dma(0, 0);
    } else {
      St st;
      fetch(st, 0, unpack(load_blocks(0)), 0);
      commit(st, 0, 0);
    }
  }
  // on every path (the tile loop is reached from both), so that no load
  // issued so far is waited for inside the loop
  if constexpr (kDma || KDMA || VWS_) wait_vmem_all();
  __syncthreads();

  const int nkb = DENSE ? (kv_len + KT - 1) / KT : 1;
  // dense: key-block scales, read one tile ahead (a load issued and used in
  // the same tile would expose its latency every tile). Read as constant
  // memory (written before this kernel), so they come through scalar loads:
  // the wait for a vector load would also wait for the tile copies issued
  // after it.
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  const const_f32_ptr ksc = DENSE ? (const_f32_ptr)(a.k_scale + a.k_rows.scale_at(z, kvh, Hkv, 0, KT)) : nullptr;
  float tsc_next = 1.0f;
  if constexpr (DENSE) tsc_next = ntiles > 0 ? ksc[0] : 1.0f;
  int pb_next = ntiles > 0 ? load_blocks(1) : 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int kbase = tile * KT;
    // the next tile (past the last one the clamped blocks are re-read and the
    // spare buffer written but never used)
    // (issued after this tile's S^T products, see below)
    St nxt;
    const Blocks pb_cur = unpack(pb_next);
    if constexpr (!kDma) pb_next = load_blocks(tile + 2);

    float tsc = 1.0f;   // dense: key-block scale of this tile
    if constexpr (DENSE) {
      tsc = tsc_next;
      tsc_next = ksc[min(tile + 1, nkb - 1)];
    }

    // ---- S^T = K Q^T for the 64 keys x (16*QG) queries -------------------------
    // acc[qg][2*half + u][i] holds key 32*half + 8*g + 4*u + i of query n.
    // Dense: the accumulators start at the bit pattern of 1.5 * 2^23, so the
    // INT32 sum read as a float is 1.5 * 2^23 + dot exactly (the sum stays in
    // [2^23, 2^24), where floats are the integers, because |dot| <=
    // 127*127*256 = 4,129,024 < 2^22): no conversion instruction per score;
    // the offset is folded into the exponent's constant term.
    v4i acc[QG][4];
    if constexpr (kPrio & 1) __builtin_amdgcn_s_setprio(1);
    if constexpr (!DENSE) {
      // paged: K fragments stream through a ring of 4 registers, read 3
      // products ahead, the query fragments once per tile (a fence per
      // product keeps the compiler from reading further ahead, or later)
      auto kfrag = [&](int i) {                    // fragment i = KS*hu + s
        const int hu = i / KS, s = i % KS;
        const int tau = 32 * (hu >> 1) + 8 * (n >> 2) + 4 * (hu & 1) + (n & 3);
        return *reinterpret_cast<const v4i*>(&s_k[buf][(tau >> 4) * KBS + (tau & 15) * 16 + g * 256 + s * 1024]);
      };
      v4i qv[QG][KS];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int s = 0; s < KS; ++s) qv[qg][s] = QLDS ? s_q[(wave * QG + qg) * KS + s][lane] : qf[qg][s];
      constexpr int NF = 4 * KS, AHEAD = 3;
      v4i kf[4];
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) kf[i] = kfrag(i);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        if (i + AHEAD < NF) kf[(i + AHEAD) & 3] = kfrag(i + AHEAD);
        const int hu = i / KS, s = i % KS;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          acc[qg][hu] = mfma_i8(kf[i & 3], qv[qg][s], s == 0 ? v4i{0, 0, 0, 0} : acc[qg][hu]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int hu = 0; hu < (DENSE ? 4 : 0); ++hu) {
      const int tau = 32 * (hu >> 1) + 8 * (n >> 2) + 4 * (hu & 1) + (n & 3);
      const int8_t* kp = &s_k[buf][(tau >> 4) * KBS + (tau & 15) * 16 + g * 256];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) acc[qg][hu] = v4i{kAcc0, kAcc0, kAcc0, kAcc0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v4i kf = *reinterpret_cast<const v4i*>(kp + s * 1024);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          acc[qg][hu] = mfma_i8(kf, QLDS ? s_q[(wave * QG + qg) * KS + s][lane] : qf[qg][s], acc[qg][hu]);
      }
    }

    if constexpr (kPrio & 1) __builtin_amdgcn_s_setprio(0);
    // the next tile's loads and copies go out after the S^T products (issued
    // before them, they sit in front of every wave's first products; measured
    // 2-3% slower for the paged prefill, 0.3-1.3% for dense)
    if constexpr (kDma) dma(buf ^ 1, tile + 1);
    else fetch(nxt, tile + 1, pb_cur, buf ^ 1);
    // key of x[j] below: kbase + 32*(j/8) + 8*g + j%8
    const int tl = 8 * g;
    // masks only on tiles that cross the context end or the causal diagonal
    bool need_mask = kbase + KT > kv_len;
    if constexpr (CAUSAL) need_mask = need_mask || (kbase + KT - 1 > wq_first + offset);
    if constexpr (DENSE && !PV8) {
      // ---- dense: the softmax by key halves --------------------------------
      // P of keys 0..31 (both query groups) first; the P.V products of that
      // half then go out between the exponentials of keys 32..63, so that the
      // wave's matrix and vector work overlap. Hidden keys get x = -inf (their
      // P is exp2(-inf) = 0 before any product), which needs a positive tile
      // factor: a zero factor (a zero query or key block) scores every key 0,
      // and the smallest normal float in its place moves no score by an
      // amount a float resolves. One factor sQ_blk * sK_blk * scale for the
      // workgroup and tile, held as a scalar; the folded accumulator offset
      // costs half an ulp of offset*f in the exponent, so when offset*f >
      // 2^12 (scores of large-magnitude inputs) the offset is subtracted
      // exactly instead (bit patterns of positive floats compare like them).
      const int fwb = max(__builtin_amdgcn_readfirstlane(__float_as_int(qsc[0] * tsc)), 0x00800000);
      const float fw = __int_as_float(fwb);
      const bool exact_off = fwb > __float_as_int(4096.0f / kOffset);
      const float off = exact_off ? 0.0f : kOffset;
      float x[QG][16], cterm[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        // this lane's maximum of its raw accumulators (a chain of three-input
        // maxima; read as floats in [2^23, 2^24) they order like their bits)
        auto A = [&](int j) { return acc[qg][j >> 2][j & 3]; };
        int im = max(max(A(0), A(1)), A(2));
#pragma unroll
        for (int j = 3; j < 15; j += 2) im = max(max(im, A(j)), A(j + 1));
        im = max(im, A(15));
#pragma unroll
        for (int j = 0; j < 16; ++j) x[qg][j] = __int_as_float(A(j));
        // this lane's largest visible score
        float mt;
        if (need_mask) {
          const int pos = qi[qg] + offset;
          float mx = kNegInf;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int tk = kbase + 32 * (j >> 3) + tl + (j & 7);
            bool ok = tk < kv_len;
            if constexpr (CAUSAL) ok = ok && tk <= pos;
            x[qg][j] = ok ? x[qg][j] : kNegInf;
            mx = fmaxf(mx, x[qg][j]);
          }
          mt = mx == kNegInf ? kNegInf : (mx - kOffset) * fw;
        } else {
          mt = (__int_as_float(im) - kOffset) * fw;
        }
        if (exact_off) {
#pragma unroll
          for (int j = 0; j < 16; ++j) x[qg][j] -= kOffset;
        }
        // lazy rescale, tested on each lane's own maximum (see below)
        if (__any(mt > m_run[qg] + kRescaleSlack)) {
          const float m_new = fmaxf(m_run[qg], group4_max(mt));
          const float alpha = fast_exp2(m_run[qg] - m_new);
          l_run[qg] *= alpha;
          Ls[qg] *= alpha;
#pragma unroll
          for (int c = 0; c < CG; ++c) O[qg][c] *= alpha;
          m_run[qg] = m_new;
        }
        // x*f + cterm = score - reference
        cterm[qg] = -fmaf(off, fw, m_run[qg]);
      }
      // keys 0..31: O^T += V^T P^T and the row sums against an all-ones
      // block; keys 32..63: P, scheduled in between (the two products of a
      // channel group, then three vector instructions; measured against four
      // and five and against no pattern). fp16 V fragments come through a
      // ring of three registers, read two products ahead, the first two
      // before the exponentials of keys 0..31.
      const int so = 8 * (g & 1);
      auto vfrag = [&](int half, int c) -> v8h {
        if constexpr (VTOK) {
          // channel 16c + n, keys 32 half + 8g + 0..7: two transposing reads,
          // each of four token rows x 16 channels of the lane's 16-lane group
          const int row = 32 * half + 8 * g + (n >> 2), col = 16 * c + 4 * (n & 3);
          const char* b0 = reinterpret_cast<const char*>(&s_v[buf][0]);
          // (the results are taken as whole 32-bit words: built element by
          // element from the 16-bit results, the operand came out wrong)
          auto rd = [&](int r) {
            return __builtin_bit_cast(v2i32, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(b0 + vtok_row_off<D>(r) + col * 2)));
          };
          const v2i32 lo = rd(row), hi = rd(row + 4);
          return __builtin_bit_cast(v8h, v4i{lo[0], lo[1], hi[0], hi[1]});
        } else {
          const int vb = 2 * half + (g >> 1);
          return *reinterpret_cast<const v8h*>(&s_v[buf][(vb * D + 16 * c + n) * 16 + so]);
        }
      };
      v8h vr[3];
      vr[0] = vfrag(0, 0);
      vr[1] = vfrag(0, 1);
      v8h pf[QG][2];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(x[qg][j], fw, cterm[qg]));
        pf[qg][0] = pack8(p);
      }
      if constexpr (kPrio & 2) __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        if (c + 2 < CG) vr[(c + 2) % 3] = vfrag(0, c + 2);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) O[qg][c] = mfma_f16(vr[c % 3], pf[qg][0], O[qg][c]);
      }
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) Ls[qg] = mfma_f16(ones, pf[qg][0], Ls[qg]);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(x[qg][8 + j], fw, cterm[qg]));
        pf[qg][1] = pack8(p);
      }
#pragma unroll
      for (int c = 0; c <= CG; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, QG, 0);  // matrix products
        if (c < CG) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // vector instructions
      }
      __builtin_amdgcn_sched_barrier(0);
      // keys 32..63
      vr[0] = vfrag(1, 0);
      vr[1] = vfrag(1, 1);
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        if (c + 2 < CG) vr[(c + 2) % 3] = vfrag(1, c + 2);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) O[qg][c] = mfma_f16(vr[c % 3], pf[qg][1], O[qg][c]);
      }
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) Ls[qg] = mfma_f16(ones, pf[qg][1], Ls[qg]);
    } else {
      // ---- paged tiles, and dense tiles with the FP8 P.V product: P of all
      // 64 keys, then the products ----------------------------------------
      float sk[16], sv[16];
      if constexpr (!DENSE) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sk[j] = s_ks[buf][32 * (j >> 3) + tl + (j & 7)];
      }
      if constexpr (VK == kVI8) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sv[j] = s_vs[buf][32 * (j >> 3) + tl + (j & 7)];
      }

      // dense: one factor sQ_blk * sK_blk * scale for the whole workgroup and
      // tile (one 128-row query block, one key block), held as a scalar; the
      // folded accumulator offset costs half an ulp of offset*f in the
      // exponent, so when offset*f > 2^12 (scores of large-magnitude inputs)
      // the offset is subtracted exactly instead
      float fw = 0.0f;
      bool exact_off = false;
      if constexpr (DENSE) {
        fw = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(qsc[0] * tsc)));
        // (fw >= 0: compared as integer bits, in scalar registers)
        exact_off = kMagic && __float_as_int(fw) > __float_as_int(4096.0f / kOffset);
      }
      // dense: each lane's maximum of its raw accumulators (a chain of
      // three-input maxima; read as floats in [2^23, 2^24) they order like
      // their bit patterns)
      int imq[QG];
      if constexpr (DENSE) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          auto A = [&](int j) { return acc[qg][j >> 2][j & 3]; };
          int m = max(max(A(0), A(1)), A(2));
#pragma unroll
          for (int j = 3; j < 15; j += 2) m = max(max(m, A(j)), A(j + 1));
          imq[qg] = max(m, A(15));
        }
      }
      v8h pf[QG][2];
      uint32_t pk[QG][4];                          // FP8 P.V: byte j of word w is p[4w + j]
      float al8 = 1.0f;                            // FP8 P.V: rescale of this lane's query (32x32 layout)
      bool resc8 = false;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        // score_j = x[j] * f with one lane factor f >= 0 (dense: the Q and K
        // block scales; paged: the Q scale, sK folded into x)
        float x[16], f, mx;
        int im = 0;
        if constexpr (DENSE) {
          f = fw;
          im = imq[qg];
#pragma unroll
          for (int j = 0; j < 16; ++j) x[j] = kMagic ? __int_as_float(acc[qg][j >> 2][j & 3]) : (float)acc[qg][j >> 2][j & 3];
          mx = kMagic ? __int_as_float(im) : (float)im;
        } else {
          f = qsc[qg];
#pragma unroll
          for (int j = 0; j < 16; ++j) x[j] = (float)acc[qg][j >> 2][j & 3] * sk[j];
          mx = fmaxf(x[0], x[1]);
#pragma unroll
          for (int j = 2; j < 16; j += 2) mx = fmaxf(mx, fmaxf(x[j], x[j + 1]));
        }
        uint32_t vis = 0xFFFFu;   // visible keys of this lane (bit j: the key of x[j])
        if (need_mask) {
          const int pos = qi[qg] + offset;
          vis = 0;
          mx = kNegInf;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int tk = kbase + 32 * (j >> 3) + tl + (j & 7);
            bool ok = tk < kv_len;
            if constexpr (CAUSAL) ok = ok && tk <= pos;
            vis |= ok ? 1u << j : 0u;
            mx = ok ? fmaxf(mx, x[j]) : mx;
          }
        }
        float off = kMagic ? kOffset : 0.0f;
        if (exact_off) {
#pragma unroll
          for (int j = 0; j < 16; ++j) x[j] -= kOffset;
          mx -= kOffset;
          off = 0.0f;
        }
        // this lane's largest (visible) score
        float mt;
        if (DENSE && kMagic && !need_mask) mt = (__int_as_float(im) - kOffset) * f;
        else mt = mx == kNegInf ? kNegInf : (mx - off) * f;
        // lazy rescale: move the reference only when it is exceeded by > 2^8.
        // A row's maximum exceeds it exactly when one of the row's lanes holds
        // such a score, so the test needs no maximum across the lane groups;
        // that maximum is formed only when the reference moves.
        if (__any(mt > m_run[qg] + (PV8 ? kFp8Slack : kRescaleSlack))) {
          mt = group4_max(mt);
          const float m_new = fmaxf(m_run[qg], mt);
          const float alpha = fast_exp2(m_run[qg] - m_new);
          l_run[qg] *= alpha;
          if constexpr (PV8) {
            // lane l holds query l % 32 of the wave in the 32x32 accumulators;
            // both query groups are applied in one pass after this loop
            if (((lane >> 4) & 1) == qg) al8 = alpha;
            resc8 = true;
          } else {
            Ls[qg] *= alpha;
#pragma unroll
            for (int c = 0; c < CG; ++c) O[qg][c] *= alpha;
          }
          m_run[qg] = m_new;
        }
        const float mref = m_run[qg];
        // x*f + cterm = score - mref (FP8 P.V: + log2(448) - 3)
        const float cterm = -fmaf(off, f, mref) + (PV8 ? kFp8Log2Top : 0.0f);
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = fast_exp2(fmaf(x[j], f, cterm));
        if (need_mask) {
#pragma unroll
          for (int j = 0; j < 16; ++j) p[j] = (vis >> j) & 1u ? p[j] : 0.0f;
        }
        if constexpr (!kRowSumMfma) {
          float psum = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) psum += p[j];
          l_run[qg] += psum;
        }
        if constexpr (VK == kVI8) {
#pragma unroll
          for (int j = 0; j < 16; ++j) p[j] *= sv[j];   // fold the per-token V scale into P
        }
        if constexpr (PV8) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * w], p[4 * w + 1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * w + 2], p[4 * w + 3], word, true);
            pk[qg][w] = (uint32_t)word;
          }
        } else {
          pf[qg][0] = pack8(*reinterpret_cast<const float(*)[8]>(&p[0]));
          pf[qg][1] = pack8(*reinterpret_cast<const float(*)[8]>(&p[8]));
        }
      }

      // ---- O^T += V^T P^T (and the row sums against an all-ones block) ---------
      if constexpr (PV8) {
        if (resc8) {
#pragma unroll
          for (int c = 0; c < D / 32; ++c) O8[c] *= al8;
          L8 *= al8;
        }
      }
      if constexpr (kPrio & 2) __builtin_amdgcn_s_setprio(1);
      if constexpr (PV8) {
        // B = P^T for the wave's 32 queries: rows 0/1 of the 16-lane groups
        // exchange with rows 2/3 so that lane l holds query l % 32 (query group
        // (l / 16) % 2) and keys of lane groups 2*(l/32), 2*(l/32)+1 as bytes
        // 0..15 and 16..31 (v_permlane16_swap: odd rows of the first operand
        // trade places with even rows of the second).
        v8i_t bop;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const auto xy = __builtin_amdgcn_permlane16_swap(pk[0][w], pk[1][w], false, false);
          bop[w] = (int)xy[0];
          bop[4 + w] = (int)xy[1];
        }
        // A = V^T: lane l reads channel 32*cb + l%32, the same key chunks (the
        // V blocks store them swizzled by (channel / 4) % 4)
        const uint8_t* vt = reinterpret_cast<const uint8_t*>(s_v[buf]);
        const int hh = lane >> 5;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
          const int ch = 32 * cb + (lane & 31), sw = (ch >> 2) & 3;
          const v4i lo = *reinterpret_cast<const v4i*>(vt + ch * 64 + 16 * ((2 * hh) ^ sw));
          const v4i hi = *reinterpret_cast<const v4i*>(vt + ch * 64 + 16 * ((2 * hh + 1) ^ sw));
          const v8i_t aop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          O8[cb] = mfma_fp8_32x32x64(aop, bop, O8[cb]);
        }
        const v8i_t ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                             0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
        L8 = mfma_fp8_32x32x64(ones8, bop, L8);
      }
      if constexpr (!DENSE) {
        // paged: V fragments through a ring of 4 registers, 3 products ahead
        __builtin_amdgcn_sched_barrier(0);
        auto vfrag = [&](int i) {                    // fragment i = CG*half + c
          const int half = i / CG, c = i % CG;
          const int vb = 2 * half + (g >> 1), so = 8 * (g & 1);
          return *reinterpret_cast<const v8h*>(&s_v[buf][(vb * D + 16 * c + n) * 16 + so]);
        };
        constexpr int NV = 2 * CG, AV = 3;
        v8h vr[4];
#pragma unroll
        for (int i = 0; i < AV; ++i) vr[i] = vfrag(i);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (i + AV < NV) vr[(i + AV) & 3] = vfrag(i + AV);
          const int half = i / CG, c = i % CG;
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) O[qg][c] = mfma_f16(vr[i & 3], pf[qg][half], O[qg][c]);
          if (kRowSumMfma && c == CG - 1) {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) Ls[qg] = mfma_f16(ones, pf[qg][half], Ls[qg]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (kPrio & 2) __builtin_amdgcn_s_setprio(0);
    if constexpr (kDma) wait_vmem_all();   // the next tile has landed
    else commit(nxt, buf ^ 1, tile + 1);
    if constexpr (KDMA || VWS_) wait_vmem_all();   // K (and V) of the next tile have landed
    __syncthreads();
  }

  // ---- normalize and store ----------------------------------------------------
  if constexpr (PV8) {
    // lane l: query l % 32 (group (l/16) % 2, row l % 16); element 4*i4 + e of
    // O8[cb] is channel 32*cb + 8*i4 + 4*(l/32) + e
    const int qgl = (lane >> 4) & 1;
    const float l = L8[0];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi[qgl] < Tq) {
      const int64_t orow = a.q_rows.packed ? (q_row0 + qi[qgl]) * a.o_st
                                           : (int64_t)z * a.o_sb + (int64_t)qi[qgl] * a.o_st;
      const int64_t ob = orow + (int64_t)qh[qgl] * a.o_sh;
      const float* vsc = a.v8_scale + ((int64_t)z * Hkv + kvh) * D;
      const float* vmu = a.v_mean != nullptr && l > 0.0f ? a.v_mean + ((int64_t)z * Hkv + kvh) * D : nullptr;
      if (a.lse != nullptr && lane < 32) {
        const int64_t li = a.q_rows.row_at(z, qh[qgl], Hq, qi[qgl]);
        // l sums P * 448 * 2^-3: ln(sum exp(score)) = ln2 * (m + log2(l) - log2(448) + 3)
        float lse = l > 0.0f ? 0.69314718055994531f * (m_run[qgl] + log2f(l) - kFp8Log2Top) : kNegInf;
        if (a.lse_corr != nullptr) lse += a.lse_corr[li];
        a.lse[li] = lse;
      }
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int c0 = 32 * cb + 8 * i4 + 4 * (lane >> 5);
          const float4 sc4 = *reinterpret_cast<const float4*>(vsc + c0);
          v4f o = {O8[cb][4 * i4] * inv * sc4.x, O8[cb][4 * i4 + 1] * inv * sc4.y,
                   O8[cb][4 * i4 + 2] * inv * sc4.z, O8[cb][4 * i4 + 3] * inv * sc4.w};
          if (vmu != nullptr) {
            const float4 mu = *reinterpret_cast<const float4*>(vmu + c0);
            o[0] += mu.x;
            o[1] += mu.y;
            o[2] += mu.z;
            o[3] += mu.w;
          }
          const int64_t oi = ob + c0;
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
    return;
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const float l = kRowSumMfma ? Ls[qg][0] : group4_sum(l_run[qg]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi[qg] >= Tq) continue;
    int64_t ob;
    const float* vmu = nullptr;   // dense smooth_v: the V mean returns on rows that see a key
    if constexpr (DENSE) {
      const int64_t orow = a.q_rows.packed ? (q_row0 + qi[qg]) * a.o_st : (int64_t)z * a.o_sb + (int64_t)qi[qg] * a.o_st;
      ob = orow + (int64_t)qh[qg] * a.o_sh + 4 * g;
      if (a.v_mean != nullptr && l > 0.0f) vmu = a.v_mean + ((int64_t)z * Hkv + kvh) * D + 4 * g;
      if (a.lse != nullptr && g == 0) {
        // p = exp2(score * log2(e) - m_run) summed to l, so the natural-log
        // sum of exp(score) is ln2 * (m_run + log2 l)
        const int64_t li = a.q_rows.row_at(z, qh[qg], Hq, qi[qg]);
        float lse = l > 0.0f ? 0.69314718055994531f * (m_run[qg] + log2f(l)) : kNegInf;
        if (a.lse_corr != nullptr) lse += a.lse_corr[li];
        a.lse[li] = lse;
      }
    } else {
      ob = ((q_row0 + qi[qg]) * Hq + qh[qg]) * D + 4 * g;
    }
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      v4f o = O[qg][c] * inv;
      if (DENSE && vmu != nullptr) {
        const float4 mu = *reinterpret_cast<const float4*>(vmu + 16 * c);
        o[0] += mu.x;
        o[1] += mu.y;
        o[2] += mu.z;
        o[3] += mu.w;
      }
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

template <int D, int VK, bool DENSE, bool CAUSAL, bool PV8 = false, bool VWS = false>
hipError_t run_flash(const FlashArgs& a, hipStream_t st) {
  // d = 256: waves of 16 rows (one workgroup per CU: its double-buffered
  // tiles take 99 KB of LDS), 8 waves for dense, 12 for the paged prefill,
  // whose 192-row workgroups (32 tokens x 6 heads for 6:1 GQA) cut 2048
  // tokens x 24 heads into exactly one round of 256 workgroups; smaller
  // heads: four waves of 32 rows
  constexpr int QG = D == 256 ? 1 : kQG;
  constexpr int NW = D == 256 ? (DENSE ? kNWD256Dense : kNWD256Paged) : kNW;
  constexpr int QT = NW * 16 * QG;
  const int G = DENSE ? 1 : a.G;
  const int qtiles = (int)(((int64_t)(DENSE ? a.Nq : a.max_seqlen_q) * G + QT - 1) / QT);
  if (qtiles == 0 || a.num_seqs == 0) return hipSuccess;
  int64_t total = (int64_t)qtiles * (DENSE ? a.Hq : a.Hkv) * a.num_seqs;
  if (DENSE && a.q_rows.packed) {
    if (QT != 128) return hipErrorInvalidValue;   // the map is of 128-row query blocks
    total = a.q_rows.nblocks(QT) * a.Hq;
  }
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  if constexpr (PV8) {
    if constexpr (QG == 2 && D <= 128) k_flash<D, QG, NW, VK, DENSE, CAUSAL, true><<<dim3((unsigned)total), NW * 64, 0, st>>>(a);
    else return hipErrorInvalidValue;    // FP8 P.V needs two query groups per wave
  } else if (DENSE && a.v_tok != nullptr) {
    k_flash<D, QG, NW, VK, DENSE, CAUSAL, false, false, DENSE><<<dim3((unsigned)total), NW * 64, 0, st>>>(a);
  } else {
    k_flash<D, QG, NW, VK, DENSE, CAUSAL, false, VWS><<<dim3((unsigned)total), NW * 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

// The V of each paged sequence in the attention kernel's LDS layout, once per
// call: fp16 blocks [seq][logical block][Hkv][D][16 tokens] in the workspace
// (bf16 rounded to fp16 and INT8 codes exactly, the tile staging's own
// conversions), tokens past the context zero. Workgroup (logical block, KV
// head, sequence); unit u = tokens 8*(u%2) .. +7 of channel u/2. Blocks past
// the context are not written (the kernel never reads them).
template <int D, bool VI8>
__global__ __launch_bounds__(256) void k_v16_blocks(FlashArgs a) {
  const int lb = blockIdx.x, kvh = blockIdx.y, z = blockIdx.z;
  const int ctx = a.ctx_lens[z];
  if (lb * 16 >= ctx) return;
  const int64_t bh = (int64_t)a.tables[(int64_t)z * a.max_blocks + lb] * a.Hkv + kvh;
  _Float16* dst = reinterpret_cast<_Float16*>(a.v_ws) + (((int64_t)z * a.max_blocks + lb) * a.Hkv + kvh) * D * 16;
  for (int u = threadIdx.x; u < 2 * D; u += 256) {
    const int ch = u >> 1, h = u & 1;
    v8h f;
    if constexpr (VI8) {
      f = i8x8_to_f16x8(*reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(a.v_blocks) +
                                                        (bh * D + ch) * 16 + 8 * h));
    } else {
      f = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v_blocks) +
                                                          (bh * D + ch) * 16 + 8 * h));
    }
    const int t0 = lb * 16 + 8 * h;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (t0 + e >= ctx) f[e] = (_Float16)0.0f;
    *reinterpret_cast<v8h*>(dst + ch * 16 + 8 * h) = f;
  }
}

template <int D>
hipError_t flash_d(const FlashArgs& a, hipStream_t st) {
  // dense V blocks are always fp16 (the preprocessing converts bf16), or E4M3
  if (a.dense && a.pv_fp8)
    return a.causal ? run_flash<D, kVF16, true, true, true>(a, st) : run_flash<D, kVF16, true, false, true>(a, st);
  if (a.dense) return a.causal ? run_flash<D, kVF16, true, true>(a, st) : run_flash<D, kVF16, true, false>(a, st);
  if (a.v_ws != nullptr) {
    // paged prefill with V converted once into the workspace
    const dim3 g((unsigned)a.max_blocks, (unsigned)a.Hkv, (unsigned)a.num_seqs);
    if (a.v_int8) k_v16_blocks<D, true><<<g, 256, 0, st>>>(a);
    else k_v16_blocks<D, false><<<g, 256, 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return a.v_int8 ? run_flash<D, kVI8, false, true, false, true>(a, st)
                    : run_flash<D, kVBf16, false, true, false, true>(a, st);
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
