// Quantization and cache-writing kernels (memory-bound).
//
// Row rule ([QK-MMAC] §1, §2.1, §4): s = fl32(max|x| / 127), code =
// clamp(rne(fl32(x / s)), -127, 127), with correctly rounded fp32 divisions.
// A zero row gets s = 0 and zero codes.
#include "common.h"
#include "quant.h"
#include "internal.h"

namespace qa {
namespace {

// Load E consecutive 16-bit values (E = 1, 2, 4) from a 2E-byte aligned address.
template <int E, bool BF16>
__device__ __forceinline__ void load_halves(const uint16_t* p, float (&v)[E]) {
  if constexpr (E == 4) {
    uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = half_to_f32<BF16>(w.x & 0xFFFFu);
    v[1] = half_to_f32<BF16>(w.x >> 16);
    v[2] = half_to_f32<BF16>(w.y & 0xFFFFu);
    v[3] = half_to_f32<BF16>(w.y >> 16);
  } else if constexpr (E == 2) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = half_to_f32<BF16>(w & 0xFFFFu);
    v[1] = half_to_f32<BF16>(w >> 16);
  } else {
    v[0] = half_to_f32<BF16>(*p);
  }
}

template <int E>
__device__ __forceinline__ void store_codes(int8_t* p, uint32_t packed) {
  if constexpr (E == 4) *reinterpret_cast<uint32_t*>(p) = packed;
  else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(p) = (uint16_t)packed;
  else *reinterpret_cast<uint8_t*>(p) = (uint8_t)packed;
}

// Quantize E values held by one lane against the wave-wide scale of its row
// (amax the row's largest |x|, s = quant_scale(amax)).
template <int E>
__device__ __forceinline__ uint32_t quant_lane(const float (&v)[E], float amax, float s) {
  uint32_t w[1];
  quant_bytes<E>(v, amax, s, __fdiv_rn(1.0f, s), w);
  return w[0];
}

// Quantize one (token, head) row of head_dim values with one wave.
template <int D, bool BF16>
__device__ __forceinline__ void quant_row(const uint16_t* __restrict__ x, int64_t row, int32_t H, int64_t st,
                                          int64_t sh, int8_t* __restrict__ q, float* __restrict__ scale,
                                          int lane, const Rope& rope = Rope{}) {
  constexpr int E = D / 64;
  const int64_t t = row / H;
  const int h = (int)(row - t * H);
  float v[E];
  const uint16_t* src = x + t * st + (int64_t)h * sh;
  load_halves<E, BF16>(src + lane * E, v);
  if (rope.pos != nullptr) rope_lane<E, BF16>(src, lane * E, v, rope.cs + rope.pos[t] * rope.rot, rope.rot, rope.neox);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = wave_max(amax);
  const float s = quant_scale(amax);
  store_codes<E>(q + row * D + lane * E, quant_lane<E>(v, amax, s));
  if (lane == 0) scale[row] = s;
}

// Write one (token, KV head) row: K -> INT8 codes in [blk, h, D/16, 16, 16] plus
// a per-token scale; V copied (or quantized) into [blk, h, D, 16].
template <int D, bool BF16, bool V_I8>
__device__ __forceinline__ void write_kv_row(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                             int64_t row, int32_t H, int64_t st, int64_t sh,
                                             const int64_t* __restrict__ slots, int8_t* __restrict__ kc,
                                             float* __restrict__ ks, void* __restrict__ vc,
                                             float* __restrict__ vs, int lane, const Rope& rope = Rope{}) {
  constexpr int E = D / 64;
  const int64_t t = row / H;
  const int h = (int)(row - t * H);
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t bh = blk * H + h;
  const int64_t src = t * st + (int64_t)h * sh + lane * E;

  float kv[E];
  load_halves<E, BF16>(k + src, kv);
  if (rope.pos != nullptr)
    rope_lane<E, BF16>(k + (src - lane * E), lane * E, kv, rope.cs + rope.pos[t] * rope.rot, rope.rot, rope.neox);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(kv[e]));
  amax = wave_max(amax);
  const float s = quant_scale(amax);
  // channels lane*E .. lane*E+E-1 share one 16-channel chunk
  const int ch = lane * E;
  store_codes<E>(kc + (bh * (D / 16) + ch / 16) * 256 + off * 16 + (ch % 16), quant_lane<E>(kv, amax, s));
  if (lane == 0) ks[bh * 16 + off] = s;

  if constexpr (V_I8) {
    float vv[E];
    load_halves<E, BF16>(v + src, vv);
    float vmax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) vmax = fmaxf(vmax, fabsf(vv[e]));
    vmax = wave_max(vmax);
    const float sv = quant_scale(vmax);
    int8_t* vd = reinterpret_cast<int8_t*>(vc);
    const uint32_t codes = quant_lane<E>(vv, vmax, sv);
#pragma unroll
    for (int e = 0; e < E; ++e) vd[(bh * D + ch + e) * 16 + off] = (int8_t)(codes >> (8 * e));
    if (lane == 0) vs[bh * 16 + off] = sv;
  } else {
    uint16_t* vd = reinterpret_cast<uint16_t*>(vc);
#pragma unroll
    for (int e = 0; e < E; ++e) vd[(bh * D + ch + e) * 16 + off] = v[src + e];
  }
}

// Rows held by 16 lanes: lane li of a 16-lane row holds D/16 channels of
// one (token, head) row, in pieces of kPieceLen consecutive channels
// (16-byte loads for D >= 128); piece p starts at channel (16p + li) *
// kPieceLen, so each load instruction of the row reads one contiguous span.
template <int D>
constexpr int kPieceLen = D >= 128 ? 8 : D / 16;
template <int D>
constexpr int kPieces = D / 16 / kPieceLen<D>;
template <int D>
__device__ __forceinline__ int piece_ch(int li, int p) { return (16 * p + li) * kPieceLen<D>; }

// The lane's D/16 16-bit values of `row`, two per word, in channel order.
template <int D>
__device__ __forceinline__ void load_row16(const uint16_t* row, int li, uint32_t (&w)[D / 32]) {
  constexpr int PL = kPieceLen<D>;
#pragma unroll
  for (int p = 0; p < kPieces<D>; ++p) {
    if constexpr (PL == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + piece_ch<D>(li, p));
      w[4 * p] = u.x; w[4 * p + 1] = u.y; w[4 * p + 2] = u.z; w[4 * p + 3] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(row + piece_ch<D>(li, p));
      w[2 * p] = u.x; w[2 * p + 1] = u.y;
    }
  }
}

template <int N, bool BF16>
__device__ __forceinline__ float unpack_absmax(const uint32_t (&w)[N / 2], float (&v)[N]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    v[i] = half_to_f32<BF16>(i & 1 ? w[i / 2] >> 16 : w[i / 2] & 0xFFFFu);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  return amax;
}

// The lane's codes (quant_bytes words, channel order) to row / block memory:
// piece p goes to dst(p), 8 (or 4) bytes.
template <int D, typename F>
__device__ __forceinline__ void store_pieces(const uint32_t (&c)[D / 64], F dst) {
  constexpr int PL = kPieceLen<D>;
#pragma unroll
  for (int p = 0; p < kPieces<D>; ++p) {
    if constexpr (PL == 8) *reinterpret_cast<uint2*>(dst(p)) = make_uint2(c[2 * p], c[2 * p + 1]);
    else *reinterpret_cast<uint32_t*>(dst(p)) = c[p];
  }
}

// Each wave quantizes groups of 4 (token, head) rows, 16 lanes per row:
// group g holds rows 4g .. 4g+3, and the waves of the grid take the groups
// round-robin (wave w: groups w, w + nw, ...), loading the next group while
// they quantize the current one, so that the loads of one group overlap the
// arithmetic of the previous (in a single pass every wave would load, then
// every wave compute, with memory idle meanwhile). The row maximum is
// reduced inside its 16 lanes through DPP (no LDS); the codes are
// quant_bytes', i.e. those of quant_code.
// Row 4*grp + sub (clamped to the last row: rows past the end re-read it and
// are not stored). The division by H is done once per wave on the scalar
// unit for the group's first row; each lane then steps over at most
// sub / H + 1 token boundaries.
template <int D, bool BF16>
__device__ __forceinline__ void load_row_group(const uint16_t* __restrict__ x, int64_t rows, int32_t H, int64_t st,
                                               int64_t sh, int64_t grp, int sub, int li, uint32_t (&w)[D / 32]) {
  const int64_t r0 = __builtin_amdgcn_readfirstlane((uint32_t)(4 * grp)) |
                     ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((4 * grp) >> 32)) << 32);
  const int64_t t0 = r0 / H;                        // wave-uniform
  const int h0 = (int)(r0 - t0 * H);
  int64_t t = t0;
  int h = h0 + (int)(min(r0 + sub, rows - 1) - r0);
  while (h >= H) {                                  // at most 3 steps (sub < 4)
    h -= H;
    ++t;
  }
  load_row16<D>(x + t * st + (int64_t)h * sh, li, w);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                       int32_t H, int64_t st, int64_t sh,
                                                       int8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int E = D / 16;
  const int lane = threadIdx.x & 63, li = lane & 15, sub = lane >> 4;
  const int64_t ngroups = (rows + 3) / 4;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= ngroups) return;                      // the whole wave
  uint32_t w[D / 32];
  load_row_group<D, BF16>(x, rows, H, st, sh, grp, sub, li, w);
  for (; grp < ngroups; grp += nw) {
    float v[E];
    const float amax_l = unpack_absmax<E, BF16>(w, v);
    if (grp + nw < ngroups) load_row_group<D, BF16>(x, rows, H, st, sh, grp + nw, sub, li, w);
    const int64_t row = 4 * grp + sub;
    const float amax = row16_max(amax_l);
    const float s = quant_scale(amax);
    uint32_t c[E / 4];
    quant_bytes<E>(v, amax, s, __fdiv_rn(1.0f, s), c);
    if (row < rows) {
      store_pieces<D>(c, [&](int p) { return q + row * D + piece_ch<D>(li, p); });
      if (li == 0) scale[row] = s;
    }
  }
}

template <int D, bool BF16, bool V_I8>
__global__ __launch_bounds__(256) void k_write_kv(const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v, int64_t rows,
                                                  int32_t H, int64_t st, int64_t sh,
                                                  const int64_t* __restrict__ slots,
                                                  int8_t* __restrict__ kc, float* __restrict__ ks,
                                                  void* __restrict__ vc, float* __restrict__ vs) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  write_kv_row<D, BF16, V_I8>(k, v, row, H, st, sh, slots, kc, ks, vc, vs, threadIdx.x & 63);
}

// The cache write for runs of tokens: workgroup (group of 16 tokens, head).
// When the group's 16 slots are the 16 slots of one cache block in order
// (slot_j = 16*blk + j: a chunk written from a block boundary), each wave
// quantizes 4 token rows (16 lanes each), the codes and V values are gathered in LDS in the
// block's own layout, and the workgroup then writes the K block (D*16 bytes)
// and the V block (D*16 values) as contiguous 16-byte pieces: a token's V
// row alone lands in D places 32 (16) bytes apart, which costs a memory
// transaction per 2 (1) bytes. Any other group (unaligned, partly skipped,
// the ragged end) writes its rows one by one as k_write_kv does. The codes
// and scales are those of write_kv_row in either case.
template <int D, bool BF16, bool V_I8>
__global__ __launch_bounds__(256) void k_write_kv_blocks(const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int64_t T,
                                                         int32_t H, int64_t st, int64_t sh,
                                                         const int64_t* __restrict__ slots,
                                                         int8_t* __restrict__ kc, float* __restrict__ ks,
                                                         void* __restrict__ vc, float* __restrict__ vs) {
  constexpr int VB = V_I8 ? 1 : 2;                  // bytes per cached V value
  __shared__ __attribute__((aligned(16))) int8_t s_k[D * 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[D * 16 * VB];
  __shared__ float s_ks[16], s_vs[16];
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the group is a whole block in order when every lane j < 16 finds slot t0 + j = slot t0 + j
  int64_t slot0 = -1;
  bool whole = t0 + 16 <= T;
  if (whole) {
    slot0 = slots[t0];
    const int64_t sj = lane < 16 ? slots[t0 + lane] : slot0 + lane;
    whole = slot0 >= 0 && (slot0 & 15) == 0 && __all(sj == slot0 + lane);
  }
  if (!whole) {
    for (int j = wave; j < 16; j += 4) {
      const int64_t t = t0 + j;
      if (t < T) write_kv_row<D, BF16, V_I8>(k, v, t * H + h, H, st, sh, slots, kc, ks, vc, vs, lane);
    }
    return;
  }
  // 16 lanes per token: wave w holds tokens 4w .. 4w+3 of the group, every
  // K and V load issued before any is used; row maxima through DPP
  constexpr int N = D / 16;
  const int li = lane & 15, j = 4 * wave + (lane >> 4);
  const int64_t src = (t0 + j) * st + (int64_t)h * sh;
  uint32_t kw[D / 32], vw[D / 32];
  load_row16<D>(k + src, li, kw);
  load_row16<D>(v + src, li, vw);
  {
    float kv[N];
    const float amax = row16_max(unpack_absmax<N, BF16>(kw, kv));
    const float sk = quant_scale(amax);
    uint32_t c[N / 4];
    quant_bytes<N>(kv, amax, sk, __fdiv_rn(1.0f, sk), c);
    // channel ch of token j sits at (ch / 16) * 256 + j * 16 + ch % 16 of the K block
    store_pieces<D>(c, [&](int p) {
      const int ch = piece_ch<D>(li, p);
      return s_k + (ch / 16) * 256 + j * 16 + (ch % 16);
    });
    if (li == 0) s_ks[j] = sk;
  }
  // V: channel ch of token j at ch * 16 + j of the V block
  if constexpr (V_I8) {
    float vv[N];
    const float vmax = row16_max(unpack_absmax<N, BF16>(vw, vv));
    const float sv = quant_scale(vmax);
    uint32_t c[N / 4];
    quant_bytes<N>(vv, vmax, sv, __fdiv_rn(1.0f, sv), c);
#pragma unroll
    for (int i = 0; i < N; ++i)
      s_v[(piece_ch<D>(li, i / kPieceLen<D>) + i % kPieceLen<D>) * 16 + j] = (uint8_t)(c[i / 4] >> (8 * (i % 4)));
    if (li == 0) s_vs[j] = sv;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i)
      reinterpret_cast<uint16_t*>(s_v)[(piece_ch<D>(li, i / kPieceLen<D>) + i % kPieceLen<D>) * 16 + j] =
          (uint16_t)(i & 1 ? vw[i / 2] >> 16 : vw[i / 2] & 0xFFFFu);
  }
  __syncthreads();
  const int64_t bh = (slot0 >> 4) * H + h;
  uint4* kd = reinterpret_cast<uint4*>(kc + bh * (D * 16));
  for (int u = threadIdx.x; u < D; u += 256) kd[u] = reinterpret_cast<const uint4*>(s_k)[u];
  uint4* vd = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(vc) + bh * (D * 16 * VB));
  for (int u = threadIdx.x; u < D * VB; u += 256) vd[u] = reinterpret_cast<const uint4*>(s_v)[u];
  if (threadIdx.x < 16) {
    ks[bh * 16 + threadIdx.x] = s_ks[threadIdx.x];
    if constexpr (V_I8) vs[bh * 16 + threadIdx.x] = s_vs[threadIdx.x];
  }
}

// Fused producer: workgroups [0, qblocks) quantize query rows, the rest write
// K/V rows into the cache (one launch for both).
template <int D, bool BF16, bool V_I8>
__global__ __launch_bounds__(256) void k_producer(ProducerArgs a, int64_t qblocks) {
  const int lane = threadIdx.x & 63;
  if ((int64_t)blockIdx.x < qblocks) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row < a.q_rows)
      quant_row<D, BF16>((const uint16_t*)a.q, row, a.Hq, a.q_st, a.q_sh, a.q_i8, a.q_scale, lane, a.rope);
  } else {
    const int64_t row = ((int64_t)blockIdx.x - qblocks) * 4 + (threadIdx.x >> 6);
    if (row < a.kv_rows)
      write_kv_row<D, BF16, V_I8>((const uint16_t*)a.k, (const uint16_t*)a.v, row, a.Hkv, a.kv_st, a.kv_sh,
                                  a.slots, a.k_cache, a.k_scale, a.v_cache, a.v_scale, lane, a.rope);
  }
}

// ---------------------------------------------------------------------------
// SageAttention-style preprocessing
// ---------------------------------------------------------------------------

constexpr int kSumChunk = 64;  // tokens per partial column sum (= the K block, so varlen chunks share its map)

// Sequence and block of this workgroup. Batched grids are (heads, blocks, B),
// heads fastest so that consecutive workgroups read neighbouring pieces of the
// same token rows; varlen grids run over all packed blocks,
// (rows.nblocks(R), heads), and map[j] names the sequence of packed block j
// (-1 for the gap before a sequence): only workgroups with work are launched
// beyond one per gap. head_of gives the head index of either grid.
struct BlockRef {
  int b, blk;
};
__device__ __forceinline__ int head_of(const Rows& rows) { return rows.packed ? (int)blockIdx.y : (int)blockIdx.x; }
__device__ __forceinline__ BlockRef block_of(const Rows& rows, const int32_t* map, int R, int zdim_b) {
  if (!rows.packed) return {zdim_b, (int)blockIdx.y};
  const int b = map[blockIdx.x];
  if (b < 0 || b >= rows.B) return {-1, 0};
  return {b, (int)(blockIdx.x - rows.block0(b, R))};
}

// map[j] = b for the packed R-row blocks j of sequence b, -1 for the blocks of
// the gap before the next sequence; one workgroup per sequence, and the
// ranges of the sequences partition [0, rows.nblocks(R)).
__global__ __launch_bounds__(256) void k_block_map(Rows rows, int32_t R, int32_t* __restrict__ map) {
  const int b = blockIdx.x;
  const int64_t j0 = rows.block0(b, R);
  const int64_t j1 = b + 1 < rows.B ? rows.block0(b + 1, R) : rows.nblocks(R);
  const int64_t nb = (rows.len(b) + R - 1) / R;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) map[j] = j - j0 < nb ? b : -1;
}

// partial[b][chunk][c] = sum over the chunk's tokens of K[b, t, c], c in [0, Hkv*D),
// accumulated in fp64. Every K value is a multiple of 2^-24 (f16) or of a power
// of two bounded by its exponent (bf16), and the sums stay far below 2^53 units,
// so every partial sum is exact and the total does not depend on the order.
// (b, t, h, c) of k lives at b*sb + t*st + h*sh + c (batched) or at
// (rows.start(b) + t)*st + h*sh + c (varlen). Chunks are counted from the
// start of each sequence; chunks past its end hold zeros.
// ABSMAX: the chunk's largest |fl32(x - mu[b, c])| instead of the sum (mu
// optional), for the per-channel FP8 scale of V.
// A workgroup covers 64 groups of 8 columns and one chunk; its four waves
// take the chunk's rows in four interleaved slices, every row load of a thread
// in flight at once, and meet through LDS.
constexpr int kSumSlices = 4;
constexpr int kSumCols = 64 * 8;   // columns per workgroup

template <bool BF16, bool ABSMAX = false>
__global__ __launch_bounds__(256) void k_colsum(const uint16_t* __restrict__ k, Rows rows, const int32_t* map,
                                                int32_t D, int32_t HD, int64_t sb, int64_t st, int64_t sh,
                                                double* __restrict__ partial, const float* __restrict__ mu = nullptr) {
  constexpr int RPS = kSumChunk / kSumSlices;   // rows per slice
  __shared__ double red[kSumSlices - 1][8][64];
  const int chunks = (rows.N + kSumChunk - 1) / kSumChunk;
  // batched grid (column groups, chunks, B); varlen (packed chunks, column groups)
  int b = blockIdx.z, chunk = blockIdx.y, cg = blockIdx.x;
  if (rows.packed) {
    const int j = blockIdx.x;
    b = map[j];
    if (b < 0 || b >= rows.B) return;
    chunk = (int)(j - rows.block0(b, kSumChunk));
    cg = blockIdx.y;
  }
  const int sl = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c8 = (cg * 64 + lane) * 8;
  const bool live = c8 < HD;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int t0 = chunk * kSumChunk, t1 = min(t0 + kSumChunk, rows.len(b));
  const int64_t seq0 = rows.packed ? rows.start(b) * st : (int64_t)b * sb;
  const uint16_t* base = k + seq0 + (int64_t)(live ? c8 / D : 0) * sh + (live ? c8 % D : 0);
  float m8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ABSMAX && mu != nullptr && live) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m8[i] = mu[(int64_t)b * HD + c8 + i];
  }
  auto add = [&](uint4 w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = half_to_f32<BF16>(ws[i] & 0xFFFFu), hi = half_to_f32<BF16>(ws[i] >> 16);
      if constexpr (ABSMAX) {
        acc[2 * i] = fmax(acc[2 * i], (double)fabsf(lo - m8[2 * i]));
        acc[2 * i + 1] = fmax(acc[2 * i + 1], (double)fabsf(hi - m8[2 * i + 1]));
      } else {
        acc[2 * i] += (double)lo;
        acc[2 * i + 1] += (double)hi;
      }
    }
  };
  // rows t0 + sl + 4i of the slice (past the chunk: the last row, not added)
  if (live && t1 > t0) {
    uint4 w[RPS];
#pragma unroll
    for (int i = 0; i < RPS; ++i)
      w[i] = *reinterpret_cast<const uint4*>(base + (int64_t)min(t0 + sl + kSumSlices * i, t1 - 1) * st);
#pragma unroll
    for (int i = 0; i < RPS; ++i)
      if (t0 + sl + kSumSlices * i < t1) add(w[i]);
  }
  if (sl > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[sl - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (sl > 0 || !live) return;
#pragma unroll
  for (int s2 = 0; s2 < kSumSlices - 1; ++s2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = ABSMAX ? fmax(acc[i], red[s2][i][lane]) : acc[i] + red[s2][i][lane];
  }
  double* dst = partial + ((int64_t)b * chunks + chunk) * HD + c8;
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = acc[i];
}

// The column reductions below (the smooth_k / smooth_v mean, the FP8 V
// scale): a workgroup covers kRedCols columns, kRedSlices threads per column
// each take every kRedSlices-th chunk partial (loads unrolled, all in flight),
// then the slices meet through LDS. The sums are exact (see k_colsum) and the
// maxima exact, so the order does not matter.
constexpr int kRedCols = 16, kRedSlices = 16;

template <bool MAX>
__device__ __forceinline__ double reduce_column(const double* __restrict__ p, int32_t HD, int used, int slice) {
  double acc = 0.0;
  int j = slice;
  for (; j + 7 * kRedSlices < used; j += 8 * kRedSlices) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(j + u * kRedSlices) * HD];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = MAX ? fmax(acc, v[u]) : acc + v[u];
  }
  for (; j < used; j += kRedSlices) acc = MAX ? fmax(acc, p[(int64_t)j * HD]) : acc + p[(int64_t)j * HD];
  return acc;
}

// mu[b][c] = fl32(fl64(sum / Nk_b)); zeros when smoothing is off or the
// sequence is empty.
__global__ __launch_bounds__(256) void k_mean(const double* __restrict__ partial, Rows rows,
                                              int32_t HD, bool smooth, float* __restrict__ mean) {
  __shared__ double red[kRedSlices][kRedCols];
  const int col = threadIdx.x % kRedCols, slice = threadIdx.x / kRedCols;
  const int64_t i = (int64_t)blockIdx.x * kRedCols + col;   // b * HD + c
  const bool live = i < (int64_t)rows.B * HD;
  const int b = live ? (int)(i / HD) : 0;
  const int Nk = live ? rows.len(b) : 0;
  double s = 0.0;
  if (live && smooth && Nk > 0) {
    const int c = (int)(i % HD);
    const int chunks = (rows.N + kSumChunk - 1) / kSumChunk;
    s = reduce_column<false>(partial + (int64_t)b * chunks * HD + c, HD, (Nk + kSumChunk - 1) / kSumChunk, slice);
  }
  red[slice][col] = s;
  __syncthreads();
  if (slice == 0 && live) {
    if (!smooth || Nk <= 0) {
      mean[i] = 0.0f;
    } else {
      double tot = 0.0;
#pragma unroll
      for (int k = 0; k < kRedSlices; ++k) tot += red[k][col];
      mean[i] = (float)(tot / (double)Nk);
    }
  }
}

// FP8 scale of V per (b, KV head, channel): fl32(max |V'| / 448) from the
// chunk maxima of k_colsum<.., true> (0 for an empty sequence).
__global__ __launch_bounds__(256) void k_vscale(const double* __restrict__ partial, Rows rows, int32_t HD,
                                                float* __restrict__ vscale) {
  __shared__ double red[kRedSlices][kRedCols];
  const int col = threadIdx.x % kRedCols, slice = threadIdx.x / kRedCols;
  const int64_t i = (int64_t)blockIdx.x * kRedCols + col;   // b * HD + c
  const bool live = i < (int64_t)rows.B * HD;
  double m = 0.0;
  if (live) {
    const int b = (int)(i / HD), c = (int)(i % HD);
    const int chunks = (rows.N + kSumChunk - 1) / kSumChunk;
    const int used = (rows.len(b) + kSumChunk - 1) / kSumChunk;
    m = reduce_column<true>(partial + (int64_t)b * chunks * HD + c, HD, used, slice);
  }
  red[slice][col] = m;
  __syncthreads();
  if (slice == 0 && live) {
    double mx = 0.0;
#pragma unroll
    for (int k = 0; k < kRedSlices; ++k) mx = fmax(mx, red[k][col]);
    vscale[i] = __fdiv_rn((float)mx, 448.0f);
  }
}

// V -> FP8 (E4M3) blocks of 64 tokens for the FP8 P.V product:
// [block64][H][D channels][64 bytes]; code = E4M3(fl32(fl32(V - mu) / s_c))
// (hardware conversion: round to nearest even), 0 where s_c = 0 and for
// tokens past the sequence. Within a channel's 64 bytes, 16-byte chunk q holds
// the keys the attention kernel's lane group q owns after its S^T product,
// key(q, j) = 32*(j/8) + 8*q + j%8, stored at chunk q ^ ((c/4) % 4) so that the
// kernel's 16-byte LDS reads of 16 consecutive channels hit distinct banks.
// Thread (8-channel group, q) reads those 16 token rows of its 8 channels and
// writes the 8 chunks directly (no LDS); a workgroup covers D/32 blocks x heads
// worth of threads: 256 threads = 256 / (4 * D/8) (block, head) units.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_v8_blocks(const uint16_t* __restrict__ v, Rows rows, const int32_t* map,
                                                   int32_t H, int64_t sb, int64_t st, int64_t sh,
                                                   const float* __restrict__ vmean, const float* __restrict__ vscale,
                                                   uint8_t* __restrict__ out) {
  constexpr int TPU = 4 * (D / 8);                 // threads per (block, head)
  constexpr int UPW = 256 / TPU;                   // (block, head) units per workgroup
  const int unit = threadIdx.x / TPU, r = threadIdx.x % TPU;
  const int q = r & 3, c8 = (r >> 2) * 8;
  const int h = head_of(rows) * UPW + unit;
  if (h >= H) return;
  const BlockRef br = block_of(rows, map, 64, blockIdx.z);
  if (br.b < 0) return;
  const int blk = br.blk, b = br.b;
  const int N = rows.len(b);
  if (blk * 64 >= N) return;
  const int64_t seq0 = rows.packed ? rows.start(b) * st : (int64_t)b * sb;
  float mu[8], sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mu[i] = vmean != nullptr ? vmean[((int64_t)b * H + h) * D + c8 + i] : 0.0f;
    sc[i] = vscale[((int64_t)b * H + h) * D + c8 + i];
  }
  float x[16][8];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int t = blk * 64 + 32 * (j >> 3) + 8 * q + (j & 7);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (t < N) w = *reinterpret_cast<const uint4*>(v + seq0 + (int64_t)t * st + (int64_t)h * sh + c8);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[j][2 * i] = half_to_f32<BF16>(ws[i] & 0xFFFFu);
      x[j][2 * i + 1] = half_to_f32<BF16>(ws[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float val = vmean != nullptr ? x[j][i] - mu[i] : x[j][i];
      x[j][i] = (t < N && sc[i] > 0.0f) ? __fdiv_rn(val, sc[i]) : 0.0f;
    }
  }
  uint8_t* dst = out + ((rows.block0(b, 64) + blk) * H + h) * (int64_t)D * 64;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c8 + i;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k][i], x[4 * k + 1][i], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k + 2][i], x[4 * k + 3][i], word, true);
      w[k] = (uint32_t)word;
    }
    *reinterpret_cast<uint4*>(dst + c * 64 + 16 * (q ^ ((c >> 2) & 3))) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Per-block quantization of one (b, head, block) of ROWS tokens x D channels:
// one scale over all ROWS*D values (after subtracting mu when given).
// Writes NHD codes (codes_nhd) and/or the blocked K layout (codes_blk).
// (b, t, h, c) of x lives at b*sb + t*st + h*sh + c. With corr != nullptr
// (query blocks, smooth_k with an LSE output) it also stores, per row,
// corr_scale * sum_c x_c * corr_mu[b, h / corr_G, c] (fp32, the D/8 threads
// of a row reduce their partial sums with shuffles).
template <int D, int ROWS, bool BF16, bool CORR = false>
__global__ __launch_bounds__(256) void k_block_quant(const uint16_t* __restrict__ x, Rows rows,
                                                     const int32_t* map, int32_t H, int64_t sb, int64_t st,
                                                     int64_t sh,
                                                     const float* __restrict__ mean,
                                                     int8_t* __restrict__ codes_nhd,
                                                     int8_t* __restrict__ codes_blk,
                                                     float* __restrict__ scale,
                                                     const float* __restrict__ corr_mu, int32_t corr_G,
                                                     float corr_scale, float* __restrict__ corr) {
  constexpr int G8 = D / 8;                // 8-channel groups per row
  constexpr int PER = ROWS * G8 / 256;     // groups per thread
  static_assert(ROWS * G8 % 256 == 0, "block must tile the workgroup");
  const BlockRef br = block_of(rows, map, ROWS, blockIdx.z);
  if (br.b < 0) return;
  const int blk = br.blk, h = head_of(rows), b = br.b;
  const int N = rows.len(b);                 // tokens of this sequence
  if (blk * ROWS >= N) return;               // batched grids cover the longest sequence
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq0 = rows.packed ? rows.start(b) * st : (int64_t)b * sb;
  __shared__ float red[4];

  // All PER row loads of the thread are issued before any is used (a row
  // past the sequence end re-reads the last row, and counts as zeros), and
  // the raw 16-bit values stay in registers: the fp32 values are formed again
  // for the codes below, exactly as here.
  uint4 wv[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int gi = threadIdx.x + 256 * k;
    const int r = gi / G8, c = (gi % G8) * 8;
    const int t = min(blk * ROWS + r, N - 1);
    wv[k] = *reinterpret_cast<const uint4*>(x + seq0 + (int64_t)t * st + (int64_t)h * sh + c);
  }
  // the thread's 8 channels are the same in every row (256 is a multiple of G8)
  const int c_thr = (threadIdx.x % G8) * 8;
  float mu8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mu8[i] = mean != nullptr ? mean[((int64_t)b * H + h) * D + c_thr + i] : 0.0f;
  // fp32 values of unit k (minus the mean when given), zeros past the end
  auto values = [&](int k, float (&v)[8]) {
    const int t = blk * ROWS + (threadIdx.x + 256 * k) / G8;
    const uint32_t ws[4] = {wv[k].x, wv[k].y, wv[k].z, wv[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = half_to_f32<BF16>(ws[i] & 0xFFFFu);
      v[2 * i + 1] = half_to_f32<BF16>(ws[i] >> 16);
    }
    if (mean != nullptr) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] - mu8[i];
    }
    if (t >= N) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
  };
  float amax = 0.0f;
  float cm[CORR ? 8 : 1];                    // LSE correction: the mean of this thread's channels
  float dsum[CORR ? PER : 1];
  if constexpr (CORR) {
#pragma unroll
    for (int i = 0; i < 8; ++i) cm[i] = corr_mu[((int64_t)b * (H / corr_G) + h / corr_G) * D + c_thr + i];
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    float v[8];
    values(k, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    if constexpr (CORR) {
      dsum[k] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dsum[k] = fmaf(v[i], cm[i], dsum[k]);
    }
  }
  if constexpr (CORR) {
    // the G8 threads of a row are consecutive lanes of one wave (G8 divides 64)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int gi = threadIdx.x + 256 * k;
      const int t = blk * ROWS + gi / G8;
#pragma unroll
      for (int o = 1; o < G8; o <<= 1) dsum[k] += __shfl_xor(dsum[k], o, 64);
      if (gi % G8 == 0 && t < N) corr[rows.row_at(b, h, H, t)] = dsum[k] * corr_scale;
    }
  }
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // the fp32 values are formed again below rather than kept (the compiler
  // would otherwise keep all PER x 8 of them live across the reduction)
#pragma unroll
  for (int k = 0; k < PER; ++k) asm volatile("" : "+v"(wv[k].x), "+v"(wv[k].y), "+v"(wv[k].z), "+v"(wv[k].w));
  const float s = quant_scale(amax);
  const float rs = __fdiv_rn(1.0f, s);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int gi = threadIdx.x + 256 * k;
    const int r = gi / G8, c = (gi % G8) * 8;
    const int t = blk * ROWS + r;
    float v[8];
    values(k, v);
    uint32_t w[2];
    quant_bytes<8>(v, amax, s, rs, w);
    uint32_t lo = w[0], hi = w[1];
    if (t >= N) lo = hi = 0;
    if (codes_nhd != nullptr && t < N)
      *reinterpret_cast<uint2*>(codes_nhd + ((rows.start(b) + t) * H + h) * D + c) = make_uint2(lo, hi);
    if (codes_blk != nullptr) {
      // blocked layout: block (block0 + t/16), head h, chunk c/16, slot t%16
      const int64_t pb = rows.block0(b, 16) + t / 16;
      if (t / 16 < (N + 15) / 16)
        *reinterpret_cast<uint2*>(codes_blk + ((pb * H + h) * (D / 16) + c / 16) * 256 + (t % 16) * 16 + (c % 16)) =
            make_uint2(lo, hi);
    }
  }
  if (threadIdx.x == 0) scale[rows.scale_at(b, h, H, blk, ROWS)] = s;
}

// K blocks of 64 tokens straight into the blocked layout
// [block16][head][D/16][16 tokens][16 channels]: the codes, scale and mean
// handling of k_block_quant<D, 64> (codes_blk only), with each thread unit 16
// channels of one token (two 16-byte loads, one 16-byte store) placed so that
// the 64 lanes of a wave write 16 token slots of four neighbouring 16-channel
// chunks, 1 KB of contiguous codes (eight-byte units 256 bytes apart wrote
// 16-byte pieces).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_kblock_quant(const uint16_t* __restrict__ x, Rows rows,
                                                      const int32_t* map, int32_t H, int64_t sb, int64_t st,
                                                      int64_t sh, const float* __restrict__ mean,
                                                      int8_t* __restrict__ codes_blk, float* __restrict__ scale) {
  constexpr int ROWS = 64, CH = D / 16;          // 16-channel chunks per row
  constexpr int PER = ROWS * CH / 256;           // units per thread
  static_assert(ROWS * CH % 256 == 0 && 256 % (16 * CH) == 0, "units must tile the workgroup");
  const BlockRef br = block_of(rows, map, ROWS, blockIdx.z);
  if (br.b < 0) return;
  const int blk = br.blk, h = head_of(rows), b = br.b;
  const int N = rows.len(b);
  if (blk * ROWS >= N) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq0 = rows.packed ? rows.start(b) * st : (int64_t)b * sb;
  __shared__ float red[4];
  // unit u = threadIdx.x + 256 k: token slot u % 16 of 16-row group u / (16 CH),
  // chunk (u / 16) % CH (the same chunk for every k of a thread)
  const int slot = threadIdx.x % 16, cc = (threadIdx.x / 16) % CH;
  uint4 wv[PER][2];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int r = ((threadIdx.x + 256 * k) / (16 * CH)) * 16 + slot;
    const int t = min(blk * ROWS + r, N - 1);
    const uint16_t* src = x + seq0 + (int64_t)t * st + (int64_t)h * sh + cc * 16;
    wv[k][0] = *reinterpret_cast<const uint4*>(src);
    wv[k][1] = *reinterpret_cast<const uint4*>(src + 8);
  }
  float mu[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) mu[i] = mean != nullptr ? mean[((int64_t)b * H + h) * D + cc * 16 + i] : 0.0f;
  auto values = [&](int k, float (&v)[16]) {
    const int t = blk * ROWS + ((threadIdx.x + 256 * k) / (16 * CH)) * 16 + slot;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t ws[4] = {wv[k][q].x, wv[k][q].y, wv[k][q].z, wv[k][q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = half_to_f32<BF16>(ws[i] & 0xFFFFu) - mu[8 * q + 2 * i];
        v[8 * q + 2 * i + 1] = half_to_f32<BF16>(ws[i] >> 16) - mu[8 * q + 2 * i + 1];
      }
    }
    if (t >= N) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
  };
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    float v[16];
    values(k, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // the fp32 values are formed again below rather than kept
#pragma unroll
  for (int k = 0; k < PER; ++k)
#pragma unroll
    for (int q = 0; q < 2; ++q) asm volatile("" : "+v"(wv[k][q].x), "+v"(wv[k][q].y), "+v"(wv[k][q].z), "+v"(wv[k][q].w));
  const float s = quant_scale(amax);
  const float rs = __fdiv_rn(1.0f, s);
  const int nb16 = (N + 15) / 16;                // 16-token blocks of the sequence
  const int64_t pb0 = rows.block0(b, 16) + blk * (ROWS / 16);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int g16 = (threadIdx.x + 256 * k) / (16 * CH);
    float v[16];
    values(k, v);
    uint32_t w[4];
    quant_bytes<16>(v, amax, s, rs, w);
    if (blk * (ROWS / 16) + g16 < nb16)
      *reinterpret_cast<uint4*>(codes_blk + (((pb0 + g16) * H + h) * CH + cc) * 256 + slot * 16) =
          make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (threadIdx.x == 0) scale[rows.scale_at(b, h, H, blk, ROWS)] = s;
}

// V [B, N, H, D] (bf16 or fp16) -> fp16 [B*ceil(N/16), H, D, 16]: row ch of a block
// holds its 16 tokens of channel ch in order (the attention kernel's LDS layout,
// so its tiles are copied unchanged); padding tokens of the last block are zero. bf16 values become the
// nearest fp16 (exact in the fp16 normal range).
// (b, t, h, c) of v lives at b*sb + t*st + h*sh + c. With vmean (smooth_v)
// each value becomes fl16(fl32(v) - vmean[b, h, c]).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_v_blocks(const uint16_t* __restrict__ v, Rows rows,
                                                  const int32_t* map, int32_t H, int64_t sb, int64_t st,
                                                  int64_t sh,
                                                  const float* __restrict__ vmean, uint16_t* __restrict__ vb) {
  constexpr int UPR = D / 8;                 // 16-byte units per token row
  __shared__ __attribute__((aligned(16))) uint16_t tile[16][D + 8];
  const BlockRef br = block_of(rows, map, 16, blockIdx.z);
  if (br.b < 0) return;
  const int blk = br.blk, h = head_of(rows), b = br.b;
  const int N = rows.len(b);
  if (blk * 16 >= N) return;                 // batched grids cover the longest sequence
  const int64_t seq0 = rows.packed ? rows.start(b) * st : (int64_t)b * sb;
  for (int u = threadIdx.x; u < 16 * UPR; u += 256) {
    const int r = u / UPR, c8 = (u % UPR) * 8;
    const int t = blk * 16 + r;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (t < N) {
      w = *reinterpret_cast<const uint4*>(v + seq0 + (int64_t)t * st + (int64_t)h * sh + c8);
      if (vmean != nullptr) {
        const float* mu = vmean + ((int64_t)b * H + h) * D + c8;
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = half_to_f32<BF16>(ws[i] & 0xFFFFu) - mu[2 * i];
          const float hi = half_to_f32<BF16>(ws[i] >> 16) - mu[2 * i + 1];
          o[i] = f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
        }
        w = make_uint4(o[0], o[1], o[2], o[3]);
      } else if constexpr (BF16) {
        w = __builtin_bit_cast(uint4, bf16x8_to_f16x8(w));
      }
    }
    *reinterpret_cast<uint4*>(&tile[r][c8]) = w;
  }
  __syncthreads();
  uint16_t* dst = vb + ((rows.block0(b, 16) + blk) * H + h) * D * 16;
  for (int u = threadIdx.x; u < 2 * D; u += 256) {   // output unit: channel u/2, half u%2
    const int ch = u >> 1;
    const int t0 = 8 * (u & 1);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)tile[t0 + 2 * i][ch] | ((uint32_t)tile[t0 + 2 * i + 1][ch] << 16);
    *reinterpret_cast<uint4*>(dst + u * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// workgroups of the row quantizer: four per CU (16 waves)
constexpr int64_t kQuantGrid = 1024;

template <int D>
hipError_t quantize_rows_d(const void* x, bool bf16, int64_t T, int32_t H, int64_t st, int64_t sh,
                           int8_t* q, float* scale, hipStream_t s) {
  const int64_t rows = T * H;
  // four waves of 4-row groups per workgroup; at most kQuantGrid workgroups,
  // each wave then walks several groups
  const int64_t wgs = ((rows + 3) / 4 + 3) / 4;
  const dim3 grid((unsigned)(wgs < kQuantGrid ? wgs : kQuantGrid));
  if (bf16)
    k_quantize_rows<D, true><<<grid, 256, 0, s>>>((const uint16_t*)x, rows, H, st, sh, q, scale);
  else
    k_quantize_rows<D, false><<<grid, 256, 0, s>>>((const uint16_t*)x, rows, H, st, sh, q, scale);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t write_kv_d(const void* k, const void* v, int64_t T, int32_t H, int64_t st, int64_t sh,
                      const int64_t* slots, int8_t* kc, float* ks, void* vc, bool v_i8, float* vs,
                      hipStream_t s) {
  const int64_t rows = T * H;
  if (T >= 16) {
    // groups of 16 tokens (whole blocks written at once when aligned)
    const dim3 g((unsigned)((T + 15) / 16), (unsigned)H);
    if (v_i8)
      k_write_kv_blocks<D, BF16, true><<<g, 256, 0, s>>>((const uint16_t*)k, (const uint16_t*)v, T, H, st, sh,
                                                         slots, kc, ks, vc, vs);
    else
      k_write_kv_blocks<D, BF16, false><<<g, 256, 0, s>>>((const uint16_t*)k, (const uint16_t*)v, T, H, st, sh,
                                                          slots, kc, ks, vc, vs);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (v_i8)
    k_write_kv<D, BF16, true><<<grid, 256, 0, s>>>((const uint16_t*)k, (const uint16_t*)v, rows, H, st,
                                                   sh, slots, kc, ks, vc, vs);
  else
    k_write_kv<D, BF16, false><<<grid, 256, 0, s>>>((const uint16_t*)k, (const uint16_t*)v, rows, H, st,
                                                    sh, slots, kc, ks, vc, vs);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t sage_prep_d(const SagePrepArgs& a, hipStream_t s) {
  const int HD = a.Hkv * D;
  const int chunks = (a.Nk + kSumChunk - 1) / kSumChunk;
  const int cgs = (HD + kSumCols - 1) / kSumCols;   // column groups of the sums
  const bool vl = a.k_rows.packed;
  // varlen grids run over the packed blocks of all sequences (block maps first)
  auto grid = [&](const Rows& r, int R, int heads) {
    return vl ? dim3((unsigned)r.nblocks(R), heads, 1) : dim3(heads, (unsigned)((r.N + R - 1) / R), a.B);
  };
  if (vl) {
    k_block_map<<<a.B, 256, 0, s>>>(a.q_rows, 128, a.q_map);
    k_block_map<<<a.B, 256, 0, s>>>(a.k_rows, 64, a.k_map64);
    k_block_map<<<a.B, 256, 0, s>>>(a.k_rows, 16, a.k_map16);
  }
  const dim3 gsum = vl ? dim3((unsigned)a.k_rows.nblocks(kSumChunk), cgs, 1) : dim3(cgs, chunks, a.B);
  const unsigned gmean = (unsigned)(((int64_t)a.B * HD + kRedCols - 1) / kRedCols);
  if (a.smooth_k && a.Nk > 0)
    k_colsum<BF16><<<gsum, 256, 0, s>>>((const uint16_t*)a.k, a.k_rows, a.k_map64, D, HD, a.k_sb, a.k_st, a.k_sh,
                                        a.partial);
  k_mean<<<gmean, 256, 0, s>>>(a.partial, a.k_rows, HD, a.smooth_k, a.k_mean);
  if (a.Nq > 0 && !a.skip_q) {
    float* corr = a.smooth_k ? a.lse_corr : nullptr;
    auto qk = corr != nullptr ? k_block_quant<D, 128, BF16, true> : k_block_quant<D, 128, BF16, false>;
    qk<<<grid(a.q_rows, 128, a.Hq), 256, 0, s>>>(
        (const uint16_t*)a.q, a.q_rows, a.q_map, a.Hq, a.q_sb, a.q_st, a.q_sh, nullptr, a.q_i8, nullptr, a.q_scale,
        a.k_mean, a.Hq / a.Hkv, a.corr_scale, corr);
  }
  if (a.Nk > 0) {
    if (a.k_i8 == nullptr && a.k_paged != nullptr)
      k_kblock_quant<D, BF16><<<grid(a.k_rows, 64, a.Hkv), 256, 0, s>>>(
          (const uint16_t*)a.k, a.k_rows, a.k_map64, a.Hkv, a.k_sb, a.k_st, a.k_sh, a.k_mean, a.k_paged,
          a.k_scale);
    else
      k_block_quant<D, 64, BF16><<<grid(a.k_rows, 64, a.Hkv), 256, 0, s>>>(
          (const uint16_t*)a.k, a.k_rows, a.k_map64, a.Hkv, a.k_sb, a.k_st, a.k_sh, a.k_mean, a.k_i8, a.k_paged,
          a.k_scale, nullptr, 1, 0.0f, nullptr);
    if ((a.v_paged != nullptr || a.v8 != nullptr) && !a.skip_v) {
      if (a.smooth_v) {
        // the column sums of K are consumed: the buffer takes those of V
        k_colsum<BF16><<<gsum, 256, 0, s>>>((const uint16_t*)a.v, a.k_rows, a.k_map64, D, HD, a.v_sb, a.v_st,
                                            a.v_sh, a.partial);
        k_mean<<<gmean, 256, 0, s>>>(a.partial, a.k_rows, HD, true, a.v_mean);
      }
      const float* vmu = a.smooth_v ? a.v_mean : nullptr;
      if (a.v8 != nullptr) {
        // per-channel maxima of V (- mu), the FP8 scales, then the E4M3 blocks
        k_colsum<BF16, true><<<gsum, 256, 0, s>>>((const uint16_t*)a.v, a.k_rows, a.k_map64, D, HD, a.v_sb,
                                                  a.v_st, a.v_sh, a.partial, vmu);
        k_vscale<<<gmean, 256, 0, s>>>(a.partial, a.k_rows, HD, a.v8_scale);
        constexpr int UPW = 256 / (4 * (D / 8));     // heads per workgroup
        dim3 g8 = grid(a.k_rows, 64, (a.Hkv + UPW - 1) / UPW);
        k_v8_blocks<D, BF16><<<g8, 256, 0, s>>>((const uint16_t*)a.v, a.k_rows, a.k_map64, a.Hkv, a.v_sb, a.v_st,
                                               a.v_sh, vmu, a.v8_scale, a.v8);
      } else {
        k_v_blocks<D, BF16><<<grid(a.k_rows, 16, a.Hkv), 256, 0, s>>>(
            (const uint16_t*)a.v, a.k_rows, a.k_map16, a.Hkv, a.v_sb, a.v_st, a.v_sh, vmu, a.v_paged);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, bool bf16, int64_t T, int32_t H, int32_t D, int64_t st,
                                int64_t sh, int8_t* q, float* scale, hipStream_t s) {
  switch (D) {
    case 64: return quantize_rows_d<64>(x, bf16, T, H, st, sh, q, scale, s);
    case 128: return quantize_rows_d<128>(x, bf16, T, H, st, sh, q, scale, s);
    default: return quantize_rows_d<256>(x, bf16, T, H, st, sh, q, scale, s);
  }
}

hipError_t launch_write_kv_cache(const void* k, const void* v, bool bf16, int64_t T, int32_t H,
                                 int32_t D, int64_t st, int64_t sh, const int64_t* slots,
                                 int8_t* kc, float* ks, void* vc, bool v_i8, float* vs,
                                 hipStream_t s) {
#define QA_WKV(DD)                                                                   \
  return bf16 ? write_kv_d<DD, true>(k, v, T, H, st, sh, slots, kc, ks, vc, v_i8, vs, s) \
              : write_kv_d<DD, false>(k, v, T, H, st, sh, slots, kc, ks, vc, v_i8, vs, s)
  switch (D) {
    case 64: QA_WKV(64);
    case 128: QA_WKV(128);
    default: QA_WKV(256);
  }
#undef QA_WKV
}

template <int D, bool BF16>
hipError_t producer_d(const ProducerArgs& a, hipStream_t s) {
  const int64_t qb = (a.q_rows + 3) / 4, kb = (a.kv_rows + 3) / 4;
  if (qb + kb == 0) return hipSuccess;
  if (a.v_int8)
    k_producer<D, BF16, true><<<(unsigned)(qb + kb), 256, 0, s>>>(a, qb);
  else
    k_producer<D, BF16, false><<<(unsigned)(qb + kb), 256, 0, s>>>(a, qb);
  return hipGetLastError();
}

hipError_t launch_producer(const ProducerArgs& a, hipStream_t s) {
#define QA_PROD(DD) return a.bf16 ? producer_d<DD, true>(a, s) : producer_d<DD, false>(a, s)
  switch (a.D) {
    case 64: QA_PROD(64);
    case 128: QA_PROD(128);
    default: QA_PROD(256);
  }
#undef QA_PROD
}

size_t sage_partial_bytes(int32_t B, int32_t Nk, int32_t Hkv, int32_t D) {
  const size_t chunks = (size_t)((Nk + kSumChunk - 1) / kSumChunk);
  return (size_t)B * (chunks > 0 ? chunks : 1) * (size_t)Hkv * D * sizeof(double);
}

hipError_t launch_sage_prep(const SagePrepArgs& a, hipStream_t s) {
#define QA_PREP(DD) return a.bf16 ? sage_prep_d<DD, true>(a, s) : sage_prep_d<DD, false>(a, s)
  switch (a.D) {
    case 64: QA_PREP(64);
    case 128: QA_PREP(128);
    default: QA_PREP(256);
  }
#undef QA_PREP
}

}  // namespace qa
