// Host-side interface between the C ABI (api.hip) and the kernel files.
// Every launcher assumes its arguments were validated by the caller and
// returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qa {

// quantize.hip ---------------------------------------------------------------
hipError_t launch_quantize_rows(const void* x, bool bf16, int64_t num_tokens, int32_t num_heads,
                                int32_t head_dim, int64_t stride_t, int64_t stride_h,
                                int8_t* q, float* scale, hipStream_t st);

hipError_t launch_write_kv_cache(const void* k, const void* v, bool bf16, int64_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int64_t stride_t,
                                 int64_t stride_h, const int64_t* slots, int8_t* k_cache,
                                 float* k_scale, void* v_cache, bool v_int8, float* v_scale,
                                 hipStream_t st);

// Rotary embedding applied ahead of quantization (pos == nullptr: none).
// Table row p holds cos(p w_i) at i and sin(p w_i) at rot/2 + i; neox pairs
// channel i with i + rot/2, otherwise 2i with 2i + 1 (pair i uses w_i);
// channels from rot on pass through.
struct Rope {
  const int64_t* pos;   // [tokens] position of each token
  const float* cs;      // [max_position, rot] fp32
  int32_t rot;
  bool neox;
};

struct ProducerArgs {
  const void* q;           // [q_tokens, Hq, D] rows at q + t*q_st + h*q_sh
  const void* k;           // [kv_tokens, Hkv, D] rows at k/v + t*kv_st + h*kv_sh
  const void* v;
  const int64_t* slots;
  bool bf16, v_int8;
  int32_t D, Hq, Hkv;
  int64_t q_rows, kv_rows;  // tokens * heads
  int64_t q_st, q_sh, kv_st, kv_sh;
  int8_t* q_i8;
  float* q_scale;
  int8_t* k_cache;
  float* k_scale;
  void* v_cache;
  float* v_scale;
  Rope rope;               // rotates query rows and K rows (token t at rope.pos[t])
};
hipError_t launch_producer(const ProducerArgs& a, hipStream_t st);

// Where the tokens of sequence b of a dense call live. Batched (cu == nullptr):
// every sequence has N tokens, token t of sequence b is row b*N + t, and its
// R-token blocks start at b*ceil(N/R). Varlen (packed rows): sequence b is rows
// cu[b] .. cu[b+1]-1 and N is the largest length; its blocks start at
// cu[b]/R + b, so each sequence begins a fresh block and all of them fit in
// total/R + B blocks (the gap left before each sequence is under one block).
struct Rows {
  const int32_t* cu;   // [B+1] device row offsets (varlen) or nullptr
  int32_t B, N;
  int64_t total;       // varlen: number of rows (cu[B])
  bool packed;         // varlen (cu is set in every launch; the host sizes buffers without it)
  __device__ __forceinline__ int64_t start(int b) const { return packed ? (int64_t)cu[b] : (int64_t)b * N; }
  __device__ __forceinline__ int len(int b) const { return packed ? cu[b + 1] - cu[b] : N; }
  __host__ __device__ __forceinline__ int64_t nblocks(int R) const {
    return packed ? total / R + B : (int64_t)B * ((N + R - 1) / R);
  }
  __device__ __forceinline__ int64_t block0(int b, int R) const {
    return packed ? (int64_t)(cu[b] / R) + b : (int64_t)b * ((N + R - 1) / R);
  }
  // per-(sequence, head) block scales: batched [B, H, ceil(N/R)], varlen [H, total/R + B]
  __device__ __forceinline__ int64_t scale_at(int b, int h, int H, int blk, int R) const {
    return packed ? (int64_t)h * nblocks(R) + block0(b, R) + blk : ((int64_t)b * H + h) * ((N + R - 1) / R) + blk;
  }
  // per-(sequence, head, token) values (LSE): batched [B, H, N], varlen [H, total]
  __device__ __forceinline__ int64_t row_at(int b, int h, int H, int t) const {
    return packed ? (int64_t)h * total + cu[b] + t : ((int64_t)b * H + h) * N + t;
  }
};

struct SagePrepArgs {
  const void* q;
  const void* k;
  const void* v;          // only for the V transpose
  // element strides of (batch, token, head) in q, k and v (channels contiguous):
  // NHD = (N*H*D, H*D, D), HND = (H*N*D, D, N*D); varlen rows (q_rows.cu set)
  // are packed [total, H, D]: token t of sequence b is row start(b) + t and the
  // batch strides are unused
  int64_t q_sb, q_st, q_sh, k_sb, k_st, k_sh, v_sb, v_st, v_sh;
  Rows q_rows, k_rows;    // sequence geometry of q and of k/v (N = Nq / Nk)
  // varlen: sequence of each packed block (-1 for the gap before a sequence),
  // written here: q_map [q_rows.nblocks(128)], k_map64 and k_map16 likewise
  int32_t* q_map;
  int32_t* k_map64;
  int32_t* k_map16;
  bool bf16;
  int32_t B, Nq, Nk, Hq, Hkv, D;
  bool smooth_k;
  bool smooth_v;          // subtract the per-channel V mean (v_mean) in the V blocks
  float* v_mean;          // [B, Hkv, D] (smooth_v)
  float* lse_corr;        // q_rows.row_at layout: smooth_k correction of the LSE, or nullptr
  bool skip_q;            // the attention kernel quantizes the query blocks itself
  bool skip_v;            // the attention kernel reads V in token order itself
  float corr_scale;       // softmax scale (natural-log units) for lse_corr
  int8_t* q_i8;           // NHD codes
  float* q_scale;         // q_rows.scale_at(.., 128) layout
  int8_t* k_i8;           // NHD codes (public layout) or nullptr
  int8_t* k_paged;        // blocked layout [k_rows.nblocks(16), Hkv, D/16, 16, 16] or nullptr
  float* k_scale;         // k_rows.scale_at(.., 64) layout
  float* k_mean;          // [B, Hkv, D]
  double* partial;        // fp64 column sums [B, chunks, Hkv*D]
  uint16_t* v_paged;      // V transposed into [k_rows.nblocks(16), Hkv, D, 16] or nullptr
  // FP8 P.V instead: V in E4M3 blocks [k_rows.nblocks(64), Hkv, D, 64] (v8)
  // with per-(b, KV head, channel) scales v8_scale [B, Hkv, D]
  uint8_t* v8;
  float* v8_scale;
};
size_t sage_partial_bytes(int32_t B, int32_t Nk, int32_t Hkv, int32_t D);
hipError_t launch_sage_prep(const SagePrepArgs& a, hipStream_t st);

// decode.hip -----------------------------------------------------------------
struct DecodeArgs {
  const int8_t* q;
  const float* q_scale;
  const int8_t* k_cache;
  const float* k_scale;
  const void* v_cache;
  const float* v_scale;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* ws_o;            // [S, ...] partial outputs (S > 1)
  float* ws_ml;           // partial (max, sum)
  void* out;
  int32_t* acc_out;       // debug export
  int32_t num_seqs, Hq, Hkv, G, D, max_blocks, num_splits;
  int32_t tq;             // query tokens per sequence (G*tq <= 16 columns); 1 for plain decode
  bool seq_split;         // split each sequence's own blocks into S segments (else max_blocks / S)
  bool lpt;               // workgroup slot z runs the sequence ranked z by context length (2..64 sequences)
  float scale_log2;       // softmax_scale * log2(e)
  bool v_int8, out_bf16;
  // fused step (q_in != nullptr): the split kernel quantizes the query rows
  // and writes the new token's K/V (position ctx-1 of each sequence) itself
  const uint16_t* q_in;   // [num_seqs] rows of [Hq, D] at q_in + s*q_st + h*q_sh
  const uint16_t* k_new;  // [num_seqs] rows of [Hkv, D] at k_new/v_new + s*kv_st + h*kv_sh
  const uint16_t* v_new;
  int64_t q_st, q_sh, kv_st, kv_sh;
  const int64_t* slots;   // cache slot of each sequence's new token (< 0: not written)
  int8_t* kc_w;           // the caches again, writable
  float* ks_w;
  void* vc_w;
  float* vs_w;
  bool in_bf16;           // q_in/k_new/v_new are bf16 (else f16)
  Rope rope;              // fused step: rotate the query rows and the new K row
                          // (position rope.pos[seq]) before quantizing them
};
// kPartials: the split kernel only (with one split it writes the output);
// kCombine: the merge of the split partials only; kBoth: one after the other.
enum class DecodePhase { kBoth, kPartials, kCombine };
hipError_t launch_decode(const DecodeArgs& a, DecodePhase phase, hipStream_t st);
hipError_t launch_debug_qk(const DecodeArgs& a, hipStream_t st);
int32_t choose_decode_splits(int32_t num_seqs, int32_t Hkv, int32_t max_blocks);
// The decode kernels' static scratch for callers that cannot allocate (the
// split partials): kDecodeScratchBytes per GPU. decode_scratch returns the
// current device's copy of it (looked up once per device; no allocation).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

// flash.hip (chunked prefill and dense) --------------------------------------
struct FlashArgs {
  const int8_t* q;         // codes, row (token, head) at (q_row0 + i)*q_row_stride + h*D
  const float* q_scale;    // per-token [T, Hq] (paged) or per-block [B, Hq, nqb] (dense)
  const int8_t* k_blocks;  // [blocks, Hkv, D/16, 16, 16]
  const float* k_scale;    // per-token [blocks, Hkv, 16] (paged) or per-64 [B, Hkv, nkb] (dense)
  const void* v_blocks;    // [blocks, Hkv, D, 16] bf16 / f16 / int8
  const float* v_scale;    // per-token (int8 V)
  const int32_t* tables;   // [num_seqs, max_blocks] (paged) or nullptr (dense: identity)
  const int32_t* cu_q;     // [num_seqs+1] (paged) or nullptr (dense: b*Nq)
  const int32_t* ctx_lens; // [num_seqs] (paged) or nullptr (dense: Nk)
  void* out;               // [rows, Hq, D] (dense: element (b, i, h, c) at b*o_sb + i*o_st + h*o_sh + c)
  int64_t o_sb, o_st, o_sh; // dense output strides
  const float* v_mean;     // dense smooth_v: [B, Hkv, D] added back on rows that see a key, or nullptr
  float* lse;              // dense: natural-log LSE of each row (q_rows.row_at layout), or nullptr
  const float* lse_corr;   // dense: added to lse (smooth_k correction, same layout), or nullptr
  Rows q_rows, k_rows;     // dense: sequence geometry (varlen when q_rows.packed)
  const int32_t* q_map;    // varlen: sequence of each packed 128-row query block, -1 for gaps
  const float* v8_scale;   // dense FP8 P.V: per-(b, KV head, channel) V scales (v_blocks holds E4M3 blocks)
  int32_t num_seqs, Hq, Hkv, G, D, max_blocks, max_seqlen_q;
  int32_t Nq, Nk;          // dense only
  float scale_log2;
  bool dense, causal, v_int8, v_f16, out_bf16, out_f16;
  bool pv_fp8;             // dense: FP8 P.V (head_dim 64 or 128)
  void* v_ws;              // paged: workspace for the fp16 V blocks [seq][max_blocks][Hkv][D][16], or nullptr
  // dense: the 16-bit queries themselves, quantized per 128-row block by the
  // attention kernel (q and q_scale unused), element (b, t, h, c) at
  // b*q_sb + t*q_st + h*q_sh + c (varlen: (start(b) + t)*q_st + h*q_sh + c); or nullptr
  const uint16_t* q_in;
  int64_t q_sb, q_st, q_sh;
  bool q_in_bf16;
  // dense: the fp16 V input read by the attention kernel in token order (no
  // V block pass; no smooth_v), element (b, t, h, c) at b*v_sb + t*v_st +
  // h*v_sh + c (varlen: (start(b) + t)*v_st + h*v_sh + c); or nullptr
  const uint16_t* v_tok;
  int64_t v_sb, v_st, v_sh;
};
hipError_t launch_flash(const FlashArgs& a, hipStream_t st);

// Chunked prefill with the FP8 (E4M3) P.V product: two passes over V into the
// workspace (partial maxima, then channel scales and E4M3 tiles of 128 keys in
// the kernel's LDS layout), then the attention.
constexpr int kV8Parts = 32;   // token slices of the partial-maximum pass
struct PrefillFp8Args {
  const int8_t* q;         // [total_q, Hq, D] codes
  const float* q_scale;    // [total_q, Hq]
  const int8_t* k_blocks;  // [blocks, Hkv, D/16, 16, 16]
  const float* k_scale;    // [blocks, Hkv, 16]
  const void* v_cache;     // [blocks, Hkv, D, 16] bf16 or int8
  const float* v_scale;    // [blocks, Hkv, 16] (int8 V)
  const int32_t* tables;   // [num_seqs, max_blocks]
  const int32_t* cu_q;     // [num_seqs + 1]
  const int32_t* ctx_lens; // [num_seqs]
  void* out;               // [total_q, Hq, D] fp32 or bf16
  uint8_t* v8;             // workspace: [num_seqs, v8_seq_tiles, Hkv, 4, D, 32] E4M3
  float* v8_scale;         // workspace: [num_seqs, Hkv, D]
  float* partial;          // workspace: [num_seqs, Hkv, kV8Parts, D]
  int32_t num_seqs, Hq, Hkv, G, D, max_blocks, max_seqlen_q, v8_seq_tiles;
  float scale_log2;
  bool v_int8, out_bf16;
};
hipError_t launch_prefill_fp8(const PrefillFp8Args& a, hipStream_t st);

}  // namespace qa
