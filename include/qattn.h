/*
 * qattn.h - C ABI of the INT8-QK quantized attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources the operations follow:
 *   [QK-MMAC]   "INT8 QK MMAC on the gfx936 DCU: paged access, fragment
 *               mapping and GQA" (forum article).
 *   [SAGE-MACA] "SageAttention - MetaX MXMACA port (v3.0.0)" README.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or synchronizes; buffers must stay valid until
 *     the work queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is queued asynchronously on it, in call order.
 *   - Host-side argument checks run before any HIP call. A non-zero status
 *     means nothing was queued; qa_last_error() describes the problem.
 *   - Device-data preconditions are documented but not checked: block-table
 *     entries lie in [0, num_blocks), context_lens[s] <= max_blocks_per_seq *
 *     block_size, cache slots written by one call are distinct, and inputs
 *     are finite. Violating them gives unspecified results.
 *   - Supported shapes: head_dim in {64, 128, 256}; block_size 16; in paged
 *     paths num_q_heads % num_kv_heads == 0 with a group of at most 16 query
 *     heads per KV head. Other valid shapes return QA_ERR_UNSUPPORTED rather
 *     than run with a wrong mapping ([QK-MMAC] §7 applicability guards).
 */
#ifndef QATTN_H
#define QATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QA_ABI_VERSION 1

typedef enum {
  QA_OK = 0,
  QA_ERR_INVALID_ARG = 1,        /* null pointer, bad shape, stride or dtype */
  QA_ERR_UNSUPPORTED = 2,        /* valid request outside the supported set  */
  QA_ERR_WORKSPACE_TOO_SMALL = 3,
  QA_ERR_HIP = 4                 /* a HIP launch reported an error           */
} qa_status_t;

typedef enum {
  QA_DT_BF16 = 0,
  QA_DT_F16 = 1,
  QA_DT_F32 = 2,
  QA_DT_I8 = 3
} qa_dtype_t;

typedef void* qa_stream_t;       /* hipStream_t */

/* ABI version of the loaded library (QA_ABI_VERSION at build time). */
int qa_abi_version(void);

/* Message for the last non-zero status returned on the calling thread.
 * The string is owned by the library and valid until the next call. */
const char* qa_last_error(void);

/*
 * Per-row symmetric dynamic INT8 quantization of the query.
 * [QK-MMAC] §1 (one scale per query token and query head), §4 (scale =
 * max|x| / 127, code = round(x / scale), done once before attention and
 * reused by all split-K segments), §2.1 (codes in [-127, 127]).
 *
 * Arithmetic per row of head_dim values x (bf16/f16 widened exactly):
 *   s = fl32(max|x| / 127);  q = clamp(rne(fl32(x / s)), -127, 127)
 * with IEEE-correctly-rounded fp32 divisions and ties to even. A row whose
 * max|x| is 0 gets s = 0 and zero codes.
 *
 *   q        [num_tokens, num_heads, head_dim] bf16 or f16 (dtype), element
 *            (t, h, i) at q + t*stride_token + h*stride_head + i (strides in
 *            elements, multiples of 8; the innermost stride is 1); 16-byte
 *            aligned
 *   q_i8     out [num_tokens, num_heads, head_dim] int8, contiguous, 8-byte
 *            aligned
 *   q_scale  out [num_tokens, num_heads] fp32, contiguous
 * num_tokens == 0 is a no-op; a misaligned pointer or stride is
 * QA_ERR_INVALID_ARG.
 */
qa_status_t qa_quantize_q(const void* q, qa_dtype_t dtype, int64_t num_tokens,
                          int32_t num_heads, int32_t head_dim, int64_t stride_token,
                          int64_t stride_head, int8_t* q_i8, float* q_scale,
                          qa_stream_t stream);

/*
 * Quantize K (and optionally V) per (token, KV head) and write the tokens
 * into the paged cache. [QK-MMAC] §1 (key scale per key token and KV head),
 * §3 (K cache layout [block, kv_head, head_dim/16, block_size, 16]).
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim] bf16/f16 (dtype); element
 *                 (t, h, i) at base + t*stride_token + h*stride_head + i
 *   slot_mapping  [num_tokens] int64: slot = block * block_size + offset;
 *                 a negative slot skips the token
 *   k_cache       [num_blocks, num_kv_heads, head_dim/16, block_size, 16] int8
 *   k_scale       [num_blocks, num_kv_heads, block_size] fp32
 *   v_cache       [num_blocks, num_kv_heads, head_dim, block_size]: each
 *                 channel's tokens of a block are contiguous. v_cache_dtype is
 *                 the input dtype (V copied bit for bit) or QA_DT_I8 (V
 *                 quantized like K, codes here and scales in v_scale)
 *   v_scale       [num_blocks, num_kv_heads, block_size] fp32; NULL unless
 *                 v_cache_dtype == QA_DT_I8
 * Only the written slots change. block_size must be 16.
 */
qa_status_t qa_write_kv_cache(const void* k, const void* v, qa_dtype_t dtype,
                              int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int64_t stride_token, int64_t stride_head,
                              const int64_t* slot_mapping, int64_t num_blocks,
                              int32_t block_size, int8_t* k_cache, float* k_scale,
                              void* v_cache, qa_dtype_t v_cache_dtype, float* v_scale,
                              qa_stream_t stream);

/*
 * Fused producer of one step: quantize the new query rows (exactly as
 * qa_quantize_q) and write the new K/V tokens into the paged cache (exactly
 * as qa_write_kv_cache) in a single launch. [QK-MMAC] §4: the query is
 * quantized once, inside the producer that also writes the KV cache, and
 * every split-K segment reuses it (qa_rope_quantize_q_write_kv adds the
 * rotary embedding). Arguments are those of the two calls above; either part may be
 * empty (num_q_tokens == 0 or num_kv_tokens == 0). q, k and v share `dtype`.
 */
qa_status_t qa_quantize_q_write_kv(const void* q, int64_t num_q_tokens, int32_t num_q_heads,
                                   int64_t q_stride_token, int64_t q_stride_head, const void* k,
                                   const void* v, int64_t num_kv_tokens, int32_t num_kv_heads,
                                   int64_t kv_stride_token, int64_t kv_stride_head,
                                   const int64_t* slot_mapping, qa_dtype_t dtype, int32_t head_dim,
                                   int64_t num_blocks, int32_t block_size, int8_t* q_i8, float* q_scale,
                                   int8_t* k_cache, float* k_scale, void* v_cache,
                                   qa_dtype_t v_cache_dtype, float* v_scale, qa_stream_t stream);

/*
 * Rotary position embedding applied by the producer ahead of quantization
 * ([QK-MMAC] §4: the producer that quantizes the query is the RoPE/KV
 * producer). The pages give no rotary parameters; the table is an input.
 *   positions  device int64 [tokens]: position of token t (query row t and
 *              K row t use the same entry); each < the table's row count
 *              (device data: not checked)
 *   cos_sin    device fp32 [max_position, rot_dim]: cos(p w_i) in column i,
 *              sin(p w_i) in column rot_dim/2 + i
 *   rot_dim    rotated channels: even, 2 <= rot_dim <= head_dim; channels
 *              from rot_dim on pass through (partial rotary)
 *   neox       nonzero: pair i is channels (i, i + rot_dim/2); zero: (2i, 2i+1)
 * Pair (a, b) becomes (fl32(fl32(a cos) - fl32(b sin)), fl32(fl32(b cos) +
 * fl32(a sin))) in fp32 from the widened 16-bit inputs (no fused
 * multiply-add), and those fp32 values are quantized (no rounding back to
 * 16 bits). V is not rotated.
 */
typedef struct {
  const int64_t* positions;
  const float* cos_sin;
  int32_t rot_dim;
  int32_t neox;
} qa_rope_t;

/*
 * qa_quantize_q_write_kv with the rotary embedding of `rope` applied to the
 * query rows and K rows before they are quantized: RoPE, query quantization
 * and the KV-cache write in one launch. Same arguments and errors, plus
 * QA_ERR_INVALID_ARG for a NULL rope, table or positions, or a rot_dim that is
 * odd, < 2 or > head_dim.
 */
qa_status_t qa_rope_quantize_q_write_kv(const qa_rope_t* rope, const void* q, int64_t num_q_tokens,
                                        int32_t num_q_heads, int64_t q_stride_token,
                                        int64_t q_stride_head, const void* k, const void* v,
                                        int64_t num_kv_tokens, int32_t num_kv_heads,
                                        int64_t kv_stride_token, int64_t kv_stride_head,
                                        const int64_t* slot_mapping, qa_dtype_t dtype,
                                        int32_t head_dim, int64_t num_blocks, int32_t block_size,
                                        int8_t* q_i8, float* q_scale, int8_t* k_cache,
                                        float* k_scale, void* v_cache, qa_dtype_t v_cache_dtype,
                                        float* v_scale, qa_stream_t stream);

/* Shape and options of a decode call (one query token per sequence). */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;          /* must be 16 */
  int32_t max_blocks_per_seq;  /* row length of block_tables */
  int64_t num_blocks;          /* physical blocks in the pool */
  qa_dtype_t v_cache_dtype;    /* QA_DT_BF16 or QA_DT_I8 */
  qa_dtype_t out_dtype;        /* QA_DT_F32 or QA_DT_BF16 */
  float softmax_scale;         /* <= 0 selects 1/sqrt(head_dim) */
  int32_t num_splits;          /* split-K segments per sequence; 0 = choose */
} qa_decode_params_t;

/* Number of split-K segments a decode call with these parameters uses. */
int32_t qa_paged_decode_num_splits(const qa_decode_params_t* p);

/* Workspace bytes a decode call needs (0 when it runs unsplit): the split
 * partials (max, sum and unnormalized output per split and query head),
 * S*num_seqs*num_q_heads*(head_dim + 2)*4 bytes plus alignment ([QK-MMAC] §4:
 * each segment keeps its running max, sum and output for the merge). Its
 * contents need no initialization. Calls that share a workspace must not
 * run concurrently. 0 for parameters the decode call would reject. */
size_t qa_paged_decode_workspace_bytes(const qa_decode_params_t* p);
/* The same value under its earlier name. */
size_t qa_paged_decode_workspace_size(const qa_decode_params_t* p);

/*
 * Paged decode attention with INT8 Q x INT8 K.
 * [QK-MMAC] §1: score = acc_int32 * sQ(query head) * sK(key token, KV head)
 * * softmax_scale, recovered per element before the online softmax; §2.1-2.2:
 * INT8 matrix instructions with INT32 accumulation; §3: K read through the
 * block table in its INT8 paged layout; §4: long contexts are cut into
 * segments (split-K) that reuse one quantized query; §5.1: the query heads
 * of one KV head share the matrix rows. P.V uses 16-bit matrix instructions
 * with fp32 accumulation: bf16 V directly against P written as the sum of two
 * bf16 numbers (hi = bf16(p), lo = bf16(p - hi)); INT8 V as fp16 codes against
 * fp16 P with the per-token V scale folded into P.
 *
 * Split-K ([QK-MMAC] §4 cuts long contexts into segments): split j of a
 * sequence covers its tokens [16*j*P, min(16*(j+1)*P, ctx)) (possibly none),
 * with P = ceil(ceil(ctx / 16) / S) blocks, the sequence's own blocks cut
 * into S equal segments, when num_seqs > 1, and P = ceil(max_blocks_per_seq
 * / S) for a single sequence (there the table is read without waiting for
 * the context length). Each
 * split stores (max, sum, unnormalized output) in the workspace and a second
 * kernel merges them. S = 1 writes the output directly. Results are
 * bit-identical from run to run. With 2 to 64 sequences the sequences are
 * run longest first (an order of execution only: it changes no result).
 * num_splits = 0 chooses S so that num_seqs * num_kv_heads * S reaches 256
 * workgroups for one sequence and 512 for several (segments of unequal
 * length balance better two to a compute unit), keeping at least 16 blocks
 * per segment and at most 256 segments.
 *
 *   q_i8          [num_seqs, num_q_heads, head_dim] int8 (from qa_quantize_q)
 *   q_scale       [num_seqs, num_q_heads] fp32
 *   k_cache, k_scale, v_cache, v_scale   as written by qa_write_kv_cache
 *                 (v_scale NULL unless v_cache_dtype == QA_DT_I8)
 *   block_tables  [num_seqs, max_blocks_per_seq] int32 physical block ids
 *   context_lens  [num_seqs] int32 visible keys per sequence (0 gives zeros)
 *   workspace     device scratch of >= qa_paged_decode_workspace_bytes bytes
 *   out           [num_seqs, num_q_heads, head_dim] fp32 or bf16
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
qa_status_t qa_paged_attention_decode(const qa_decode_params_t* p, const int8_t* q_i8,
                                      const float* q_scale, const int8_t* k_cache,
                                      const float* k_scale, const void* v_cache,
                                      const float* v_scale, const int32_t* block_tables,
                                      const int32_t* context_lens, void* workspace,
                                      size_t workspace_bytes, void* out, qa_stream_t stream);

/*
 * One decode step in a single call: exactly qa_quantize_q_write_kv for one
 * new token per sequence followed by qa_paged_attention_decode, with the
 * same results bit for bit ([QK-MMAC] §4: the query is quantized once per
 * step and shared by every segment; §1/§3: the new token's K is quantized
 * per token into the paged layout). The split kernel quantizes the query
 * rows itself, and the workgroup whose segment holds the new token
 * quantizes its K (and INT8 V) row, writes it to the cache and uses it
 * directly, so no separate producer launch is needed. The quantized query
 * is not stored.
 *
 *   q             [num_seqs, num_q_heads, head_dim] bf16/f16, row (s, h) at
 *                 q + s*q_stride_token + h*q_stride_head (elements)
 *   k, v          [num_seqs, num_kv_heads, head_dim] the new token's K/V, rows
 *                 at + s*kv_stride_token + h*kv_stride_head (elements)
 *   dtype         QA_DT_BF16 or QA_DT_F16 (BF16 when v_cache_dtype is BF16)
 *   slot_mapping  [num_seqs] int64 cache slot of sequence s's new token; it
 *                 must be the slot of position context_lens[s] - 1 in
 *                 block_tables (not checked); < 0: nothing is written
 *   other arguments as in qa_paged_attention_decode (context_lens include
 *   the new token); the caches are written, so they are non-const.
 */
qa_status_t qa_paged_decode_step(const qa_decode_params_t* p, const void* q, int64_t q_stride_token,
                                 int64_t q_stride_head, const void* k, const void* v,
                                 int64_t kv_stride_token, int64_t kv_stride_head, qa_dtype_t dtype,
                                 const int64_t* slot_mapping, int8_t* k_cache, float* k_scale,
                                 void* v_cache, float* v_scale, const int32_t* block_tables,
                                 const int32_t* context_lens, void* workspace,
                                 size_t workspace_bytes, void* out, qa_stream_t stream);
/* Its first phase alone (the split kernel, new-token write included); finish
 * with qa_paged_attention_decode_combine. Same arguments and errors. */
qa_status_t qa_paged_decode_step_partials(const qa_decode_params_t* p, const void* q,
                                          int64_t q_stride_token, int64_t q_stride_head,
                                          const void* k, const void* v, int64_t kv_stride_token,
                                          int64_t kv_stride_head, qa_dtype_t dtype,
                                          const int64_t* slot_mapping, int8_t* k_cache,
                                          float* k_scale, void* v_cache, float* v_scale,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          void* workspace, size_t workspace_bytes, void* out,
                                          qa_stream_t stream);

/*
 * qa_paged_decode_step with the rotary embedding of `rope` (see qa_rope_t)
 * applied to each sequence's query rows and new K row before they are
 * quantized: rotary embedding, query quantization, the new token's cache
 * write and split-K attention in one kernel ([QK-MMAC] §4), then the combine.
 * rope->positions has one entry per sequence: the position of its new token.
 * Bit-identical to qa_rope_quantize_q_write_kv + qa_paged_attention_decode.
 * Errors as qa_paged_decode_step, plus QA_ERR_INVALID_ARG for a NULL rope,
 * table or positions, or a rot_dim that is odd, < 2 or > head_dim.
 */
qa_status_t qa_paged_decode_step_rope(const qa_rope_t* rope, const qa_decode_params_t* p, const void* q,
                                      int64_t q_stride_token, int64_t q_stride_head, const void* k,
                                      const void* v, int64_t kv_stride_token, int64_t kv_stride_head,
                                      qa_dtype_t dtype, const int64_t* slot_mapping, int8_t* k_cache,
                                      float* k_scale, void* v_cache, float* v_scale,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      void* workspace, size_t workspace_bytes, void* out,
                                      qa_stream_t stream);

/*
 * The two phases of qa_paged_attention_decode as separate calls, for callers
 * that schedule (or time) them apart: _partials launches the split kernel
 * (with S = 1 it writes `out` directly and _combine does nothing); _combine
 * merges the split partials of the workspace into `out` ([QK-MMAC] §4:
 * segment results are merged with their running max and sum). Same
 * arguments, layouts and errors as qa_paged_attention_decode; _partials then
 * _combine on one stream gives its result bit for bit. `out` must be valid
 * in both calls (_partials writes it only when S = 1).
 */
qa_status_t qa_paged_attention_decode_partials(const qa_decode_params_t* p, const int8_t* q_i8,
                                               const float* q_scale, const int8_t* k_cache,
                                               const float* k_scale, const void* v_cache,
                                               const float* v_scale, const int32_t* block_tables,
                                               const int32_t* context_lens, void* workspace,
                                               size_t workspace_bytes, void* out, qa_stream_t stream);
qa_status_t qa_paged_attention_decode_combine(const qa_decode_params_t* p, void* workspace,
                                              size_t workspace_bytes, void* out, qa_stream_t stream);

/* Size of the library's static device scratch used by
 * qa_paged_attention_decode_noalloc (one copy per GPU, held until the process
 * ends). */
#define QA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * qa_paged_attention_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and the same result bit for bit, but the
 * split partials live in a static device array of QA_DECODE_SCRATCH_BYTES
 * owned by the library instead of a caller workspace. Nothing is allocated:
 * the first call on a device looks up that device's copy of the array once
 * (hipGetSymbolAddress; the calling thread's current device must be the
 * stream's device). Its contents need no initialization.
 *   Limit: qa_paged_decode_workspace_bytes(p) <= QA_DECODE_SCRATCH_BYTES, else
 *   QA_ERR_WORKSPACE_TOO_SMALL (checked on the host before any HIP call;
 *   lower num_splits or num_seqs).
 *   Every call on one GPU shares that GPU's array: calls that can overlap on
 *   one device (other streams, other threads) race and give undefined
 *   results; calls queued in order on one stream are safe.
 * Other arguments, layouts and errors as qa_paged_attention_decode.
 */
qa_status_t qa_paged_attention_decode_noalloc(const qa_decode_params_t* p, const int8_t* q_i8,
                                              const float* q_scale, const int8_t* k_cache,
                                              const float* k_scale, const void* v_cache,
                                              const float* v_scale, const int32_t* block_tables,
                                              const int32_t* context_lens, void* out,
                                              qa_stream_t stream);

/*
 * Multi-token decode (speculative or multi-token prediction steps): T new
 * query tokens per sequence attend to the paged cache, which already holds
 * them; token j of sequence s sits at position context_lens[s] - T + j and
 * sees the keys up to that position (causal among the new tokens, as in a
 * chunk of qa_chunked_prefill_attention). [QK-MMAC] §5.1 counts 6 distinct
 * query rows of 16 for one-token decode with 6:1 GQA; §7 asks that the rows
 * be filled by tokens or by several GQA groups: here the G heads of a KV
 * head times the T tokens share the 16 columns of the matrix instruction
 * (G*T <= 16, e.g. 12 of 16 for G = 6, T = 2), so the K/V bytes of a step
 * are read once for all T tokens. T = 1 is qa_paged_attention_decode, bit
 * for bit.
 *
 *   tokens_per_seq  T >= 1 with G*T <= 16 (else QA_ERR_UNSUPPORTED) and
 *                   num_seqs*T <= 65535
 *   q_i8            [num_seqs, T, num_q_heads, head_dim] int8
 *   q_scale         [num_seqs, T, num_q_heads] fp32
 *   out             [num_seqs, T, num_q_heads, head_dim] fp32 or bf16
 *   workspace       >= qa_paged_decode_mt_workspace_size bytes
 *   other arguments and the split-K segments as in qa_paged_attention_decode.
 * A token with no visible key (context_lens[s] - T + j < 0) gives zeros.
 */
size_t qa_paged_decode_mt_workspace_size(const qa_decode_params_t* p, int32_t tokens_per_seq);
qa_status_t qa_paged_attention_decode_mt(const qa_decode_params_t* p, int32_t tokens_per_seq,
                                         const int8_t* q_i8, const float* q_scale,
                                         const int8_t* k_cache, const float* k_scale,
                                         const void* v_cache, const float* v_scale,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         void* workspace, size_t workspace_bytes, void* out,
                                         qa_stream_t stream);

/*
 * Test hook: runs the decode kernel's own block-table gather and INT8
 * matrix product and stores the raw INT32 accumulators, so they can be
 * compared bit for bit. acc_out [num_seqs, num_q_heads, max_blocks_per_seq *
 * block_size] int32; entries at or beyond context_lens[s] are left untouched.
 * [QK-MMAC] §7 (validation layer checking the fragment mapping over full
 * head_dim, paging and scales).
 */
qa_status_t qa_debug_paged_qk_int32(const qa_decode_params_t* p, const int8_t* q_i8,
                                    const int8_t* k_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t* acc_out,
                                    qa_stream_t stream);

/* Shape and options of a chunked-prefill call. */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;          /* must be 16 */
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int64_t total_q;             /* rows of q_i8 = cu_seqlens_q[num_seqs] */
  int32_t max_seqlen_q;        /* >= every cu_seqlens_q[s+1] - cu_seqlens_q[s] */
  qa_dtype_t v_cache_dtype;    /* QA_DT_BF16 or QA_DT_I8 */
  qa_dtype_t out_dtype;        /* QA_DT_F32 or QA_DT_BF16 */
  float softmax_scale;         /* <= 0 selects 1/sqrt(head_dim) */
} qa_prefill_params_t;

/*
 * Chunked prefill over a paged history ([QK-MMAC] §5.2: matrix rows are
 * query tokens, one query head at a time, KV head = query head / G; the
 * query is quantized before attention, §4). Sequence s has
 * Tq = cu_seqlens_q[s+1] - cu_seqlens_q[s] new tokens, which are the last Tq
 * of its context_lens[s] cached tokens (so the chunk must already be written
 * to the cache). Query i of the chunk sits at position ctx - Tq + i and sees
 * keys t <= that position.
 *
 *   q_i8, q_scale  [total_q, num_q_heads, head_dim] int8, [total_q, num_q_heads] fp32
 *   cu_seqlens_q   [num_seqs + 1] int32, non-decreasing, starting at 0
 *   context_lens   [num_seqs] int32 (>= the sequence's Tq)
 *   out            [total_q, num_q_heads, head_dim] fp32 or bf16
 */
qa_status_t qa_chunked_prefill_attention(const qa_prefill_params_t* p, const int8_t* q_i8,
                                         const float* q_scale, const int32_t* cu_seqlens_q,
                                         const int32_t* context_lens, const int8_t* k_cache,
                                         const float* k_scale, const void* v_cache,
                                         const float* v_scale, const int32_t* block_tables,
                                         void* out, qa_stream_t stream);

/*
 * qa_chunked_prefill_attention with V converted once per call: every V block
 * of each sequence's context is rounded to fp16 (INT8 codes exactly) into the
 * workspace, in the order the attention kernel's LDS holds it, and the
 * attention kernel copies those blocks straight into LDS instead of each
 * workgroup converting them again. Same rows, masks and arguments as
 * qa_chunked_prefill_attention ([QK-MMAC] §5.2), and the same arithmetic: the
 * output equals that call's bit for bit.
 *
 *   workspace  >= qa_chunked_prefill_ws_workspace_bytes(p) =
 *              num_seqs * max_blocks_per_seq * num_kv_heads * head_dim * 32
 *              bytes of device memory, 16-byte aligned; no initialization
 *              needed. After the call it holds V as fp16 [num_seqs,
 *              max_blocks_per_seq, num_kv_heads, head_dim, 16] (logical block
 *              j of sequence s; tokens past context_lens[s] zero; blocks
 *              wholly past it left unset). Calls that share a workspace must
 *              not overlap.
 * Errors as qa_chunked_prefill_attention; QA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t qa_chunked_prefill_ws_workspace_bytes(const qa_prefill_params_t* p);
qa_status_t qa_chunked_prefill_attention_ws(const qa_prefill_params_t* p, const int8_t* q_i8,
                                            const float* q_scale, const int32_t* cu_seqlens_q,
                                            const int32_t* context_lens, const int8_t* k_cache,
                                            const float* k_scale, const void* v_cache,
                                            const float* v_scale, const int32_t* block_tables,
                                            void* workspace, size_t workspace_bytes, void* out,
                                            qa_stream_t stream);

/*
 * Chunked prefill with the P.V product in FP8 (E4M3) ([SAGE-MACA] lists the
 * FP8 P.V product of later SageAttention versions among the features its
 * hardware cannot run; the rows, masks and arguments are those of
 * qa_chunked_prefill_attention, [QK-MMAC] §5.2). V of each (sequence, KV
 * head) is scaled per channel over the sequence's context_lens[s] cached
 * tokens, s_c = fl32(max|V| / 448) (INT8 V as fl32(code * scale)), and
 * rounded to E4M3(fl32(V / s_c)); P is rounded to E4M3 at 448 * 2^-3 times
 * exp(score - reference), the reference being moved only when a 128-key tile
 * exceeds it by more than 3 (base 2); out = (sum P8 V8 / sum P8) * s_c. The
 * error is of the order of the E4M3 step (about 2^-4 per rounded term), not
 * of the 16-bit path.
 *
 *   workspace  >= qa_chunked_prefill_fp8pv_workspace_bytes(p) bytes of device
 *              memory, 16-byte aligned; no initialization needed. After the
 *              call it holds, from offset 0, the E4M3 codes as [num_seqs, T,
 *              num_kv_heads, 4, head_dim, 32] bytes (T = ceil(16 *
 *              max_blocks_per_seq / 128); key 32*j + 16*h + e of tile t sits
 *              in group j, byte 16 * (h XOR bit 3 of the channel) + e; zero
 *              past the context), then, at the next multiple of 256 bytes,
 *              the channel scales [num_seqs, num_kv_heads, head_dim] fp32
 *              (left unset for a sequence with no cached token). Calls that
 *              share a workspace must not overlap.
 * Errors as qa_chunked_prefill_attention; QA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t qa_chunked_prefill_fp8pv_workspace_bytes(const qa_prefill_params_t* p);
qa_status_t qa_chunked_prefill_attention_fp8pv(const qa_prefill_params_t* p, const int8_t* q_i8,
                                               const float* q_scale, const int32_t* cu_seqlens_q,
                                               const int32_t* context_lens, const int8_t* k_cache,
                                               const float* k_scale, const void* v_cache,
                                               const float* v_scale, const int32_t* block_tables,
                                               void* workspace, size_t workspace_bytes, void* out,
                                               qa_stream_t stream);

/* Shape and options of a dense SageAttention-style call (NHD layout). */
typedef struct {
  int32_t batch;
  int32_t seq_q;
  int32_t seq_k;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  qa_dtype_t dtype;            /* Q, K, V: QA_DT_F16 or QA_DT_BF16 */
  int32_t smooth_k;            /* 1 = subtract the per-channel K mean */
  int32_t is_causal;
  float softmax_scale;         /* <= 0 selects 1/sqrt(head_dim) */
  qa_dtype_t out_dtype;        /* QA_DT_F32, QA_DT_F16 or QA_DT_BF16 */
} qa_dense_params_t;

/* Query rows per quantization block and key rows per block. */
#define QA_SAGE_Q_BLOCK 128
#define QA_SAGE_K_BLOCK 64

/*
 * SageAttention-style preprocessing ([SAGE-MACA] feature matrix "smooth_k";
 * quantization-kernel table; "per_block" granularity). With smooth_k the
 * per-(batch, KV head, channel) mean of K over all seq_k tokens is
 * accumulated exactly in fp64, divided by seq_k in fp64 and rounded to fp32
 * (mu); K' = fl32(K - mu). Q is quantized per block of QA_SAGE_Q_BLOCK rows of
 * one (batch, head), K' per block of QA_SAGE_K_BLOCK rows, each block with one
 * scale computed over all its rows x head_dim values (same rounding rule as
 * qa_quantize_q; the last block takes the remaining rows).
 *
 *   q [batch, seq_q, num_q_heads, head_dim], k [batch, seq_k, num_kv_heads, head_dim]
 *   q_i8    out, same shape as q, int8
 *   q_scale out [batch, num_q_heads, ceil(seq_q / 128)] fp32
 *   k_i8    out, same shape as k, int8
 *   k_scale out [batch, num_kv_heads, ceil(seq_k / 64)] fp32
 *   k_mean  out [batch, num_kv_heads, head_dim] fp32 (zeros without smooth_k)
 *   workspace  >= qa_dense_sage_quantize_workspace_size bytes (fp64 partial sums)
 */
size_t qa_dense_sage_quantize_workspace_size(const qa_dense_params_t* p);
qa_status_t qa_dense_sage_quantize(const qa_dense_params_t* p, const void* q, const void* k,
                                   int8_t* q_i8, float* q_scale, int8_t* k_i8,
                                   float* k_scale, float* k_mean, void* workspace,
                                   size_t workspace_bytes, qa_stream_t stream);

/*
 * Dense SageAttention-style forward ([SAGE-MACA] attention-kernel compute
 * pipeline, path "accum_f32"): INT8 Q x INT8 K' to INT32, scaled by the
 * query-block scale, the key-block scale and softmax_scale; online softmax in
 * base 2; P.V with fp16 matrix instructions and fp32 accumulation; the
 * causal mask is applied on the diagonal tiles only and tiles above the
 * diagonal are skipped. Causal alignment is bottom-right: query i sees keys
 * j <= i + (seq_k - seq_q). Runs the preprocessing above into the workspace
 * first (full chain). num_q_heads % num_kv_heads == 0; seq_q and seq_k at
 * most 65535 * 16 = 1,048,560 (QA_ERR_UNSUPPORTED beyond; the varlen call
 * has no such bound).
 *
 *   q, k, v   NHD bf16/f16 (dtype); v [batch, seq_k, num_kv_heads, head_dim]
 *   out       [batch, seq_q, num_q_heads, head_dim] in out_dtype
 *   workspace >= qa_dense_sage_workspace_bytes bytes: the preprocessing's fp64
 *             column sums, the Q and K' codes, the V blocks and the block scales
 *             ([SAGE-MACA] quantization-kernel table); no initialization needed.
 *             0 for parameters the call would reject.
 */
size_t qa_dense_sage_workspace_bytes(const qa_dense_params_t* p);
/* The same value under its earlier name. */
size_t qa_dense_sage_workspace_size(const qa_dense_params_t* p);
qa_status_t qa_dense_sage_attention(const qa_dense_params_t* p, const void* q, const void* k,
                                    const void* v, void* workspace, size_t workspace_bytes,
                                    void* out, qa_stream_t stream);

/* Tensor layouts of the dense call: NHD = [batch, seq, heads, head_dim],
 * HND = [batch, heads, seq, head_dim] ([SAGE-MACA] API, tensor_layout). */
typedef enum { QA_LAYOUT_NHD = 0, QA_LAYOUT_HND = 1 } qa_layout_t;

typedef struct {
  int32_t layout;    /* qa_layout_t of q, k, v and out (all four alike) */
  int32_t smooth_v;  /* nonzero: V' = fl16(fl32(V) - mu_v), mu_v the per-(batch, KV head,
                        channel) mean of V over seq_k (fp64 sum, fp32 result); mu_v is added
                        back in fp32 to every output row that sees at least one key */
  int32_t pv_fp8;    /* nonzero: P.V in FP8 E4M3 on the matrix units (head_dim 64 or 128;
                        else QA_ERR_UNSUPPORTED). V (or V' with smooth_v) is quantized per
                        (batch, KV head, channel): s_c = fl32(max |V| / 448), codes
                        E4M3(fl32(V / s_c)) rounded to nearest even; over 64-key tiles the
                        softmax reference m moves to the running row maximum when a tile
                        exceeds it by more than 3 (base 2), and each P is rounded to
                        E4M3(56 exp(score - m)) (56 = 448 / 2^3); O and the row sum accumulate
                        those rounded values in fp32; out = O / l * s_c. Accuracy is that
                        of the E4M3 step (about 2^-4 per rounded term), not of the 16-bit
                        path; the LSE, when asked for, is that of the rounded P */
} qa_dense_options_t;

/*
 * The dense forward with its options ([SAGE-MACA] API: tensor_layout,
 * smooth_k, smooth_v, return_lse). Same computation as
 * qa_dense_sage_attention, plus:
 *   layout    HND inputs and output are accepted as they are (no transpose
 *             pass; the kernels read and write with the layout's strides)
 *   smooth_v  as described in qa_dense_options_t
 *   lse       NULL, or out [batch, num_q_heads, seq_q] fp32: the natural-log
 *             log-sum-exp of each row's scores softmax_scale * q . k over
 *             the keys it sees; with smooth_k the kernel sees K' = K - mu, and
 *             softmax_scale * q . mu (unquantized q, fp32) is added back
 *             (the "LSE correction"), so lse is that of the unsmoothed
 *             scores. Rows that see no key get -inf.
 * options NULL means NHD without smooth_v or FP8 P.V. workspace >=
 * qa_dense_sage_ex_workspace_size bytes (a superset of qa_dense_sage_workspace_bytes).
 * Errors as qa_dense_sage_attention; QA_ERR_INVALID_ARG for an unknown layout.
 */
size_t qa_dense_sage_ex_workspace_size(const qa_dense_params_t* p, const qa_dense_options_t* options);
qa_status_t qa_dense_sage_attention_ex(const qa_dense_params_t* p, const qa_dense_options_t* options,
                                       const void* q, const void* k, const void* v, void* workspace,
                                       size_t workspace_bytes, void* out, float* lse,
                                       qa_stream_t stream);

/*
 * Variable-length dense forward ([SAGE-MACA] API sageattn_varlen, packed
 * format): B independent sequences whose rows are packed one after another,
 * each attended exactly as one sequence of qa_dense_sage_attention_ex would
 * be — smooth_k and smooth_v means per sequence, Q blocks of 128 and K blocks
 * of 64 rows counted from each sequence's first row, causal alignment
 * bottom-right within each sequence — but in one batched launch per pass
 * instead of a loop over sequences (the pages' implementation loops on the
 * host and launches once per sequence).
 *
 *   q     [total_q, num_q_heads, head_dim], k and v [total_k, num_kv_heads, head_dim]
 *         (bf16/f16 dtype, contiguous); sequence b is rows cu_seqlens_q[b] ..
 *         cu_seqlens_q[b+1]-1 of q and cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *         of k and v
 *   cu_seqlens_q, cu_seqlens_k  device int32 [batch+1]: nondecreasing, from 0
 *         to total_q / total_k, no sequence longer than max_seqlen_q /
 *         max_seqlen_k (device data: not checked; rows past max_seqlen are not
 *         computed)
 *   out   [total_q, num_q_heads, head_dim] in out_dtype
 *   lse   NULL or [num_q_heads, total_q] fp32 (natural log, smooth_k
 *         corrected as in qa_dense_sage_attention_ex; -inf for rows that see
 *         no key)
 *   workspace >= qa_dense_sage_varlen_workspace_size bytes (grows with
 *         total_q, total_k, batch and max_seqlen_k)
 * A sequence with no query rows writes nothing; one with queries but no
 * keys gets zero rows. Errors: QA_ERR_INVALID_ARG (null or misaligned
 * pointers, negative sizes), QA_ERR_UNSUPPORTED (dtype, head_dim, GQA ratio,
 * batch or sizes beyond int32 indexing), QA_ERR_WORKSPACE_TOO_SMALL.
 */
typedef struct {
  int32_t batch;
  int64_t total_q, total_k;
  int32_t max_seqlen_q, max_seqlen_k;
  int32_t num_q_heads, num_kv_heads, head_dim;
  qa_dtype_t dtype;            /* QA_DT_F16 or QA_DT_BF16 */
  int32_t smooth_k, smooth_v, is_causal;
  float softmax_scale;         /* <= 0 selects 1/sqrt(head_dim) */
  qa_dtype_t out_dtype;        /* QA_DT_F32, QA_DT_F16 or QA_DT_BF16 */
  int32_t pv_fp8;              /* FP8 P.V as in qa_dense_options_t */
} qa_varlen_params_t;

size_t qa_dense_sage_varlen_workspace_size(const qa_varlen_params_t* p);
qa_status_t qa_dense_sage_attention_varlen(const qa_varlen_params_t* p, const void* q, const void* k,
                                           const void* v, const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, void* workspace,
                                           size_t workspace_bytes, void* out, float* lse,
                                           qa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QATTN_H */
