// C ABI: argument validation, workspace sizing and dispatch. Nothing here
// allocates or synchronizes; all checks run before the first HIP call.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/qattn.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

qa_status_t fail(qa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

qa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QA_OK;
  return fail(QA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define QA_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

float natural_scale(float softmax_scale, int32_t d) {
  return softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / std::sqrt((double)d));
}

float log2_scale(float softmax_scale, int32_t d) {
  const double s = softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / std::sqrt((double)d);
  return (float)(s * 1.4426950408889634);
}

qa_status_t check_decode(const qa_decode_params_t* p) {
  QA_REQUIRE(p != nullptr, QA_ERR_INVALID_ARG, "params is NULL");
  QA_REQUIRE(p->num_seqs >= 0 && p->num_q_heads > 0 && p->num_kv_heads > 0 && p->head_dim > 0,
             QA_ERR_INVALID_ARG, "non-positive shape (num_seqs=%d, heads=%d/%d, head_dim=%d)",
             p->num_seqs, p->num_q_heads, p->num_kv_heads, p->head_dim);
  QA_REQUIRE(p->num_q_heads % p->num_kv_heads == 0, QA_ERR_INVALID_ARG,
             "num_q_heads (%d) not a multiple of num_kv_heads (%d)", p->num_q_heads, p->num_kv_heads);
  QA_REQUIRE(p->max_blocks_per_seq > 0 && p->num_blocks > 0, QA_ERR_INVALID_ARG,
             "max_blocks_per_seq and num_blocks must be positive");
  QA_REQUIRE(p->num_splits >= 0, QA_ERR_INVALID_ARG, "num_splits < 0");
  QA_REQUIRE(p->v_cache_dtype == QA_DT_BF16 || p->v_cache_dtype == QA_DT_I8, QA_ERR_UNSUPPORTED,
             "v_cache_dtype must be BF16 or I8");
  QA_REQUIRE(p->out_dtype == QA_DT_F32 || p->out_dtype == QA_DT_BF16, QA_ERR_UNSUPPORTED,
             "decode out_dtype must be F32 or BF16");
  QA_REQUIRE(supported_dim(p->head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", p->head_dim);
  QA_REQUIRE(p->block_size == 16, QA_ERR_UNSUPPORTED, "block_size %d != 16", p->block_size);
  QA_REQUIRE(p->num_q_heads / p->num_kv_heads <= 16, QA_ERR_UNSUPPORTED,
             "GQA group %d > 16 query heads per KV head", p->num_q_heads / p->num_kv_heads);
  QA_REQUIRE(p->num_splits <= 65535, QA_ERR_UNSUPPORTED, "num_splits %d too large", p->num_splits);
  QA_REQUIRE(p->num_seqs <= 65535 && p->num_kv_heads <= 65535, QA_ERR_UNSUPPORTED, "grid too large");
  QA_REQUIRE((int64_t)p->num_seqs * p->num_q_heads <= (1 << 24), QA_ERR_UNSUPPORTED,
             "num_seqs x num_q_heads %lld > 2^24", (long long)p->num_seqs * p->num_q_heads);
  return QA_OK;
}

int32_t splits_of(const qa_decode_params_t* p) {
  if (p->num_splits > 0) return p->num_splits;
  return qa::choose_decode_splits(p->num_seqs, p->num_kv_heads, p->max_blocks_per_seq);
}

// Decode workspace: [partial O][partial (max, sum)], each part 256-byte aligned.
struct DecodeWs {
  size_t o, ml, total;
};

DecodeWs decode_layout(const qa_decode_params_t* p, int32_t S, int32_t T = 1) {
  DecodeWs w{};
  if (S <= 1) return w;
  const size_t units = (size_t)p->num_seqs * T * p->num_q_heads * S;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.o = 0;
  w.ml = al(units * p->head_dim * sizeof(float));
  w.total = w.ml + al(units * 2 * sizeof(float));
  return w;
}

size_t decode_ws(const qa_decode_params_t* p, int32_t S, int32_t T = 1) { return decode_layout(p, S, T).total; }

// query tokens per sequence of a multi-token decode: G*T columns must fit
// the 16 columns of the matrix instruction
qa_status_t check_tokens(const qa_decode_params_t* p, int32_t T) {
  QA_REQUIRE(T >= 1, QA_ERR_INVALID_ARG, "tokens_per_seq %d < 1", T);
  const int32_t G = p->num_q_heads / p->num_kv_heads;
  QA_REQUIRE((int64_t)G * T <= 16, QA_ERR_UNSUPPORTED, "group %d x %d tokens > 16 query columns", G, T);
  QA_REQUIRE((int64_t)p->num_seqs * T <= 65535, QA_ERR_UNSUPPORTED, "num_seqs x tokens > 65535");
  return QA_OK;
}

qa_status_t producer_impl(const qa_rope_t* rope, const void* q, int64_t num_q_tokens, int32_t num_q_heads,
                          int64_t q_stride_token, int64_t q_stride_head, const void* k, const void* v,
                          int64_t num_kv_tokens, int32_t num_kv_heads, int64_t kv_stride_token,
                          int64_t kv_stride_head, const int64_t* slot_mapping, qa_dtype_t dtype, int32_t head_dim,
                          int64_t num_blocks, int32_t block_size, int8_t* q_i8, float* q_scale, int8_t* k_cache,
                          float* k_scale, void* v_cache, qa_dtype_t v_cache_dtype, float* v_scale,
                          qa_stream_t stream);

qa_status_t check_dense(const qa_dense_params_t* p) {
  QA_REQUIRE(p != nullptr, QA_ERR_INVALID_ARG, "params is NULL");
  QA_REQUIRE(p->batch >= 0 && p->seq_q >= 0 && p->seq_k >= 0 && p->num_q_heads > 0 &&
                 p->num_kv_heads > 0 && p->head_dim > 0,
             QA_ERR_INVALID_ARG, "bad dense shape");
  QA_REQUIRE(p->num_q_heads % p->num_kv_heads == 0, QA_ERR_INVALID_ARG,
             "num_q_heads (%d) not a multiple of num_kv_heads (%d)", p->num_q_heads, p->num_kv_heads);
  QA_REQUIRE(p->dtype == QA_DT_F16 || p->dtype == QA_DT_BF16, QA_ERR_UNSUPPORTED, "dtype must be F16 or BF16");
  QA_REQUIRE(p->out_dtype == QA_DT_F32 || p->out_dtype == QA_DT_F16 || p->out_dtype == QA_DT_BF16,
             QA_ERR_UNSUPPORTED, "out_dtype must be F32, F16 or BF16");
  QA_REQUIRE(supported_dim(p->head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", p->head_dim);
  QA_REQUIRE(p->batch <= 65535 && p->num_q_heads <= 65535, QA_ERR_UNSUPPORTED, "grid too large");
  // the preprocessing grids put 16-token blocks in their second dimension
  QA_REQUIRE(p->seq_q <= 65535 * 16 && p->seq_k <= 65535 * 16, QA_ERR_UNSUPPORTED, "sequence longer than %d tokens",
             65535 * 16);
  return QA_OK;
}

// Element strides (batch, token, head) of a [batch, N, H, D] (NHD) or
// [batch, H, N, D] (HND) tensor.
struct Strides {
  int64_t b, t, h;
};
Strides layout_strides(int32_t layout, int64_t N, int64_t H, int64_t D) {
  if (layout == QA_LAYOUT_HND) return {H * N * D, D, N * D};
  return {N * H * D, H * D, D};
}

// One validated dense call, batched or varlen (packed rows).
struct DenseCall {
  qa::Rows q, k;               // sequence geometry; N = length (batched) or the longest (varlen)
  int32_t Hq, Hkv, D;
  bool bf16, smooth_k, smooth_v, causal, pv_fp8;
  float softmax_scale;
  qa_dtype_t out_dtype;
  Strides sq, sk, so;          // q, k/v, out
  int64_t q_rows() const { return q.packed ? q.total : (int64_t)q.B * q.N; }
};

DenseCall dense_call(const qa_dense_params_t* p, int32_t layout, bool smooth_v, bool pv_fp8 = false) {
  DenseCall c{};
  c.pv_fp8 = pv_fp8;
  c.q = qa::Rows{nullptr, p->batch, p->seq_q, 0, false};
  c.k = qa::Rows{nullptr, p->batch, p->seq_k, 0, false};
  c.Hq = p->num_q_heads; c.Hkv = p->num_kv_heads; c.D = p->head_dim;
  c.bf16 = p->dtype == QA_DT_BF16; c.smooth_k = p->smooth_k != 0; c.smooth_v = smooth_v;
  c.causal = p->is_causal != 0; c.softmax_scale = p->softmax_scale; c.out_dtype = p->out_dtype;
  c.sq = layout_strides(layout, p->seq_q, p->num_q_heads, p->head_dim);
  c.sk = layout_strides(layout, p->seq_k, p->num_kv_heads, p->head_dim);
  c.so = c.sq;
  return c;
}

// Dense workspace: [partial sums][q_i8][k blocks][v blocks][q_scale][k_scale][k_mean], 256-aligned.
// The options and varlen calls append [v_mean][lse_corr]; varlen then adds the
// packed-block maps [q 128-row][k 64-row][k 16-row].
struct DenseWs {
  size_t partial, q_i8, k_blk, v_blk, q_scale, k_scale, k_mean, v_mean, lse_corr, q_map, k_map64, k_map16, v8_scale,
      total;
};

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

DenseWs dense_layout(const DenseCall& c, bool with_attention, bool ex) {
  DenseWs w{};
  const size_t B = c.q.B, Hq = c.Hq, Hkv = c.Hkv, D = c.D, rows_q = c.q_rows();
  const size_t nb16 = c.k.nblocks(16);
  size_t off = 0;
  w.partial = off; off += al(qa::sage_partial_bytes(c.k.B, c.k.N, c.Hkv, c.D));
  if (with_attention) {
    w.q_i8 = off; off += al(rows_q * Hq * D);
    w.k_blk = off; off += al(nb16 * Hkv * D * 16);
    // 16-bit V blocks, or E4M3 blocks of 64 keys for the FP8 P.V
    w.v_blk = off; off += al(c.pv_fp8 ? c.k.nblocks(64) * Hkv * D * 64 : nb16 * Hkv * D * 16 * 2);
    w.q_scale = off; off += al(Hq * c.q.nblocks(128) * sizeof(float));
    w.k_scale = off; off += al(Hkv * c.k.nblocks(64) * sizeof(float));
    w.k_mean = off; off += al(B * Hkv * D * sizeof(float));
    if (ex) {
      w.v_mean = off; off += al(B * Hkv * D * sizeof(float));
      w.lse_corr = off; off += al(Hq * rows_q * sizeof(float));
    }
    if (c.pv_fp8) {
      w.v8_scale = off; off += al(B * Hkv * D * sizeof(float));
    }
    if (c.q.packed) {
      w.q_map = off; off += al(c.q.nblocks(128) * sizeof(int32_t));
      w.k_map64 = off; off += al(c.k.nblocks(64) * sizeof(int32_t));
      w.k_map16 = off; off += al(nb16 * sizeof(int32_t));
    }
  }
  w.total = off;
  return w;
}

// Preprocessing (smooth_k, per-block quantization, V blocks) then attention.
// Pointers, alignment and the workspace size are checked by the caller.
qa_status_t run_dense(const DenseCall& c, const void* q, const void* k, const void* v, char* ws,
                      const DenseWs& w, void* out, float* lse, qa_stream_t stream) {
  qa::SagePrepArgs pa{};
  pa.q = q; pa.k = k; pa.v = v; pa.bf16 = c.bf16;
  pa.q_sb = c.sq.b; pa.q_st = c.sq.t; pa.q_sh = c.sq.h;
  pa.k_sb = c.sk.b; pa.k_st = c.sk.t; pa.k_sh = c.sk.h;
  pa.v_sb = c.sk.b; pa.v_st = c.sk.t; pa.v_sh = c.sk.h;
  pa.q_rows = c.q; pa.k_rows = c.k;
  pa.B = c.q.B; pa.Nq = c.q.N; pa.Nk = c.k.N; pa.Hq = c.Hq; pa.Hkv = c.Hkv; pa.D = c.D;
  pa.smooth_k = c.smooth_k;
  pa.smooth_v = c.smooth_v && c.k.N > 0;
  pa.v_mean = pa.smooth_v ? (float*)(ws + w.v_mean) : nullptr;
  pa.lse_corr = lse != nullptr && pa.smooth_k ? (float*)(ws + w.lse_corr) : nullptr;
  pa.corr_scale = natural_scale(c.softmax_scale, c.D);
  pa.q_i8 = (int8_t*)(ws + w.q_i8); pa.q_scale = (float*)(ws + w.q_scale); pa.k_i8 = nullptr;
  pa.k_paged = (int8_t*)(ws + w.k_blk); pa.k_scale = (float*)(ws + w.k_scale); pa.k_mean = (float*)(ws + w.k_mean);
  pa.partial = (double*)(ws + w.partial); pa.v_paged = (uint16_t*)(ws + w.v_blk);
  if (c.pv_fp8) {
    pa.v_paged = nullptr;
    pa.v8 = (uint8_t*)(ws + w.v_blk);
    pa.v8_scale = (float*)(ws + w.v8_scale);
  }
  if (c.q.packed) {
    pa.q_map = (int32_t*)(ws + w.q_map); pa.k_map64 = (int32_t*)(ws + w.k_map64);
    pa.k_map16 = (int32_t*)(ws + w.k_map16);
  }
  // the attention kernel quantizes its own query block (one workgroup, one
  // 128-row block of one head) unless the LSE correction needs the separate pass
  pa.skip_q = pa.lse_corr == nullptr;
  // fp16 V without smooth_v: the attention kernel copies V tiles in token
  // order (no V block pass)
  pa.skip_v = !c.bf16 && !pa.smooth_v && !c.pv_fp8 && c.k.N > 0;
  qa_status_t st = hip_status(qa::launch_sage_prep(pa, (hipStream_t)stream), "dense preprocessing launch");
  if (st != QA_OK) return st;
  qa::FlashArgs a{};
  a.q = pa.q_i8; a.q_scale = pa.q_scale; a.k_blocks = pa.k_paged; a.k_scale = pa.k_scale; a.v_blocks = pa.v_paged;
  if (pa.skip_q) {
    a.q_in = (const uint16_t*)q; a.q_sb = c.sq.b; a.q_st = c.sq.t; a.q_sh = c.sq.h; a.q_in_bf16 = c.bf16;
  }
  if (pa.skip_v) {
    a.v_tok = (const uint16_t*)v; a.v_sb = c.sk.b; a.v_st = c.sk.t; a.v_sh = c.sk.h;
  }
  if (c.pv_fp8) { a.v_blocks = pa.v8; a.v8_scale = pa.v8_scale; a.pv_fp8 = true; }
  a.v_scale = nullptr; a.tables = nullptr; a.cu_q = nullptr; a.ctx_lens = nullptr; a.out = out;
  a.o_sb = c.so.b; a.o_st = c.so.t; a.o_sh = c.so.h;
  a.v_mean = pa.v_mean; a.lse = lse; a.lse_corr = pa.lse_corr;
  a.q_rows = c.q; a.k_rows = c.k; a.q_map = pa.q_map;
  a.num_seqs = c.q.B; a.Hq = c.Hq; a.Hkv = c.Hkv; a.G = c.Hq / c.Hkv;
  a.D = c.D; a.max_blocks = 0; a.max_seqlen_q = c.q.N; a.Nq = c.q.N; a.Nk = c.k.N;
  a.scale_log2 = log2_scale(c.softmax_scale, c.D);
  a.dense = true; a.causal = c.causal; a.v_int8 = false; a.v_f16 = true;  // V blocks are fp16
  a.out_bf16 = c.out_dtype == QA_DT_BF16; a.out_f16 = c.out_dtype == QA_DT_F16;
  return hip_status(qa::launch_flash(a, (hipStream_t)stream), "dense attention launch");
}

qa_status_t dense_attention_impl(const qa_dense_params_t* p, const qa_dense_options_t* o, const void* q,
                                 const void* k, const void* v, void* workspace, size_t workspace_bytes,
                                 void* out, float* lse, qa_stream_t stream, bool ex) {
  qa_status_t st = check_dense(p);
  if (st != QA_OK) return st;
  const int32_t layout = o ? o->layout : QA_LAYOUT_NHD;
  QA_REQUIRE(layout == QA_LAYOUT_NHD || layout == QA_LAYOUT_HND, QA_ERR_INVALID_ARG, "unknown layout %d",
             layout);
  if (p->batch == 0 || p->seq_q == 0) return QA_OK;
  QA_REQUIRE(q && k && v && out && workspace, QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(workspace),
             QA_ERR_INVALID_ARG, "q, k, v, out and workspace must be 16-byte aligned");
  QA_REQUIRE(((uintptr_t)lse & 3u) == 0, QA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const bool fp8 = o && o->pv_fp8 != 0;
  QA_REQUIRE(!fp8 || p->head_dim <= 128, QA_ERR_UNSUPPORTED, "FP8 P.V needs head_dim 64 or 128");
  const DenseCall c = dense_call(p, layout, o && o->smooth_v != 0, fp8);
  const DenseWs w = dense_layout(c, true, ex);
  QA_REQUIRE(workspace_bytes >= w.total, QA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
             workspace_bytes, w.total);
  return run_dense(c, q, k, v, (char*)workspace, w, out, lse, stream);
}

qa_status_t check_varlen(const qa_varlen_params_t* p) {
  QA_REQUIRE(p != nullptr, QA_ERR_INVALID_ARG, "params is NULL");
  QA_REQUIRE(p->batch >= 0 && p->total_q >= 0 && p->total_k >= 0 && p->max_seqlen_q >= 0 &&
                 p->max_seqlen_k >= 0 && p->num_q_heads > 0 && p->num_kv_heads > 0 && p->head_dim > 0,
             QA_ERR_INVALID_ARG, "bad varlen shape");
  QA_REQUIRE(p->num_q_heads % p->num_kv_heads == 0, QA_ERR_INVALID_ARG,
             "num_q_heads (%d) not a multiple of num_kv_heads (%d)", p->num_q_heads, p->num_kv_heads);
  QA_REQUIRE(p->dtype == QA_DT_F16 || p->dtype == QA_DT_BF16, QA_ERR_UNSUPPORTED, "dtype must be F16 or BF16");
  QA_REQUIRE(p->out_dtype == QA_DT_F32 || p->out_dtype == QA_DT_F16 || p->out_dtype == QA_DT_BF16,
             QA_ERR_UNSUPPORTED, "out_dtype must be F32, F16 or BF16");
  QA_REQUIRE(supported_dim(p->head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", p->head_dim);
  QA_REQUIRE(p->batch <= 65535 && p->num_q_heads <= 65535, QA_ERR_UNSUPPORTED, "grid too large");
  QA_REQUIRE(p->total_q <= INT32_MAX && p->total_k <= INT32_MAX, QA_ERR_UNSUPPORTED,
             "total rows beyond int32 offsets");
  QA_REQUIRE(p->pv_fp8 == 0 || p->head_dim <= 128, QA_ERR_UNSUPPORTED, "FP8 P.V needs head_dim 64 or 128");
  return QA_OK;
}

DenseCall varlen_call(const qa_varlen_params_t* p, const int32_t* cu_q, const int32_t* cu_k) {
  DenseCall c{};
  c.q = qa::Rows{cu_q, p->batch, p->max_seqlen_q, p->total_q, true};
  c.k = qa::Rows{cu_k, p->batch, p->max_seqlen_k, p->total_k, true};
  c.Hq = p->num_q_heads; c.Hkv = p->num_kv_heads; c.D = p->head_dim;
  c.bf16 = p->dtype == QA_DT_BF16; c.smooth_k = p->smooth_k != 0; c.smooth_v = p->smooth_v != 0;
  c.causal = p->is_causal != 0; c.softmax_scale = p->softmax_scale; c.out_dtype = p->out_dtype;
  c.pv_fp8 = p->pv_fp8 != 0;
  const int64_t D = p->head_dim;
  c.sq = Strides{0, p->num_q_heads * D, D};     // packed [total, H, D] rows
  c.sk = Strides{0, p->num_kv_heads * D, D};
  c.so = c.sq;
  return c;
}

}  // namespace

extern "C" {

int qa_abi_version(void) { return QA_ABI_VERSION; }

const char* qa_last_error(void) { return g_err.c_str(); }

qa_status_t qa_quantize_q(const void* q, qa_dtype_t dtype, int64_t num_tokens, int32_t num_heads,
                          int32_t head_dim, int64_t stride_token, int64_t stride_head, int8_t* q_i8,
                          float* q_scale, qa_stream_t stream) {
  QA_REQUIRE(num_tokens >= 0 && num_heads > 0 && head_dim > 0, QA_ERR_INVALID_ARG,
             "bad shape (tokens=%lld, heads=%d, head_dim=%d)", (long long)num_tokens, num_heads, head_dim);
  QA_REQUIRE(dtype == QA_DT_BF16 || dtype == QA_DT_F16, QA_ERR_UNSUPPORTED, "dtype must be BF16 or F16");
  QA_REQUIRE(supported_dim(head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  if (num_tokens == 0) return QA_OK;
  QA_REQUIRE(q && q_i8 && q_scale, QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(aligned16(q) && stride_token % 8 == 0 && stride_head % 8 == 0 && stride_token >= 0 &&
                 stride_head >= 0,
             QA_ERR_INVALID_ARG, "q must be 16-byte aligned with strides that are multiples of 8 elements");
  QA_REQUIRE(((uintptr_t)q_i8 & 7u) == 0, QA_ERR_INVALID_ARG, "q_i8 must be 8-byte aligned");
  QA_REQUIRE(num_tokens * num_heads / 4 < (int64_t)INT32_MAX, QA_ERR_UNSUPPORTED, "too many rows");
  return hip_status(qa::launch_quantize_rows(q, dtype == QA_DT_BF16, num_tokens, num_heads, head_dim,
                                             stride_token, stride_head, q_i8, q_scale, (hipStream_t)stream),
                    "qa_quantize_q launch");
}

qa_status_t qa_write_kv_cache(const void* k, const void* v, qa_dtype_t dtype, int64_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int64_t stride_token,
                              int64_t stride_head, const int64_t* slot_mapping, int64_t num_blocks,
                              int32_t block_size, int8_t* k_cache, float* k_scale, void* v_cache,
                              qa_dtype_t v_cache_dtype, float* v_scale, qa_stream_t stream) {
  QA_REQUIRE(num_tokens >= 0 && num_kv_heads > 0 && head_dim > 0 && num_blocks > 0, QA_ERR_INVALID_ARG,
             "bad shape");
  QA_REQUIRE(dtype == QA_DT_BF16 || dtype == QA_DT_F16, QA_ERR_UNSUPPORTED, "dtype must be BF16 or F16");
  QA_REQUIRE(v_cache_dtype == dtype || v_cache_dtype == QA_DT_I8, QA_ERR_UNSUPPORTED,
             "v_cache_dtype must equal dtype or be I8");
  QA_REQUIRE(supported_dim(head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  QA_REQUIRE(block_size == 16, QA_ERR_UNSUPPORTED, "block_size %d != 16", block_size);
  if (num_tokens == 0) return QA_OK;
  QA_REQUIRE(k && v && slot_mapping && k_cache && k_scale && v_cache, QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(v_cache_dtype != QA_DT_I8 || v_scale != nullptr, QA_ERR_INVALID_ARG, "INT8 V needs v_scale");
  QA_REQUIRE(aligned16(k) && aligned16(v) && stride_token % 8 == 0 && stride_head % 8 == 0 &&
                 stride_token >= 0 && stride_head >= 0,
             QA_ERR_INVALID_ARG, "k/v must be 16-byte aligned with strides that are multiples of 8 elements");
  QA_REQUIRE(aligned16(k_cache), QA_ERR_INVALID_ARG, "k_cache must be 16-byte aligned");
  QA_REQUIRE(num_tokens * num_kv_heads / 4 < (int64_t)INT32_MAX, QA_ERR_UNSUPPORTED, "too many rows");
  return hip_status(qa::launch_write_kv_cache(k, v, dtype == QA_DT_BF16, num_tokens, num_kv_heads, head_dim,
                                              stride_token, stride_head, slot_mapping, k_cache, k_scale,
                                              v_cache, v_cache_dtype == QA_DT_I8, v_scale,
                                              (hipStream_t)stream),
                    "qa_write_kv_cache launch");
}

qa_status_t qa_quantize_q_write_kv(const void* q, int64_t num_q_tokens, int32_t num_q_heads,
                                   int64_t q_stride_token, int64_t q_stride_head, const void* k,
                                   const void* v, int64_t num_kv_tokens, int32_t num_kv_heads,
                                   int64_t kv_stride_token, int64_t kv_stride_head,
                                   const int64_t* slot_mapping, qa_dtype_t dtype, int32_t head_dim,
                                   int64_t num_blocks, int32_t block_size, int8_t* q_i8, float* q_scale,
                                   int8_t* k_cache, float* k_scale, void* v_cache,
                                   qa_dtype_t v_cache_dtype, float* v_scale, qa_stream_t stream) {
  return producer_impl(nullptr, q, num_q_tokens, num_q_heads, q_stride_token, q_stride_head, k, v, num_kv_tokens,
                       num_kv_heads, kv_stride_token, kv_stride_head, slot_mapping, dtype, head_dim, num_blocks,
                       block_size, q_i8, q_scale, k_cache, k_scale, v_cache, v_cache_dtype, v_scale, stream);
}

qa_status_t qa_rope_quantize_q_write_kv(const qa_rope_t* rope, const void* q, int64_t num_q_tokens,
                                        int32_t num_q_heads, int64_t q_stride_token, int64_t q_stride_head,
                                        const void* k, const void* v, int64_t num_kv_tokens, int32_t num_kv_heads,
                                        int64_t kv_stride_token, int64_t kv_stride_head,
                                        const int64_t* slot_mapping, qa_dtype_t dtype, int32_t head_dim,
                                        int64_t num_blocks, int32_t block_size, int8_t* q_i8, float* q_scale,
                                        int8_t* k_cache, float* k_scale, void* v_cache, qa_dtype_t v_cache_dtype,
                                        float* v_scale, qa_stream_t stream) {
  QA_REQUIRE(rope != nullptr && rope->positions != nullptr && rope->cos_sin != nullptr, QA_ERR_INVALID_ARG,
             "rope, its positions and its table must be given");
  QA_REQUIRE(rope->rot_dim >= 2 && rope->rot_dim % 2 == 0 && rope->rot_dim <= head_dim, QA_ERR_INVALID_ARG,
             "rot_dim %d must be even and in [2, head_dim]", rope->rot_dim);
  return producer_impl(rope, q, num_q_tokens, num_q_heads, q_stride_token, q_stride_head, k, v, num_kv_tokens,
                       num_kv_heads, kv_stride_token, kv_stride_head, slot_mapping, dtype, head_dim, num_blocks,
                       block_size, q_i8, q_scale, k_cache, k_scale, v_cache, v_cache_dtype, v_scale, stream);
}

}  // extern "C"

namespace {

qa_status_t producer_impl(const qa_rope_t* rope, const void* q, int64_t num_q_tokens, int32_t num_q_heads,
                          int64_t q_stride_token, int64_t q_stride_head, const void* k, const void* v,
                          int64_t num_kv_tokens, int32_t num_kv_heads, int64_t kv_stride_token,
                          int64_t kv_stride_head, const int64_t* slot_mapping, qa_dtype_t dtype, int32_t head_dim,
                          int64_t num_blocks, int32_t block_size, int8_t* q_i8, float* q_scale, int8_t* k_cache,
                          float* k_scale, void* v_cache, qa_dtype_t v_cache_dtype, float* v_scale,
                          qa_stream_t stream) {
  QA_REQUIRE(num_q_tokens >= 0 && num_kv_tokens >= 0 && num_q_heads > 0 && num_kv_heads > 0 && head_dim > 0 &&
                 num_blocks > 0,
             QA_ERR_INVALID_ARG, "bad shape");
  QA_REQUIRE(dtype == QA_DT_BF16 || dtype == QA_DT_F16, QA_ERR_UNSUPPORTED, "dtype must be BF16 or F16");
  QA_REQUIRE(v_cache_dtype == dtype || v_cache_dtype == QA_DT_I8, QA_ERR_UNSUPPORTED,
             "v_cache_dtype must equal dtype or be I8");
  QA_REQUIRE(supported_dim(head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  QA_REQUIRE(block_size == 16, QA_ERR_UNSUPPORTED, "block_size %d != 16", block_size);
  if (num_q_tokens == 0 && num_kv_tokens == 0) return QA_OK;
  if (num_q_tokens > 0) {
    QA_REQUIRE(q && q_i8 && q_scale, QA_ERR_INVALID_ARG, "null query pointer");
    QA_REQUIRE(aligned16(q) && q_stride_token % 8 == 0 && q_stride_head % 8 == 0 && q_stride_token >= 0 &&
                   q_stride_head >= 0,
               QA_ERR_INVALID_ARG, "q must be 16-byte aligned with strides that are multiples of 8 elements");
  }
  if (num_kv_tokens > 0) {
    QA_REQUIRE(k && v && slot_mapping && k_cache && k_scale && v_cache, QA_ERR_INVALID_ARG, "null cache pointer");
    QA_REQUIRE(v_cache_dtype != QA_DT_I8 || v_scale != nullptr, QA_ERR_INVALID_ARG, "INT8 V needs v_scale");
    QA_REQUIRE(aligned16(k) && aligned16(v) && kv_stride_token % 8 == 0 && kv_stride_head % 8 == 0 &&
                   kv_stride_token >= 0 && kv_stride_head >= 0 && aligned16(k_cache),
               QA_ERR_INVALID_ARG, "k/v must be 16-byte aligned with strides that are multiples of 8 elements");
  }
  QA_REQUIRE((num_q_tokens * num_q_heads + num_kv_tokens * num_kv_heads) / 4 < (int64_t)INT32_MAX,
             QA_ERR_UNSUPPORTED, "too many rows");
  qa::ProducerArgs a{};
  a.q = q; a.k = k; a.v = v; a.slots = slot_mapping; a.bf16 = dtype == QA_DT_BF16;
  a.v_int8 = v_cache_dtype == QA_DT_I8; a.D = head_dim; a.Hq = num_q_heads; a.Hkv = num_kv_heads;
  a.q_rows = num_q_tokens * num_q_heads; a.kv_rows = num_kv_tokens * num_kv_heads;
  a.q_st = q_stride_token; a.q_sh = q_stride_head; a.kv_st = kv_stride_token; a.kv_sh = kv_stride_head;
  a.q_i8 = q_i8; a.q_scale = q_scale; a.k_cache = k_cache; a.k_scale = k_scale; a.v_cache = v_cache;
  a.v_scale = v_scale;
  if (rope != nullptr) a.rope = qa::Rope{rope->positions, rope->cos_sin, rope->rot_dim, rope->neox != 0};
  return hip_status(qa::launch_producer(a, (hipStream_t)stream), "producer launch");
}

}  // namespace

extern "C" {

int32_t qa_paged_decode_num_splits(const qa_decode_params_t* p) {
  if (check_decode(p) != QA_OK) return -1;
  return splits_of(p);
}

size_t qa_paged_decode_workspace_bytes(const qa_decode_params_t* p) {
  if (check_decode(p) != QA_OK) return 0;
  return decode_ws(p, splits_of(p));
}

size_t qa_paged_decode_workspace_size(const qa_decode_params_t* p) { return qa_paged_decode_workspace_bytes(p); }

namespace {

qa_status_t decode_call(const qa_decode_params_t* p, const int8_t* q_i8, const float* q_scale,
                        const int8_t* k_cache, const float* k_scale, const void* v_cache, const float* v_scale,
                        const int32_t* block_tables, const int32_t* context_lens, void* workspace,
                        size_t workspace_bytes, void* out, qa_stream_t stream, qa::DecodePhase phase,
                        const char* what, int32_t T = 1) {
  qa_status_t st = check_decode(p);
  if (st != QA_OK) return st;
  st = check_tokens(p, T);
  if (st != QA_OK) return st;
  if (p->num_seqs == 0) return QA_OK;
  const bool combine_only = phase == qa::DecodePhase::kCombine;
  if (!combine_only) {
    QA_REQUIRE(q_i8 && q_scale && k_cache && k_scale && v_cache && block_tables && context_lens,
               QA_ERR_INVALID_ARG, "null pointer");
    QA_REQUIRE(p->v_cache_dtype != QA_DT_I8 || v_scale != nullptr, QA_ERR_INVALID_ARG, "INT8 V needs v_scale");
    QA_REQUIRE(aligned16(q_i8) && aligned16(k_cache) && aligned16(k_scale) && aligned16(v_cache) &&
                   (v_scale == nullptr || aligned16(v_scale)),
               QA_ERR_INVALID_ARG, "q_i8, caches and scales must be 16-byte aligned");
  }
  QA_REQUIRE(out != nullptr, QA_ERR_INVALID_ARG, "null pointer");
  const int32_t S = splits_of(p);
  const size_t need = decode_ws(p, S, T);
  QA_REQUIRE(workspace_bytes >= need, QA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
             workspace_bytes, need);
  QA_REQUIRE(need == 0 || workspace != nullptr, QA_ERR_INVALID_ARG, "workspace is NULL");
  QA_REQUIRE(need == 0 || aligned16(workspace), QA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  qa::DecodeArgs a{};
  a.q = q_i8; a.q_scale = q_scale; a.k_cache = k_cache; a.k_scale = k_scale; a.v_cache = v_cache;
  a.v_scale = v_scale; a.tables = block_tables; a.ctx_lens = context_lens; a.out = out;
  const DecodeWs w = decode_layout(p, S, T);
  a.ws_o = need ? (float*)((char*)workspace + w.o) : nullptr;
  a.ws_ml = need ? (float*)((char*)workspace + w.ml) : nullptr;
  a.num_seqs = p->num_seqs; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads; a.D = p->head_dim; a.max_blocks = p->max_blocks_per_seq;
  a.num_splits = S; a.scale_log2 = log2_scale(p->softmax_scale, p->head_dim);
  a.v_int8 = p->v_cache_dtype == QA_DT_I8; a.out_bf16 = p->out_dtype == QA_DT_BF16;
  a.tq = T;
  a.seq_split = p->num_seqs > 1;
  a.lpt = p->num_seqs > 1 && p->num_seqs <= 64;
  return hip_status(qa::launch_decode(a, phase, (hipStream_t)stream), what);
}

}  // namespace

namespace {

qa_status_t decode_step(const qa_decode_params_t* p, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                        const void* k, const void* v, int64_t kv_stride_token, int64_t kv_stride_head,
                        qa_dtype_t dtype, const int64_t* slot_mapping, int8_t* k_cache, float* k_scale,
                        void* v_cache, float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
                        void* workspace, size_t workspace_bytes, void* out, qa_stream_t stream,
                        qa::DecodePhase phase, const char* what, const qa_rope_t* rope = nullptr) {
  qa_status_t st = check_decode(p);
  if (st != QA_OK) return st;
  if (rope != nullptr) {
    QA_REQUIRE(rope->positions != nullptr && rope->cos_sin != nullptr, QA_ERR_INVALID_ARG,
               "rope positions and table must be given");
    QA_REQUIRE(rope->rot_dim >= 2 && rope->rot_dim % 2 == 0 && rope->rot_dim <= p->head_dim, QA_ERR_INVALID_ARG,
               "rot_dim %d must be even and in [2, head_dim]", rope->rot_dim);
  }
  if (p->num_seqs == 0) return QA_OK;
  QA_REQUIRE(dtype == QA_DT_BF16 || dtype == QA_DT_F16, QA_ERR_UNSUPPORTED, "dtype must be BF16 or F16");
  QA_REQUIRE(p->v_cache_dtype == QA_DT_I8 || dtype == QA_DT_BF16, QA_ERR_UNSUPPORTED,
             "a BF16 V cache needs BF16 inputs");
  QA_REQUIRE(q && k && v && slot_mapping && k_cache && k_scale && v_cache && block_tables && context_lens && out,
             QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(p->v_cache_dtype != QA_DT_I8 || v_scale != nullptr, QA_ERR_INVALID_ARG, "INT8 V needs v_scale");
  QA_REQUIRE(q_stride_token >= 0 && q_stride_head >= 0 && kv_stride_token >= 0 && kv_stride_head >= 0,
             QA_ERR_INVALID_ARG, "negative stride");
  QA_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) % 2 == 0, QA_ERR_INVALID_ARG,
             "q, k and v must be 2-byte aligned");
  QA_REQUIRE(aligned16(k_cache) && aligned16(k_scale) && aligned16(v_cache) &&
                 (v_scale == nullptr || aligned16(v_scale)),
             QA_ERR_INVALID_ARG, "caches and scales must be 16-byte aligned");
  const int32_t S = splits_of(p);
  const size_t need = decode_ws(p, S);
  QA_REQUIRE(workspace_bytes >= need, QA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
             workspace_bytes, need);
  QA_REQUIRE(need == 0 || workspace != nullptr, QA_ERR_INVALID_ARG, "workspace is NULL");
  QA_REQUIRE(need == 0 || aligned16(workspace), QA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  qa::DecodeArgs a{};
  a.k_cache = k_cache; a.k_scale = k_scale; a.v_cache = v_cache; a.v_scale = v_scale;
  a.tables = block_tables; a.ctx_lens = context_lens; a.out = out;
  const DecodeWs w = decode_layout(p, S);
  a.ws_o = need ? (float*)((char*)workspace + w.o) : nullptr;
  a.ws_ml = need ? (float*)((char*)workspace + w.ml) : nullptr;
  a.num_seqs = p->num_seqs; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads; a.D = p->head_dim; a.max_blocks = p->max_blocks_per_seq;
  a.num_splits = S; a.scale_log2 = log2_scale(p->softmax_scale, p->head_dim);
  a.v_int8 = p->v_cache_dtype == QA_DT_I8; a.out_bf16 = p->out_dtype == QA_DT_BF16;
  a.q_in = (const uint16_t*)q; a.k_new = (const uint16_t*)k; a.v_new = (const uint16_t*)v;
  a.q_st = q_stride_token; a.q_sh = q_stride_head; a.kv_st = kv_stride_token; a.kv_sh = kv_stride_head;
  a.slots = slot_mapping; a.kc_w = k_cache; a.ks_w = k_scale; a.vc_w = v_cache; a.vs_w = v_scale;
  a.in_bf16 = dtype == QA_DT_BF16;
  a.tq = 1;
  a.seq_split = p->num_seqs > 1;
  a.lpt = p->num_seqs > 1 && p->num_seqs <= 64;
  if (rope != nullptr) a.rope = qa::Rope{rope->positions, rope->cos_sin, rope->rot_dim, rope->neox != 0};
  return hip_status(qa::launch_decode(a, phase, (hipStream_t)stream), what);
}

}  // namespace

qa_status_t qa_paged_decode_step(const qa_decode_params_t* p, const void* q, int64_t q_stride_token,
                                 int64_t q_stride_head, const void* k, const void* v, int64_t kv_stride_token,
                                 int64_t kv_stride_head, qa_dtype_t dtype, const int64_t* slot_mapping,
                                 int8_t* k_cache, float* k_scale, void* v_cache, float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens, void* workspace,
                                 size_t workspace_bytes, void* out, qa_stream_t stream) {
  return decode_step(p, q, q_stride_token, q_stride_head, k, v, kv_stride_token, kv_stride_head, dtype,
                     slot_mapping, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kBoth, "qa_paged_decode_step launch");
}

qa_status_t qa_paged_decode_step_rope(const qa_rope_t* rope, const qa_decode_params_t* p, const void* q,
                                      int64_t q_stride_token, int64_t q_stride_head, const void* k, const void* v,
                                      int64_t kv_stride_token, int64_t kv_stride_head, qa_dtype_t dtype,
                                      const int64_t* slot_mapping, int8_t* k_cache, float* k_scale, void* v_cache,
                                      float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
                                      void* workspace, size_t workspace_bytes, void* out, qa_stream_t stream) {
  QA_REQUIRE(rope != nullptr, QA_ERR_INVALID_ARG, "rope is NULL");
  return decode_step(p, q, q_stride_token, q_stride_head, k, v, kv_stride_token, kv_stride_head, dtype,
                     slot_mapping, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kBoth, "qa_paged_decode_step_rope launch", rope);
}

qa_status_t qa_paged_decode_step_partials(const qa_decode_params_t* p, const void* q, int64_t q_stride_token,
                                          int64_t q_stride_head, const void* k, const void* v,
                                          int64_t kv_stride_token, int64_t kv_stride_head, qa_dtype_t dtype,
                                          const int64_t* slot_mapping, int8_t* k_cache, float* k_scale,
                                          void* v_cache, float* v_scale, const int32_t* block_tables,
                                          const int32_t* context_lens, void* workspace, size_t workspace_bytes,
                                          void* out, qa_stream_t stream) {
  return decode_step(p, q, q_stride_token, q_stride_head, k, v, kv_stride_token, kv_stride_head, dtype,
                     slot_mapping, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kPartials,
                     "qa_paged_decode_step_partials launch");
}

qa_status_t qa_paged_attention_decode(const qa_decode_params_t* p, const int8_t* q_i8, const float* q_scale,
                                      const int8_t* k_cache, const float* k_scale, const void* v_cache,
                                      const float* v_scale, const int32_t* block_tables,
                                      const int32_t* context_lens, void* workspace, size_t workspace_bytes,
                                      void* out, qa_stream_t stream) {
  return decode_call(p, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kBoth, "qa_paged_attention_decode launch");
}

qa_status_t qa_paged_attention_decode_partials(const qa_decode_params_t* p, const int8_t* q_i8,
                                               const float* q_scale, const int8_t* k_cache, const float* k_scale,
                                               const void* v_cache, const float* v_scale,
                                               const int32_t* block_tables, const int32_t* context_lens,
                                               void* workspace, size_t workspace_bytes, void* out,
                                               qa_stream_t stream) {
  return decode_call(p, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kPartials,
                     "qa_paged_attention_decode_partials launch");
}

qa_status_t qa_paged_attention_decode_noalloc(const qa_decode_params_t* p, const int8_t* q_i8, const float* q_scale,
                                              const int8_t* k_cache, const float* k_scale, const void* v_cache,
                                              const float* v_scale, const int32_t* block_tables,
                                              const int32_t* context_lens, void* out, qa_stream_t stream) {
  static_assert(QA_DECODE_SCRATCH_BYTES == qa::kDecodeScratchBytes, "scratch size in the header");
  qa_status_t st = check_decode(p);
  if (st != QA_OK) return st;
  if (p->num_seqs == 0) return QA_OK;
  const size_t need = decode_ws(p, splits_of(p));
  QA_REQUIRE(need <= qa::kDecodeScratchBytes, QA_ERR_WORKSPACE_TOO_SMALL,
             "split partials need %zu bytes; the static decode scratch holds %zu (lower num_splits or num_seqs)",
             need, (size_t)qa::kDecodeScratchBytes);
  // the checks of the workspace call, before the scratch lookup (the first HIP call)
  QA_REQUIRE(q_i8 && q_scale && k_cache && k_scale && v_cache && block_tables && context_lens && out,
             QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(p->v_cache_dtype != QA_DT_I8 || v_scale != nullptr, QA_ERR_INVALID_ARG, "INT8 V needs v_scale");
  QA_REQUIRE(aligned16(q_i8) && aligned16(k_cache) && aligned16(k_scale) && aligned16(v_cache) &&
                 (v_scale == nullptr || aligned16(v_scale)),
             QA_ERR_INVALID_ARG, "q_i8, caches and scales must be 16-byte aligned");
  void* ws = nullptr;
  if (need > 0) {
    st = hip_status(qa::decode_scratch(&ws), "decode scratch lookup");
    if (st != QA_OK) return st;
  }
  return decode_call(p, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, ws,
                     qa::kDecodeScratchBytes, out, stream, qa::DecodePhase::kBoth,
                     "qa_paged_attention_decode_noalloc launch");
}

size_t qa_paged_decode_mt_workspace_size(const qa_decode_params_t* p, int32_t tokens_per_seq) {
  if (check_decode(p) != QA_OK || check_tokens(p, tokens_per_seq) != QA_OK) return 0;
  return decode_ws(p, splits_of(p), tokens_per_seq);
}

qa_status_t qa_paged_attention_decode_mt(const qa_decode_params_t* p, int32_t tokens_per_seq, const int8_t* q_i8,
                                         const float* q_scale, const int8_t* k_cache, const float* k_scale,
                                         const void* v_cache, const float* v_scale, const int32_t* block_tables,
                                         const int32_t* context_lens, void* workspace, size_t workspace_bytes,
                                         void* out, qa_stream_t stream) {
  return decode_call(p, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kBoth, "qa_paged_attention_decode_mt launch",
                     tokens_per_seq);
}

qa_status_t qa_paged_attention_decode_combine(const qa_decode_params_t* p, void* workspace, size_t workspace_bytes,
                                              void* out, qa_stream_t stream) {
  return decode_call(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, workspace,
                     workspace_bytes, out, stream, qa::DecodePhase::kCombine,
                     "qa_paged_attention_decode_combine launch");
}

qa_status_t qa_debug_paged_qk_int32(const qa_decode_params_t* p, const int8_t* q_i8, const int8_t* k_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t* acc_out, qa_stream_t stream) {
  qa_status_t st = check_decode(p);
  if (st != QA_OK) return st;
  if (p->num_seqs == 0) return QA_OK;
  QA_REQUIRE(q_i8 && k_cache && block_tables && context_lens && acc_out, QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(aligned16(q_i8) && aligned16(k_cache), QA_ERR_INVALID_ARG, "q_i8 and k_cache must be 16-byte aligned");
  qa::DecodeArgs a{};
  a.q = q_i8; a.k_cache = k_cache; a.tables = block_tables; a.ctx_lens = context_lens; a.acc_out = acc_out;
  a.num_seqs = p->num_seqs; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads; a.D = p->head_dim; a.max_blocks = p->max_blocks_per_seq;
  a.num_splits = 1; a.scale_log2 = 1.0f; a.v_int8 = false; a.tq = 1;
  return hip_status(qa::launch_debug_qk(a, (hipStream_t)stream), "qa_debug_paged_qk_int32 launch");
}

namespace {

qa_status_t check_prefill(const qa_prefill_params_t* p) {
  QA_REQUIRE(p != nullptr, QA_ERR_INVALID_ARG, "params is NULL");
  QA_REQUIRE(p->num_seqs >= 0 && p->num_q_heads > 0 && p->num_kv_heads > 0 && p->head_dim > 0 &&
                 p->total_q >= 0 && p->max_seqlen_q >= 0,
             QA_ERR_INVALID_ARG, "bad prefill shape");
  QA_REQUIRE(p->num_q_heads % p->num_kv_heads == 0, QA_ERR_INVALID_ARG,
             "num_q_heads (%d) not a multiple of num_kv_heads (%d)", p->num_q_heads, p->num_kv_heads);
  QA_REQUIRE(p->max_blocks_per_seq > 0 && p->num_blocks > 0, QA_ERR_INVALID_ARG,
             "max_blocks_per_seq and num_blocks must be positive");
  QA_REQUIRE(p->v_cache_dtype == QA_DT_BF16 || p->v_cache_dtype == QA_DT_I8, QA_ERR_UNSUPPORTED,
             "v_cache_dtype must be BF16 or I8");
  QA_REQUIRE(p->out_dtype == QA_DT_F32 || p->out_dtype == QA_DT_BF16, QA_ERR_UNSUPPORTED,
             "prefill out_dtype must be F32 or BF16");
  QA_REQUIRE(supported_dim(p->head_dim), QA_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", p->head_dim);
  QA_REQUIRE(p->block_size == 16, QA_ERR_UNSUPPORTED, "block_size %d != 16", p->block_size);
  QA_REQUIRE(p->num_seqs <= 65535 && p->num_q_heads <= 65535, QA_ERR_UNSUPPORTED, "grid too large");
  return QA_OK;
}

qa_status_t check_prefill_ptrs(const qa_prefill_params_t* p, const int8_t* q_i8, const float* q_scale,
                               const int32_t* cu_seqlens_q, const int32_t* context_lens, const int8_t* k_cache,
                               const float* k_scale, const void* v_cache, const float* v_scale,
                               const int32_t* block_tables, const void* out) {
  QA_REQUIRE(q_i8 && q_scale && cu_seqlens_q && context_lens && k_cache && k_scale && v_cache && block_tables && out,
             QA_ERR_INVALID_ARG, "null pointer");
  QA_REQUIRE(p->v_cache_dtype != QA_DT_I8 || v_scale != nullptr, QA_ERR_INVALID_ARG, "INT8 V needs v_scale");
  QA_REQUIRE(aligned16(q_i8) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out), QA_ERR_INVALID_ARG,
             "q_i8, caches and out must be 16-byte aligned");
  QA_REQUIRE(p->v_cache_dtype != QA_DT_I8 || aligned16(v_scale), QA_ERR_INVALID_ARG,
             "v_scale must be 16-byte aligned");
  return QA_OK;
}

// FP8 P.V prefill workspace: E4M3 tiles [num_seqs, T, Hkv, 128 * head_dim]
// (T = ceil(16 * max_blocks_per_seq / 128)), channel scales [num_seqs, Hkv,
// head_dim] fp32, partial maxima [num_seqs, Hkv, kV8Parts, head_dim] fp32;
// each region starts on a 256-byte boundary.
struct PrefillFp8Layout {
  int32_t tiles;
  size_t v8, sv, part, total;
};

PrefillFp8Layout prefill_fp8_layout(const qa_prefill_params_t* p) {
  PrefillFp8Layout l{};
  l.tiles = (int32_t)(((int64_t)p->max_blocks_per_seq * 16 + 127) / 128);
  const size_t units = (size_t)p->num_seqs * (size_t)p->num_kv_heads;
  l.v8 = 0;
  l.sv = al(l.v8 + units * (size_t)l.tiles * 128 * (size_t)p->head_dim);
  l.part = al(l.sv + units * (size_t)p->head_dim * 4);
  l.total = al(l.part + units * (size_t)qa::kV8Parts * (size_t)p->head_dim * 4);
  return l;
}

}  // namespace

qa_status_t qa_chunked_prefill_attention(const qa_prefill_params_t* p, const int8_t* q_i8, const float* q_scale,
                                         const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                         const int8_t* k_cache, const float* k_scale, const void* v_cache,
                                         const float* v_scale, const int32_t* block_tables, void* out,
                                         qa_stream_t stream) {
  qa_status_t st = check_prefill(p);
  if (st != QA_OK) return st;
  if (p->num_seqs == 0 || p->total_q == 0) return QA_OK;
  st = check_prefill_ptrs(p, q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale,
                          block_tables, out);
  if (st != QA_OK) return st;
  qa::FlashArgs a{};
  a.q = q_i8; a.q_scale = q_scale; a.k_blocks = k_cache; a.k_scale = k_scale; a.v_blocks = v_cache;
  a.v_scale = v_scale; a.tables = block_tables; a.cu_q = cu_seqlens_q; a.ctx_lens = context_lens; a.out = out;
  a.num_seqs = p->num_seqs; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = p->num_q_heads / p->num_kv_heads;
  a.D = p->head_dim; a.max_blocks = p->max_blocks_per_seq; a.max_seqlen_q = p->max_seqlen_q;
  a.scale_log2 = log2_scale(p->softmax_scale, p->head_dim);
  a.dense = false; a.causal = true; a.v_int8 = p->v_cache_dtype == QA_DT_I8; a.v_f16 = false;
  a.out_bf16 = p->out_dtype == QA_DT_BF16; a.out_f16 = false;
  return hip_status(qa::launch_flash(a, (hipStream_t)stream), "qa_chunked_prefill_attention launch");
}

size_t qa_chunked_prefill_ws_workspace_bytes(const qa_prefill_params_t* p) {
  if (check_prefill(p) != QA_OK) return 0;
  return (size_t)p->num_seqs * (size_t)p->max_blocks_per_seq * (size_t)p->num_kv_heads * (size_t)p->head_dim * 32;
}

qa_status_t qa_chunked_prefill_attention_ws(const qa_prefill_params_t* p, const int8_t* q_i8, const float* q_scale,
                                            const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                            const int8_t* k_cache, const float* k_scale, const void* v_cache,
                                            const float* v_scale, const int32_t* block_tables, void* workspace,
                                            size_t workspace_bytes, void* out, qa_stream_t stream) {
  qa_status_t st = check_prefill(p);
  if (st != QA_OK) return st;
  if (p->num_seqs == 0 || p->total_q == 0) return QA_OK;
  st = check_prefill_ptrs(p, q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale,
                          block_tables, out);
  if (st != QA_OK) return st;
  const size_t need = qa_chunked_prefill_ws_workspace_bytes(p);
  QA_REQUIRE(workspace != nullptr && aligned16(workspace), QA_ERR_INVALID_ARG,
             "workspace must be a 16-byte aligned device pointer");
  QA_REQUIRE(workspace_bytes >= need, QA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu",
             workspace_bytes, need);
  qa::FlashArgs a{};
  a.q = q_i8; a.q_scale = q_scale; a.k_blocks = k_cache; a.k_scale = k_scale; a.v_blocks = v_cache;
  a.v_scale = v_scale; a.tables = block_tables; a.cu_q = cu_seqlens_q; a.ctx_lens = context_lens; a.out = out;
  a.num_seqs = p->num_seqs; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = p->num_q_heads / p->num_kv_heads;
  a.D = p->head_dim; a.max_blocks = p->max_blocks_per_seq; a.max_seqlen_q = p->max_seqlen_q;
  a.scale_log2 = log2_scale(p->softmax_scale, p->head_dim);
  a.dense = false; a.causal = true; a.v_int8 = p->v_cache_dtype == QA_DT_I8; a.v_f16 = false;
  a.out_bf16 = p->out_dtype == QA_DT_BF16; a.out_f16 = false;
  a.v_ws = workspace;
  return hip_status(qa::launch_flash(a, (hipStream_t)stream), "qa_chunked_prefill_attention_ws launch");
}

size_t qa_chunked_prefill_fp8pv_workspace_bytes(const qa_prefill_params_t* p) {
  if (check_prefill(p) != QA_OK) return 0;
  return prefill_fp8_layout(p).total;
}

qa_status_t qa_chunked_prefill_attention_fp8pv(const qa_prefill_params_t* p, const int8_t* q_i8,
                                               const float* q_scale, const int32_t* cu_seqlens_q,
                                               const int32_t* context_lens, const int8_t* k_cache,
                                               const float* k_scale, const void* v_cache, const float* v_scale,
                                               const int32_t* block_tables, void* workspace,
                                               size_t workspace_bytes, void* out, qa_stream_t stream) {
  qa_status_t st = check_prefill(p);
  if (st != QA_OK) return st;
  if (p->num_seqs == 0 || p->total_q == 0) return QA_OK;
  st = check_prefill_ptrs(p, q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale,
                          block_tables, out);
  if (st != QA_OK) return st;
  const PrefillFp8Layout l = prefill_fp8_layout(p);
  QA_REQUIRE(workspace != nullptr && aligned16(workspace), QA_ERR_INVALID_ARG,
             "workspace must be a 16-byte aligned device pointer");
  QA_REQUIRE(workspace_bytes >= l.total, QA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu",
             workspace_bytes, l.total);
  char* ws = static_cast<char*>(workspace);
  qa::PrefillFp8Args a{};
  a.q = q_i8; a.q_scale = q_scale; a.k_blocks = k_cache; a.k_scale = k_scale; a.v_cache = v_cache;
  a.v_scale = v_scale; a.tables = block_tables; a.cu_q = cu_seqlens_q; a.ctx_lens = context_lens; a.out = out;
  a.v8 = reinterpret_cast<uint8_t*>(ws + l.v8); a.v8_scale = reinterpret_cast<float*>(ws + l.sv);
  a.partial = reinterpret_cast<float*>(ws + l.part);
  a.num_seqs = p->num_seqs; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = p->num_q_heads / p->num_kv_heads;
  a.D = p->head_dim; a.max_blocks = p->max_blocks_per_seq; a.max_seqlen_q = p->max_seqlen_q;
  a.v8_seq_tiles = l.tiles;
  a.scale_log2 = log2_scale(p->softmax_scale, p->head_dim);
  a.v_int8 = p->v_cache_dtype == QA_DT_I8; a.out_bf16 = p->out_dtype == QA_DT_BF16;
  return hip_status(qa::launch_prefill_fp8(a, (hipStream_t)stream), "qa_chunked_prefill_attention_fp8pv launch");
}

size_t qa_dense_sage_quantize_workspace_size(const qa_dense_params_t* p) {
  if (check_dense(p) != QA_OK) return 0;
  return dense_layout(dense_call(p, QA_LAYOUT_NHD, false), false, false).total;
}

qa_status_t qa_dense_sage_quantize(const qa_dense_params_t* p, const void* q, const void* k, int8_t* q_i8,
                                   float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean, void* workspace,
                                   size_t workspace_bytes, qa_stream_t stream) {
  qa_status_t st = check_dense(p);
  if (st != QA_OK) return st;
  if (p->batch == 0 || (p->seq_q == 0 && p->seq_k == 0)) return QA_OK;
  QA_REQUIRE(q && k && q_i8 && q_scale && k_i8 && k_scale && k_mean && workspace, QA_ERR_INVALID_ARG,
             "null pointer");
  QA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(workspace) && ((uintptr_t)q_i8 & 7u) == 0 &&
                 ((uintptr_t)k_i8 & 7u) == 0,
             QA_ERR_INVALID_ARG, "q, k, workspace must be 16-byte aligned and codes 8-byte aligned");
  const DenseCall c = dense_call(p, QA_LAYOUT_NHD, false);
  const DenseWs w = dense_layout(c, false, false);
  QA_REQUIRE(workspace_bytes >= w.total, QA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
             workspace_bytes, w.total);
  qa::SagePrepArgs a{};
  a.q_rows = c.q; a.k_rows = c.k;
  a.q = q; a.k = k; a.v = nullptr; a.bf16 = p->dtype == QA_DT_BF16;
  a.B = p->batch; a.Nq = p->seq_q; a.Nk = p->seq_k; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.D = p->head_dim; a.smooth_k = p->smooth_k != 0;
  a.q_sb = c.sq.b; a.q_st = c.sq.t; a.q_sh = c.sq.h;
  a.k_sb = c.sk.b; a.k_st = c.sk.t; a.k_sh = c.sk.h;
  a.q_i8 = q_i8; a.q_scale = q_scale; a.k_i8 = k_i8; a.k_paged = nullptr; a.k_scale = k_scale;
  a.k_mean = k_mean; a.partial = (double*)((char*)workspace + w.partial); a.v_paged = nullptr;
  return hip_status(qa::launch_sage_prep(a, (hipStream_t)stream), "qa_dense_sage_quantize launch");
}

size_t qa_dense_sage_workspace_bytes(const qa_dense_params_t* p) {
  if (check_dense(p) != QA_OK) return 0;
  return dense_layout(dense_call(p, QA_LAYOUT_NHD, false), true, false).total;
}

size_t qa_dense_sage_workspace_size(const qa_dense_params_t* p) { return qa_dense_sage_workspace_bytes(p); }

qa_status_t qa_dense_sage_attention(const qa_dense_params_t* p, const void* q, const void* k, const void* v,
                                    void* workspace, size_t workspace_bytes, void* out, qa_stream_t stream) {
  return dense_attention_impl(p, nullptr, q, k, v, workspace, workspace_bytes, out, nullptr, stream, false);
}

size_t qa_dense_sage_ex_workspace_size(const qa_dense_params_t* p, const qa_dense_options_t* options) {
  if (check_dense(p) != QA_OK) return 0;
  const bool fp8 = options != nullptr && options->pv_fp8 != 0;
  return dense_layout(dense_call(p, QA_LAYOUT_NHD, false, fp8), true, true).total;
}

qa_status_t qa_dense_sage_attention_ex(const qa_dense_params_t* p, const qa_dense_options_t* options,
                                       const void* q, const void* k, const void* v, void* workspace,
                                       size_t workspace_bytes, void* out, float* lse, qa_stream_t stream) {
  return dense_attention_impl(p, options, q, k, v, workspace, workspace_bytes, out, lse, stream, true);
}

size_t qa_dense_sage_varlen_workspace_size(const qa_varlen_params_t* p) {
  if (check_varlen(p) != QA_OK) return 0;
  return dense_layout(varlen_call(p, nullptr, nullptr), true, true).total;
}

qa_status_t qa_dense_sage_attention_varlen(const qa_varlen_params_t* p, const void* q, const void* k,
                                           const void* v, const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, void* workspace,
                                           size_t workspace_bytes, void* out, float* lse,
                                           qa_stream_t stream) {
  qa_status_t st = check_varlen(p);
  if (st != QA_OK) return st;
  if (p->batch == 0 || p->total_q == 0 || p->max_seqlen_q == 0) return QA_OK;
  QA_REQUIRE(q && k && v && out && workspace && cu_seqlens_q && cu_seqlens_k, QA_ERR_INVALID_ARG,
             "null pointer");
  QA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(workspace),
             QA_ERR_INVALID_ARG, "q, k, v, out and workspace must be 16-byte aligned");
  QA_REQUIRE(((uintptr_t)lse & 3u) == 0 && ((uintptr_t)cu_seqlens_q & 3u) == 0 &&
                 ((uintptr_t)cu_seqlens_k & 3u) == 0,
             QA_ERR_INVALID_ARG, "lse and cu_seqlens must be 4-byte aligned");
  const DenseCall c = varlen_call(p, cu_seqlens_q, cu_seqlens_k);
  const DenseWs w = dense_layout(c, true, true);
  QA_REQUIRE(workspace_bytes >= w.total, QA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
             workspace_bytes, w.total);
  return run_dense(c, q, k, v, (char*)workspace, w, out, lse, stream);
}

}  // extern "C"
