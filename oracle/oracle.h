/*
 * oracle.h - C interface of the CPU oracle for INT8-QK quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow definition of what the
 * GPU library computes; only the test suite, the smoke check of the build
 * harness and the CPU-baseline leg of the benchmark load it. It shares no
 * code with the GPU library (no common headers, helpers or tables).
 *
 * Sources (cited by title and section):
 *   [QK-MMAC]   "gfx936 DCU上实现INT8 QK MMAC：分页访存、Fragment映射与GQA适配"
 *               (INT8 QK MMAC on the gfx936 DCU: paged access, fragment mapping
 *               and GQA adaptation).
 *   [SAGE-MACA] "SageAttention — MetaX MXMACA 平台移植版 (v3.0.0)" README.
 *
 * Conventions: every array is host memory, C order, owned by the caller;
 * outputs are fully written by the call (entries a call does not compute are
 * set to zero, or -inf for log-sum-exp values). 16-bit inputs are passed as
 * their storage bits with a dtype code. Functions parallelize with OpenMP
 * over independent units only; each unit is computed sequentially, so the
 * results do not depend on the thread count.
 */
#ifndef QA_ORACLE_H
#define QA_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_BF16 = 0, OR_F16 = 1 };

/* ---- storage formats ----------------------------------------------------- */
void or_widen(const uint16_t* bits, int32_t dtype, int64_t n, float* out);
void or_f32_to_f16_bits(const float* x, int64_t n, uint16_t* out);
void or_e4m3_encode(const double* x, int64_t n, uint8_t* out);
void or_e4m3_decode(const uint8_t* codes, int64_t n, double* out);

/* ---- quantization and the paged cache ([QK-MMAC] §1, §2.1, §3, §4) ------ */
void or_quant_rows(const float* x, int64_t rows, int64_t n, int8_t* q, float* s);
void or_write_kv(const float* k, const uint16_t* v_bits, int32_t v_dtype, int32_t v_int8,
                 const int64_t* slots, int64_t T, int32_t H, int32_t d, int8_t* k_cache, float* k_scale,
                 void* v_cache, float* v_scale);
void or_gather_kv(const int8_t* k_cache, const float* k_scale, const void* v_cache, const float* v_scale,
                  int32_t v_dtype, int32_t H, int32_t d, const int32_t* table_row, int32_t ctx, int32_t kvh,
                  int8_t* kq, float* sk, double* v);
void or_apply_rope(const uint16_t* x_bits, int32_t dtype, int64_t T, int32_t H, int32_t d, const int64_t* pos,
                   const float* cos_sin, int32_t rot, int32_t neox, float* out);

/* ---- paged attention ([QK-MMAC] §1-§5) ----------------------------------- */
typedef struct {
  const int8_t* k_cache;   /* [NB, Hkv, d/16, 16, 16] */
  const float* k_scale;    /* [NB, Hkv, 16] */
  const void* v_cache;     /* [NB, Hkv, d, 16] 16-bit bits or int8 */
  const float* v_scale;    /* [NB, Hkv, 16] for int8 V, else NULL */
  int32_t v_dtype;         /* OR_BF16 / OR_F16 for 16-bit V */
  const int32_t* tables;   /* [num_seqs, max_blocks] */
  int32_t max_blocks;
  int32_t num_seqs, Hq, Hkv, d;
} or_paged_t;

void or_paged_qk_int32(const or_paged_t* c, const int8_t* q_i8, const int32_t* ctx, int64_t* acc);
void or_paged_decode(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* ctx,
                     double scale, const uint8_t* head_mask, double* out);
void or_split_segments(int32_t ctx, int32_t num_splits, int32_t* bounds /* [num_splits][2] */);
void or_paged_decode_split(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* ctx,
                           double scale, int32_t num_splits, double* out);
void or_chunked_prefill(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* cu_q,
                        const int32_t* ctx, int64_t total_q, double scale, const uint8_t* row_mask,
                        const uint8_t* head_mask, double* out);
void or_attention_fp64(const double* q, const double* k, const double* v, int64_t nq, int64_t nk, int32_t d,
                       double scale, const uint8_t* visible, double* out);
/* chunked prefill with the P.V product in FP8 (E4M3): the V scales and codes of
   one (sequence, KV head), codes [ctx, d] and scales [d]; the attention with
   its tolerance model (sigma may be NULL) */
void or_paged_v_fp8(const or_paged_t* c, int32_t seq, int32_t ctx, int32_t kvh, uint8_t* codes, float* scales);
void or_chunked_prefill_fp8pv(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* cu_q,
                              const int32_t* ctx, int64_t total_q, double scale, const uint8_t* row_mask,
                              const uint8_t* head_mask, double* out, double* sigma);

/* threads of the parallel loops (for timing the oracle) */
void or_set_num_threads(int32_t n);
int32_t or_max_threads(void);

/* ---- dense SageAttention-style path ([SAGE-MACA]) ------------------------ */
typedef struct {
  int32_t B, Nq, Nk, Hq, Hkv, d;
  int32_t q_block, k_block;
} or_dense_t;

void or_sage_quantize(const or_dense_t* g, const uint16_t* q_bits, const uint16_t* k_bits, int32_t dtype,
                      int32_t smooth_k, int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean);
void or_dense_attention(const or_dense_t* g, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                        const float* k_scale, const double* v, int32_t causal, double scale, const int64_t* rows,
                        int64_t nrows, const uint8_t* head_mask, const uint8_t* batch_mask, double* out,
                        double* lse);
void or_sage_smooth_v(const uint16_t* v_bits, int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t d,
                      uint16_t* vp_f16, float* mu);
void or_sage_lse_correction(const uint16_t* q_bits, int32_t dtype, const float* k_mean, int32_t B, int32_t Nq,
                            int32_t Hq, int32_t Hkv, int32_t d, double scale, double* corr);
void or_sage_forward(const or_dense_t* g, const uint16_t* q_bits, const uint16_t* k_bits, const uint16_t* v_bits,
                     int32_t dtype, int32_t causal, int32_t smooth_k, int32_t smooth_v, double scale, double* out,
                     double* lse);
void or_sage_varlen_forward(const uint16_t* q_bits, const uint16_t* k_bits, const uint16_t* v_bits, int32_t dtype,
                            const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                            int32_t causal, int32_t smooth_k, int32_t smooth_v, double scale, double* out,
                            double* lse);

/* ---- FP8 (E4M3) P.V ------------------------------------------------------ */
void or_v_fp8_per_channel(const float* v, int32_t B, int32_t N, int32_t H, int32_t d, double* vals, float* s);
void or_dense_attention_fp8pv(const or_dense_t* g, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                              const float* k_scale, const float* v, int32_t causal, double scale, int32_t smooth_v,
                              const int64_t* rows, int64_t nrows, const uint8_t* head_mask, double* out,
                              double* lse, double* sigma, double* sigma_lse);
void or_dense_attention_fp8pv_lazy(const or_dense_t* g, const int8_t* q_i8, const float* q_scale,
                                   const int8_t* k_i8, const float* k_scale, const float* v, int32_t causal,
                                   double scale, int32_t smooth_v, int32_t tile, double slack, int32_t group,
                                   double* out, double* lse);

#ifdef __cplusplus
}
#endif

#endif /* QA_ORACLE_H */
