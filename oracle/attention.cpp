// Oracle: paged INT8-QK attention (decode, split-K, chunked prefill) and
// textbook fp64 attention. TEST INFRASTRUCTURE ONLY (see oracle.h).
//
// [QK-MMAC] §1: the INT32 accumulator acc = sum_i Qq[i] * Kq[i] is rescaled
// per element, score = acc * sQ(query token, query head) * sK(key token, KV
// head) * softmax_scale, before the softmax. §2.1: codes lie in [-127, 127],
// so |acc| <= 256 * 127 * 127 = 4,129,024 and int32 holds it exactly. §3:
// K is read through the block table. §5.2: query head h reads KV head
// h / G. The pages fix no precision after the accumulator: here score
// recovery, softmax (two passes) and P.V are fp64.
#include <omp.h>

#include <algorithm>

#include "impl.h"

namespace orc {

double softmax_pv(const double* s, int64_t n, const double* v, int64_t ld, int32_t d, double* out) {
  double m = -kInf;
  for (int64_t j = 0; j < n; ++j) m = std::max(m, s[j]);
  for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
  if (!(m > -kInf)) return m;                    // no visible key: zeros
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double p = std::exp(s[j] - m);         // masked keys: exp(-inf) = 0
    if (p == 0.0) continue;
    l += p;
    const double* vj = v + j * ld;
    for (int32_t c = 0; c < d; ++c) out[c] += p * vj[c];
  }
  for (int32_t c = 0; c < d; ++c) out[c] /= l;
  return m;
}

double logsumexp(const double* s, int64_t n) {
  double m = -kInf;
  for (int64_t j = 0; j < n; ++j) m = std::max(m, s[j]);
  if (!(m > -kInf)) return -kInf;
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += std::exp(s[j] - m);
  return m + std::log(l);
}

namespace {

// The first ctx tokens of one (sequence, KV head), gathered through the table.
struct Gathered {
  std::vector<int8_t> kq;
  std::vector<float> sk;
  std::vector<double> v;
};

Gathered gather(const or_paged_t* c, int32_t seq, int32_t ctx, int32_t kvh) {
  Gathered g;
  g.kq.resize((size_t)ctx * c->d);
  g.sk.resize(ctx);
  g.v.resize((size_t)ctx * c->d);
  or_gather_kv(c->k_cache, c->k_scale, c->v_cache, c->v_scale, c->v_dtype, c->Hkv, c->d,
               c->tables + (int64_t)seq * c->max_blocks, ctx, kvh, g.kq.data(), g.sk.data(), g.v.data());
  return g;
}

int32_t int_dot(const int8_t* a, const int8_t* b, int32_t d) {
  int32_t acc = 0;
  for (int32_t i = 0; i < d; ++i) acc += (int32_t)a[i] * (int32_t)b[i];
  return acc;
}

// [QK-MMAC] §1: the recovered score of every key for one query row.
void scores_row(const int8_t* q, float q_scale, const Gathered& g, int32_t n, int32_t d, double scale,
                double* s) {
  for (int32_t t = 0; t < n; ++t)
    s[t] = (double)int_dot(q, g.kq.data() + (int64_t)t * d, d) * (double)q_scale * (double)g.sk[t] * scale;
}

}  // namespace
}  // namespace orc

using namespace orc;

extern "C" {

// INT32 accumulators of decode, one query token per sequence: acc[h][t] for
// t < ctx, sequences packed one after another (sequence s starts at
// sum_{r<s} Hq * ctx[r]).
void or_paged_qk_int32(const or_paged_t* c, const int8_t* q_i8, const int32_t* ctx, int64_t* acc) {
  const int32_t G = c->Hq / c->Hkv, d = c->d;
  int64_t base = 0;
  for (int32_t s = 0; s < c->num_seqs; ++s) {
    for (int32_t kvh = 0; kvh < c->Hkv; ++kvh) {
      const Gathered g = gather(c, s, ctx[s], kvh);
      for (int32_t h = kvh * G; h < (kvh + 1) * G; ++h)
        for (int32_t t = 0; t < ctx[s]; ++t)
          acc[base + (int64_t)h * ctx[s] + t] =
              int_dot(q_i8 + ((int64_t)s * c->Hq + h) * d, g.kq.data() + (int64_t)t * d, d);
    }
    base += (int64_t)c->Hq * ctx[s];
  }
}

// Decode attention, one query token per sequence, keys t < ctx visible; a
// sequence with ctx == 0 gives zeros. head_mask (NULL = all) selects the
// query heads computed; the others are zero. out [num_seqs, Hq, d].
void or_paged_decode(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* ctx,
                     double scale, const uint8_t* head_mask, double* out) {
  const int32_t G = c->Hq / c->Hkv, d = c->d;
  const double sc = resolve_scale(scale, d);
  std::fill(out, out + (int64_t)c->num_seqs * c->Hq * d, 0.0);
  // one unit per (sequence, query head); each reads its KV head h / G
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t s = 0; s < c->num_seqs; ++s) {
    for (int32_t h = 0; h < c->Hq; ++h) {
      if (ctx[s] <= 0 || (head_mask != nullptr && !head_mask[h])) continue;
      const Gathered g = gather(c, s, ctx[s], h / G);
      std::vector<double> sr(ctx[s]);
      const int64_t row = (int64_t)s * c->Hq + h;
      scores_row(q_i8 + row * d, q_scale[row], g, ctx[s], d, sc, sr.data());
      softmax_pv(sr.data(), ctx[s], g.v.data(), d, d, out + row * d);
    }
  }
}

// [QK-MMAC] §4 cuts long decode contexts into segments without fixing the
// cut. Reading: L = 16 * ceil(ceil(ctx / 16) / S) tokens per segment (whole
// blocks); segment j covers [jL, min((j+1)L, ctx)), possibly empty.
void or_split_segments(int32_t ctx, int32_t num_splits, int32_t* bounds) {
  const int32_t nblk = (ctx + kBlock - 1) / kBlock;
  const int32_t L = kBlock * std::max((nblk + num_splits - 1) / num_splits, 1);
  for (int32_t j = 0; j < num_splits; ++j) {
    bounds[2 * j] = std::min(j * L, ctx);
    bounds[2 * j + 1] = std::min((j + 1) * L, ctx);
  }
}

// Split-K decode then the merge ([QK-MMAC] §4), for checking the merge
// algebra against the unsplit result. Segment j (or_split_segments) yields
// (m_j, l_j, O_j) = (max score, sum exp(s - m_j), sum exp(s - m_j) v); an empty segment
// yields (-inf, 0, 0). Merge: M = max m_j, w_j = exp(m_j - M),
// O = sum w_j O_j / sum w_j l_j.
void or_paged_decode_split(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* ctx,
                           double scale, int32_t num_splits, double* out) {
  const int32_t G = c->Hq / c->Hkv, d = c->d;
  const double sc = resolve_scale(scale, d);
  std::fill(out, out + (int64_t)c->num_seqs * c->Hq * d, 0.0);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t s = 0; s < c->num_seqs; ++s) {
    for (int32_t h = 0; h < c->Hq; ++h) {
      const int32_t n = ctx[s];
      if (n <= 0) continue;
      const Gathered g = gather(c, s, n, h / G);
      std::vector<int32_t> seg(2 * num_splits);
      or_split_segments(n, num_splits, seg.data());
      std::vector<double> sr(n), m(num_splits), l(num_splits), O((size_t)num_splits * d);
      const int64_t row = (int64_t)s * c->Hq + h;
      scores_row(q_i8 + row * d, q_scale[row], g, n, d, sc, sr.data());
      double M = -kInf;
      for (int32_t j = 0; j < num_splits; ++j) {
        const int32_t a = seg[2 * j], b = seg[2 * j + 1];
        double mj = -kInf;
        for (int32_t t = a; t < b; ++t) mj = std::max(mj, sr[t]);
        double lj = 0.0;
        double* oj = O.data() + (int64_t)j * d;
        for (int32_t ch = 0; ch < d; ++ch) oj[ch] = 0.0;
        for (int32_t t = a; t < b; ++t) {
          const double p = std::exp(sr[t] - mj);
          lj += p;
          for (int32_t ch = 0; ch < d; ++ch) oj[ch] += p * g.v[(int64_t)t * d + ch];
        }
        m[j] = mj;
        l[j] = lj;
        M = std::max(M, mj);
      }
      double den = 0.0;
      double* o = out + row * d;
      for (int32_t j = 0; j < num_splits; ++j) {
        const double w = std::exp(m[j] - M);
        den += w * l[j];
        for (int32_t ch = 0; ch < d; ++ch) o[ch] += w * O[(int64_t)j * d + ch];
      }
      for (int32_t ch = 0; ch < d; ++ch) o[ch] /= den;
    }
  }
}

// Chunked prefill over a paged history ([QK-MMAC] §5.2). Sequence s has
// Tq = cu_q[s+1] - cu_q[s] new query tokens, the last Tq of its ctx cached
// tokens: query i of the chunk sits at position ctx - Tq + i and sees keys
// t <= that position (history first, then causal within the chunk).
// row_mask [total_q] and head_mask [Hq] (NULL = all) select the outputs
// computed; the others are zero. out [total_q, Hq, d].
void or_chunked_prefill(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* cu_q,
                        const int32_t* ctx, int64_t total_q, double scale, const uint8_t* row_mask,
                        const uint8_t* head_mask, double* out) {
  const int32_t G = c->Hq / c->Hkv, d = c->d;
  const double sc = resolve_scale(scale, d);
  std::fill(out, out + total_q * c->Hq * d, 0.0);
  // one unit per (sequence, query head); each reads its KV head h / G
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t s = 0; s < c->num_seqs; ++s) {
    for (int32_t h = 0; h < c->Hq; ++h) {
      const int32_t a = cu_q[s], b = cu_q[s + 1], n = ctx[s], tq = b - a;
      if (n <= 0 || tq <= 0 || (head_mask != nullptr && !head_mask[h])) continue;
      bool any = row_mask == nullptr;
      for (int32_t i = a; i < b && !any; ++i) any = row_mask[i] != 0;
      if (!any) continue;
      const Gathered g = gather(c, s, n, h / G);
      std::vector<double> sr(n);
      for (int32_t i = a; i < b; ++i) {
        if (row_mask != nullptr && !row_mask[i]) continue;
        const int64_t pos = (int64_t)n - tq + (i - a);
        if (pos < 0) continue;                   // a token placed before the first key sees none
        const int32_t nvis = (int32_t)std::min<int64_t>(pos + 1, n);
        const int64_t row = (int64_t)i * c->Hq + h;
        scores_row(q_i8 + row * d, q_scale[row], g, nvis, d, sc, sr.data());
        softmax_pv(sr.data(), nvis, g.v.data(), d, d, out + row * d);
      }
    }
  }
}

// Textbook softmax(q k^T * scale) v in fp64 for [n, d] operands, with an
// optional visibility mask [nq, nk] (nonzero = visible). Used for pins and
// for the error of the quantized method against unquantized attention.
void or_attention_fp64(const double* q, const double* k, const double* v, int64_t nq, int64_t nk, int32_t d,
                       double scale, const uint8_t* visible, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nq; ++i) {
    std::vector<double> s(nk);
    for (int64_t j = 0; j < nk; ++j) {
      double acc = 0.0;
      for (int32_t c = 0; c < d; ++c) acc += q[i * d + c] * k[j * d + c];
      s[j] = (visible == nullptr || visible[i * nk + j]) ? acc * scale : -kInf;
    }
    softmax_pv(s.data(), nk, v, d, d, out + i * d);
  }
}

// Threads of the oracle's parallel loops (harness plumbing for timing it):
// or_set_num_threads(n) with n >= 1; or_max_threads() the current limit.
void or_set_num_threads(int32_t n) { omp_set_num_threads(n); }
int32_t or_max_threads(void) { return omp_get_max_threads(); }

}  // extern "C"
