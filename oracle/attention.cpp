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

// Keys seen by row r of a chunk of tq new tokens at the end of a context of
// n tokens: the row sits at position n - tq + r and sees keys t <= that
// position; a row placed before the first key sees none.
int32_t chunk_visible_keys(int32_t n, int32_t tq, int32_t r) {
  const int64_t pos = (int64_t)n - tq + r;
  if (pos < 0) return 0;
  return (int32_t)std::min<int64_t>(pos + 1, n);
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
        const int32_t nvis = chunk_visible_keys(n, tq, i - a);
        if (nvis == 0) continue;
        const int64_t row = (int64_t)i * c->Hq + h;
        scores_row(q_i8 + row * d, q_scale[row], g, nvis, d, sc, sr.data());
        softmax_pv(sr.data(), nvis, g.v.data(), d, d, out + row * d);
      }
    }
  }
}

// ---- chunked prefill with the P.V product in FP8 (E4M3) -----------------------
// [SAGE-MACA] names the FP8 P.V product of later SageAttention versions (not
// portable to its hardware); the pages fix none of its arithmetic. Reading:
// the dense FP8 definition (or_dense_attention_fp8pv) applied to a paged
// sequence. V of a (sequence, KV head) is taken over all ctx cached tokens as
// fp32 values (16-bit V exactly, INT8 V as fl32(code * scale)); per channel
// s_c = fl32(max_t |v| / 448) and V8 = E4M3(fl32(v / s_c)), 0 where s_c = 0.
// Per query row, m = the exact maximum of its visible scores,
// P8_j = E4M3(448 exp(s_j - m)) and out = sum_j P8_j V8_j / sum_j P8_j * s_c.
// Sums and products in fp64.

// E4M3 values and channel scales of the first ctx V tokens of one (sequence,
// KV head): codes [ctx, d], scales [d].
void or_paged_v_fp8(const or_paged_t* c, int32_t seq, int32_t ctx, int32_t kvh, uint8_t* codes, float* scales) {
  const int32_t d = c->d;
  const Gathered g = gather(c, seq, ctx, kvh);
  std::vector<float> v((size_t)ctx * d);
  for (size_t i = 0; i < v.size(); ++i) v[i] = (float)g.v[i];   // fl32(code * scale) for INT8 V
  for (int32_t ch = 0; ch < d; ++ch) {
    float amax = 0.0f;
    for (int32_t t = 0; t < ctx; ++t) amax = std::max(amax, std::fabs(v[(int64_t)t * d + ch]));
    const float sc = amax / 448.0f;
    scales[ch] = sc;
    for (int32_t t = 0; t < ctx; ++t)
      codes[(int64_t)t * d + ch] = sc > 0.0f ? e4m3_encode1((double)(v[(int64_t)t * d + ch] / sc)) : 0;
  }
}

// The definition above for the rows of or_chunked_prefill (row_mask,
// head_mask, out the same). sigma (NULL = not computed) [total_q, Hq, d]:
// the standard deviation of an implementation that rounds P from a lazily
// moved reference, as in or_dense_attention_fp8pv (its model and bounds).
void or_chunked_prefill_fp8pv(const or_paged_t* c, const int8_t* q_i8, const float* q_scale, const int32_t* cu_q,
                              const int32_t* ctx, int64_t total_q, double scale, const uint8_t* row_mask,
                              const uint8_t* head_mask, double* out, double* sigma) {
  const int32_t G = c->Hq / c->Hkv, d = c->d;
  const double sc = resolve_scale(scale, d);
  const double u = std::ldexp(1.0, -4), sub = std::ldexp(1.0, -6), sub_err = std::ldexp(1.0, -10);
  std::fill(out, out + total_q * c->Hq * d, 0.0);
  if (sigma != nullptr) std::fill(sigma, sigma + total_q * c->Hq * d, 0.0);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t s = 0; s < c->num_seqs; ++s) {
    for (int32_t h = 0; h < c->Hq; ++h) {
      const int32_t a = cu_q[s], b = cu_q[s + 1], n = ctx[s], tq = b - a;
      if (n <= 0 || tq <= 0 || (head_mask != nullptr && !head_mask[h])) continue;
      bool any = row_mask == nullptr;
      for (int32_t i = a; i < b && !any; ++i) any = row_mask[i] != 0;
      if (!any) continue;
      const Gathered g = gather(c, s, n, h / G);
      std::vector<uint8_t> codes((size_t)n * d);
      std::vector<float> svc(d);
      or_paged_v_fp8(c, s, n, h / G, codes.data(), svc.data());
      std::vector<double> v8((size_t)n * d);
      for (size_t i = 0; i < v8.size(); ++i) v8[i] = e4m3_decode1(codes[i]);
      std::vector<double> sr(n), p(n), p8(n), o(d), oe(d);
      for (int32_t i = a; i < b; ++i) {
        if (row_mask != nullptr && !row_mask[i]) continue;
        const int32_t nvis = chunk_visible_keys(n, tq, i - a);
        if (nvis == 0) continue;
        const int64_t row = (int64_t)i * c->Hq + h;
        scores_row(q_i8 + row * d, q_scale[row], g, nvis, d, sc, sr.data());
        double m = -kInf;
        for (int32_t j = 0; j < nvis; ++j) m = std::max(m, sr[j]);
        double l8 = 0.0, lp = 0.0;
        for (int32_t j = 0; j < nvis; ++j) {
          p[j] = std::exp(sr[j] - m);
          p8[j] = p[j] > 0.0 ? e4m3_decode1(e4m3_encode1(448.0 * p[j])) : 0.0;
          l8 += p8[j];
          lp += p[j];
        }
        std::fill(o.begin(), o.end(), 0.0);
        std::fill(oe.begin(), oe.end(), 0.0);
        for (int32_t j = 0; j < nvis; ++j) {
          const double* vj = v8.data() + (int64_t)j * d;
          for (int32_t ch = 0; ch < d; ++ch) {
            o[ch] += p8[j] * vj[ch];
            oe[ch] += p[j] * vj[ch];
          }
        }
        for (int32_t ch = 0; ch < d; ++ch) out[row * d + ch] = o[ch] / l8 * (double)svc[ch];
        if (sigma != nullptr) {
          std::vector<double> var(d, 0.0);
          for (int32_t j = 0; j < nvis; ++j) {
            if (p[j] == 0.0) continue;
            const double w = p[j] / lp;
            const double e56 = 56.0 * p[j] >= sub ? u * w : sub_err / (56.0 * lp);
            const double e448 = 448.0 * p[j] >= sub ? u * w : sub_err / (448.0 * lp);
            const double ee = e56 * e56 + e448 * e448;
            const double* vj = v8.data() + (int64_t)j * d;
            for (int32_t ch = 0; ch < d; ++ch) {
              const double dv = (vj[ch] - oe[ch] / lp) * (double)svc[ch];
              var[ch] += dv * dv * ee;
            }
          }
          for (int32_t ch = 0; ch < d; ++ch) sigma[row * d + ch] = std::sqrt(var[ch] / 3.0);
        }
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
