// Oracle: SageAttention-style dense forward ([SAGE-MACA]) and its FP8 P.V
// variant. TEST INFRASTRUCTURE ONLY (see oracle.h).
//
// [SAGE-MACA] feature matrix and advanced options: smooth_k subtracts the
// per-channel mean of K over the tokens before quantization (with an LSE
// correction), smooth_v subtracts the V mean and adds it back to the output,
// return_lse gives the log-sum-exp of each row. Quantization-kernel table,
// "per_block" granularity: one scale per block of 128 query rows or 64 key
// rows of one (batch, head), over all rows x head_dim values of the block;
// the last block takes the remaining rows. Attention-kernel pipeline: INT8
// QK to INT32, scaled by the two block scales and the softmax scale, online
// softmax, fp16 P.V with fp32 accumulation; the causal mask covers the
// diagonal. Here the softmax and P.V after the INT32 accumulator are exact
// fp64 on the same recovered scores.
//
// Readings where the pages are silent (each listed with its reason in the
// design notes): the mean is a fp64 sum over all Nk tokens, divided by Nk in
// fp64 and rounded to fp32 (mu); K' = fl32(K - mu); V' = fl16(fl32(V) - mu_v);
// causal alignment is bottom-right (query i sees keys j <= i + Nk - Nq).
#include <algorithm>

#include "impl.h"

namespace orc {
namespace {

// fp32 values of a [count] array of 16-bit patterns.
std::vector<float> widen_all(const uint16_t* bits, int32_t dtype, int64_t count) {
  std::vector<float> v(count);
  for (int64_t i = 0; i < count; ++i) v[i] = widen1(bits[i], dtype);
  return v;
}

// mu[b][h][c] = fl32(sum_t x[b][t][h][c] / N), sum and quotient in fp64.
std::vector<float> channel_means(const float* x, int32_t B, int32_t N, int32_t H, int32_t d) {
  std::vector<float> mu((size_t)B * H * d, 0.0f);
  if (N == 0) return mu;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t h = 0; h < H; ++h)
      for (int32_t c = 0; c < d; ++c) {
        double sum = 0.0;
        for (int32_t t = 0; t < N; ++t) sum += (double)x[(((int64_t)b * N + t) * H + h) * d + c];
        mu[((int64_t)b * H + h) * d + c] = (float)(sum / (double)N);
      }
  return mu;
}

// Per-block INT8 of x [B, N, H, d]: block j of (b, h) holds rows
// [j*R, min((j+1)*R, N)); one scale per block over all its values.
void quant_blocks(const float* x, int32_t B, int32_t N, int32_t H, int32_t d, int32_t R, int8_t* codes,
                  float* scales) {
  const int32_t nb = (N + R - 1) / R;
#pragma omp parallel for collapse(3) schedule(static)
  for (int32_t b = 0; b < B; ++b)
    for (int32_t h = 0; h < H; ++h)
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t r0 = j * R, r1 = std::min(r0 + R, N);
        std::vector<float> blk((size_t)(r1 - r0) * d);
        std::vector<int8_t> q(blk.size());
        for (int32_t t = r0; t < r1; ++t)
          for (int32_t c = 0; c < d; ++c) blk[(size_t)(t - r0) * d + c] = x[(((int64_t)b * N + t) * H + h) * d + c];
        scales[((int64_t)b * H + h) * nb + j] = quant_row(blk.data(), (int64_t)blk.size(), q.data());
        for (int32_t t = r0; t < r1; ++t)
          for (int32_t c = 0; c < d; ++c) codes[(((int64_t)b * N + t) * H + h) * d + c] = q[(size_t)(t - r0) * d + c];
      }
}

int32_t int_dot(const int8_t* a, const int8_t* b, int32_t d) {
  int32_t acc = 0;
  for (int32_t i = 0; i < d; ++i) acc += (int32_t)a[i] * (int32_t)b[i];
  return acc;
}

// Recovered scores of query row i of (b, h) against every key, -inf where
// the causal mask hides the key. Returns the number of visible keys.
int32_t dense_scores(const or_dense_t* g, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, int32_t causal, double sc, int32_t b, int32_t h, int64_t i, double* s) {
  const int32_t G = g->Hq / g->Hkv, kvh = h / G, d = g->d;
  const int32_t nqb = (g->Nq + g->q_block - 1) / g->q_block, nkb = (g->Nk + g->k_block - 1) / g->k_block;
  const double qs = (double)q_scale[((int64_t)b * g->Hq + h) * nqb + i / g->q_block];
  const int8_t* qr = q_i8 + (((int64_t)b * g->Nq + i) * g->Hq + h) * d;
  const int64_t last = causal ? std::min<int64_t>(i + (g->Nk - g->Nq), (int64_t)g->Nk - 1) : (int64_t)g->Nk - 1;
  for (int32_t j = 0; j < g->Nk; ++j) {
    if (j > last) {
      s[j] = -kInf;
      continue;
    }
    const int32_t acc = int_dot(qr, k_i8 + (((int64_t)b * g->Nk + j) * g->Hkv + kvh) * d, d);
    s[j] = (double)acc * qs * (double)k_scale[((int64_t)b * g->Hkv + kvh) * nkb + j / g->k_block] * sc;
  }
  return (int32_t)std::max<int64_t>(last + 1, 0);
}

}  // namespace
}  // namespace orc

using namespace orc;

extern "C" {

// smooth_k (optional) and per-block INT8 of Q [B, Nq, Hq, d] and K' [B, Nk,
// Hkv, d]. Outputs: q_i8 and k_i8 in the input layout, q_scale [B, Hq,
// ceil(Nq/q_block)], k_scale [B, Hkv, ceil(Nk/k_block)], k_mean [B, Hkv, d]
// (zeros without smooth_k).
void or_sage_quantize(const or_dense_t* g, const uint16_t* q_bits, const uint16_t* k_bits, int32_t dtype,
                      int32_t smooth_k, int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean) {
  const int64_t nq = (int64_t)g->B * g->Nq * g->Hq * g->d, nk = (int64_t)g->B * g->Nk * g->Hkv * g->d;
  const std::vector<float> q = widen_all(q_bits, dtype, nq);
  std::vector<float> k = widen_all(k_bits, dtype, nk);
  std::vector<float> mu((size_t)g->B * g->Hkv * g->d, 0.0f);
  if (smooth_k) mu = channel_means(k.data(), g->B, g->Nk, g->Hkv, g->d);
  for (int32_t b = 0; b < g->B; ++b)
    for (int32_t t = 0; t < g->Nk; ++t)
      for (int32_t h = 0; h < g->Hkv; ++h)
        for (int32_t c = 0; c < g->d; ++c) {
          float& x = k[(((int64_t)b * g->Nk + t) * g->Hkv + h) * g->d + c];
          x = x - mu[((int64_t)b * g->Hkv + h) * g->d + c];       // fl32(K - mu)
        }
  std::copy(mu.begin(), mu.end(), k_mean);
  quant_blocks(q.data(), g->B, g->Nq, g->Hq, g->d, g->q_block, q_i8, q_scale);
  quant_blocks(k.data(), g->B, g->Nk, g->Hkv, g->d, g->k_block, k_i8, k_scale);
}

// Dense attention on pre-quantized inputs: score = acc * sQ_blk * sK_blk *
// scale, exact softmax and P.V in fp64 with v [B, Nk, Hkv, d] (fp64 values).
// rows (NULL = all Nq) lists the query rows computed; head_mask [Hq] and
// batch_mask [B] (NULL = all) select the rest. out [B, Nq, Hq, d] (rows not
// computed stay zero); lse [B, Hq, Nq] (optional; -inf where not computed or
// no key is visible): ln sum_j exp(score_j).
void or_dense_attention(const or_dense_t* g, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                        const float* k_scale, const double* v, int32_t causal, double scale, const int64_t* rows,
                        int64_t nrows, const uint8_t* head_mask, const uint8_t* batch_mask, double* out,
                        double* lse) {
  const int32_t G = g->Hq / g->Hkv, d = g->d;
  const double sc = resolve_scale(scale, d);
  const int64_t nr = rows != nullptr ? nrows : g->Nq;
  std::fill(out, out + (int64_t)g->B * g->Nq * g->Hq * d, 0.0);
  if (lse != nullptr) std::fill(lse, lse + (int64_t)g->B * g->Hq * g->Nq, -kInf);
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int32_t b = 0; b < g->B; ++b)
    for (int32_t h = 0; h < g->Hq; ++h)
      for (int64_t r = 0; r < nr; ++r) {
        if ((batch_mask != nullptr && !batch_mask[b]) || (head_mask != nullptr && !head_mask[h])) continue;
        const int64_t i = rows != nullptr ? rows[r] : r;
        std::vector<double> s(g->Nk);
        dense_scores(g, q_i8, q_scale, k_i8, k_scale, causal, sc, b, h, i, s.data());
        const double* vb = v + ((int64_t)b * g->Nk * g->Hkv + h / G) * d;
        softmax_pv(s.data(), g->Nk, vb, (int64_t)g->Hkv * d, d, out + (((int64_t)b * g->Nq + i) * g->Hq + h) * d);
        if (lse != nullptr) lse[((int64_t)b * g->Hq + h) * g->Nq + i] = logsumexp(s.data(), g->Nk);
      }
}

// smooth_v: mu_v = fl32(sum_t V / N) per (b, h, c) (fp64 sum and quotient)
// and V' = fl16(fl32(V) - mu_v), the fp16 operand of the P.V product. Since
// each softmax row sums to one, attention on V equals attention on V' plus
// mu_v up to the fp16 rounding of V'.
void or_sage_smooth_v(const uint16_t* v_bits, int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t d,
                      uint16_t* vp_f16, float* mu_out) {
  const int64_t n = (int64_t)B * N * H * d;
  std::vector<float> v = widen_all(v_bits, dtype, n);
  const std::vector<float> mu = channel_means(v.data(), B, N, H, d);
  for (int32_t b = 0; b < B; ++b)
    for (int32_t t = 0; t < N; ++t)
      for (int32_t h = 0; h < H; ++h)
        for (int32_t c = 0; c < d; ++c) {
          float& x = v[(((int64_t)b * N + t) * H + h) * d + c];
          x = x - mu[((int64_t)b * H + h) * d + c];
        }
  or_f32_to_f16_bits(v.data(), n, vp_f16);
  std::copy(mu.begin(), mu.end(), mu_out);
}

// smooth_k shifts every score of query row i by -scale * q_i . mu (K' = K -
// mu), so the LSE of the smoothed scores is corrected by adding it back
// ([SAGE-MACA] feature matrix, LSE correction):
// corr[b][h][i] = scale * sum_c q[b][i][h][c] * mu[b][h/G][c], unquantized q,
// in fp64.
void or_sage_lse_correction(const uint16_t* q_bits, int32_t dtype, const float* k_mean, int32_t B, int32_t Nq,
                            int32_t Hq, int32_t Hkv, int32_t d, double scale, double* corr) {
  const int32_t G = Hq / Hkv;
  const double sc = resolve_scale(scale, d);
  for (int32_t b = 0; b < B; ++b)
    for (int32_t h = 0; h < Hq; ++h)
      for (int32_t i = 0; i < Nq; ++i) {
        double acc = 0.0;
        for (int32_t c = 0; c < d; ++c)
          acc += (double)widen1(q_bits[(((int64_t)b * Nq + i) * Hq + h) * d + c], dtype) *
                 (double)k_mean[((int64_t)b * Hkv + h / G) * d + c];
        corr[((int64_t)b * Hq + h) * Nq + i] = acc * sc;
      }
}

// The whole dense call with its options ([SAGE-MACA] API: smooth_k,
// smooth_v, return_lse): quantize (smooth_k), optionally smooth V, attend,
// add the V mean back on rows that see a key, correct the LSE for the K
// mean. out [B, Nq, Hq, d]; lse [B, Hq, Nq] (optional).
void or_sage_forward(const or_dense_t* g, const uint16_t* q_bits, const uint16_t* k_bits, const uint16_t* v_bits,
                     int32_t dtype, int32_t causal, int32_t smooth_k, int32_t smooth_v, double scale, double* out,
                     double* lse) {
  const int32_t B = g->B, Nq = g->Nq, Nk = g->Nk, Hq = g->Hq, Hkv = g->Hkv, d = g->d, G = Hq / Hkv;
  const int32_t nqb = (Nq + g->q_block - 1) / g->q_block, nkb = (Nk + g->k_block - 1) / g->k_block;
  std::vector<int8_t> q_i8((size_t)B * Nq * Hq * d), k_i8((size_t)B * Nk * Hkv * d);
  std::vector<float> q_scale((size_t)B * Hq * nqb), k_scale((size_t)B * Hkv * nkb), k_mean((size_t)B * Hkv * d);
  or_sage_quantize(g, q_bits, k_bits, dtype, smooth_k, q_i8.data(), q_scale.data(), k_i8.data(), k_scale.data(),
                   k_mean.data());
  const int64_t nv = (int64_t)B * Nk * Hkv * d;
  std::vector<double> v(nv);
  std::vector<float> mu_v((size_t)B * Hkv * d, 0.0f);
  if (smooth_v) {
    std::vector<uint16_t> vp(nv);
    or_sage_smooth_v(v_bits, dtype, B, Nk, Hkv, d, vp.data(), mu_v.data());
    for (int64_t i = 0; i < nv; ++i) v[i] = (double)widen1(vp[i], OR_F16);
  } else {
    for (int64_t i = 0; i < nv; ++i) v[i] = (double)widen1(v_bits[i], dtype);
  }
  std::vector<double> l((size_t)B * Hq * Nq);
  or_dense_attention(g, q_i8.data(), q_scale.data(), k_i8.data(), k_scale.data(), v.data(), causal, scale, nullptr,
                     0, nullptr, nullptr, out, l.data());
  if (smooth_v) {
    for (int32_t b = 0; b < B; ++b)
      for (int32_t i = 0; i < Nq; ++i)
        for (int32_t h = 0; h < Hq; ++h) {
          if (!(l[((int64_t)b * Hq + h) * Nq + i] > -kInf)) continue;     // rows that see no key stay zero
          for (int32_t c = 0; c < d; ++c)
            out[(((int64_t)b * Nq + i) * Hq + h) * d + c] += (double)mu_v[((int64_t)b * Hkv + h / G) * d + c];
        }
  }
  if (smooth_k) {
    std::vector<double> corr((size_t)B * Hq * Nq);
    or_sage_lse_correction(q_bits, dtype, k_mean.data(), B, Nq, Hq, Hkv, d, scale, corr.data());
    for (size_t i = 0; i < l.size(); ++i) l[i] += corr[i];
  }
  if (lse != nullptr) std::copy(l.begin(), l.end(), lse);
}

// Variable-length dense forward on packed rows ([SAGE-MACA] API
// sageattn_varlen; its implementation slices out each batch element and
// attends it on its own): sequence b is rows cu_q[b] .. cu_q[b+1]-1 of q
// [total_q, Hq, d] and cu_k[b] .. cu_k[b+1]-1 of k, v [total_k, Hkv, d],
// attended as a one-sequence or_sage_forward. out [total_q, Hq, d]; lse
// [Hq, total_q] (optional; -inf for rows without keys).
void or_sage_varlen_forward(const uint16_t* q_bits, const uint16_t* k_bits, const uint16_t* v_bits, int32_t dtype,
                            const int32_t* cu_q, const int32_t* cu_k, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                            int32_t causal, int32_t smooth_k, int32_t smooth_v, double scale, double* out,
                            double* lse) {
  const int64_t total_q = cu_q[B];
  std::fill(out, out + total_q * Hq * d, 0.0);
  if (lse != nullptr) std::fill(lse, lse + (int64_t)Hq * total_q, -kInf);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t q0 = cu_q[b], q1 = cu_q[b + 1], k0 = cu_k[b], k1 = cu_k[b + 1];
    if (q1 == q0) continue;
    const or_dense_t g1{1, q1 - q0, k1 - k0, Hq, Hkv, d, 128, 64};
    std::vector<double> o((size_t)(q1 - q0) * Hq * d), l((size_t)Hq * (q1 - q0));
    or_sage_forward(&g1, q_bits + (int64_t)q0 * Hq * d, k_bits + (int64_t)k0 * Hkv * d, v_bits + (int64_t)k0 * Hkv * d,
                    dtype, causal, smooth_k, smooth_v, scale, o.data(), l.data());
    std::copy(o.begin(), o.end(), out + (int64_t)q0 * Hq * d);
    if (lse != nullptr)
      for (int32_t h = 0; h < Hq; ++h)
        for (int32_t i = 0; i < q1 - q0; ++i) lse[(int64_t)h * total_q + q0 + i] = l[(int64_t)h * (q1 - q0) + i];
  }
}

// ---- FP8 (E4M3) P.V -----------------------------------------------------------
// [SAGE-MACA] lists the FP8 P.V product of later SageAttention versions as
// not portable to its hardware; gfx950 has E4M3 matrix instructions. The
// pages fix none of its arithmetic. Readings (the plain definition, no tiling):
//   V per (b, KV head, channel) over all its tokens: s_c = fl32(max|V| / 448),
//   codes E4M3(fl32(V / s_c)) (448 = the largest E4M3 value);
//   per query row, m = the exact maximum of its visible scores and
//   P8_j = E4M3(448 * exp(s_j - m)), so the row's largest P is 448;
//   out = (sum_j P8_j V8_j / sum_j P8_j) * s_c (+ mu_v with smooth_v on rows
//   that see a key); lse = m + ln(sum_j P8_j / 448).
// Sums and products in fp64.

void or_v_fp8_per_channel(const float* v, int32_t B, int32_t N, int32_t H, int32_t d, double* vals, float* s) {
  for (int32_t b = 0; b < B; ++b)
    for (int32_t h = 0; h < H; ++h)
      for (int32_t c = 0; c < d; ++c) {
        float amax = 0.0f;
        for (int32_t t = 0; t < N; ++t) amax = std::max(amax, std::fabs(v[(((int64_t)b * N + t) * H + h) * d + c]));
        const float sc = amax / 448.0f;
        s[((int64_t)b * H + h) * d + c] = sc;
        for (int32_t t = 0; t < N; ++t) {
          const int64_t i = (((int64_t)b * N + t) * H + h) * d + c;
          vals[i] = sc > 0.0f ? e4m3_decode1(e4m3_encode1((double)(v[i] / sc))) : 0.0;
        }
      }
}

namespace {

// V for the FP8 product: fp32 values (V - mu_v with smooth_v), their E4M3
// values and channel scales, and mu_v.
struct Fp8V {
  std::vector<double> v8;
  std::vector<float> sv, mu;
};

Fp8V fp8_values(const or_dense_t* g, const float* v, int32_t smooth_v) {
  const int64_t n = (int64_t)g->B * g->Nk * g->Hkv * g->d;
  std::vector<float> vv(v, v + n);
  Fp8V r;
  r.mu.assign((size_t)g->B * g->Hkv * g->d, 0.0f);
  if (smooth_v) {
    r.mu = channel_means(vv.data(), g->B, g->Nk, g->Hkv, g->d);
    for (int32_t b = 0; b < g->B; ++b)
      for (int32_t t = 0; t < g->Nk; ++t)
        for (int32_t h = 0; h < g->Hkv; ++h)
          for (int32_t c = 0; c < g->d; ++c) {
            float& x = vv[(((int64_t)b * g->Nk + t) * g->Hkv + h) * g->d + c];
            x = x - r.mu[((int64_t)b * g->Hkv + h) * g->d + c];
          }
  }
  r.v8.resize(n);
  r.sv.resize((size_t)g->B * g->Hkv * g->d);
  or_v_fp8_per_channel(vv.data(), g->B, g->Nk, g->Hkv, g->d, r.v8.data(), r.sv.data());
  return r;
}

}  // namespace

// The plain FP8 definition above. v [B, Nk, Hkv, d] fp32 values. rows / head_mask
// as in or_dense_attention. Optional outputs for the tolerance of an
// implementation that rounds P from another reference (a lazily moved
// running maximum m' <= m, with P8' = E4M3(56 * exp(s - m')), 56 = 448 / 2^3):
// with exact weights w_j = p_j / sum p (p_j = exp(s_j - m)), each rounding
// error of a normal E4M3 value is at most u = 2^-4 relative (3 mantissa
// bits) and that of a subnormal one (below 2^-6) at most 2^-10 absolute,
// which is 2^-10 / (c sum p) of a weight for the scale c in {448, 56}. Taking
// the two roundings as independent and uniform within those bounds,
//   sigma[row][c]^2   = 1/3 sum_j (V_j,c - O_c)^2 (e56_j^2 + e448_j^2)
//   sigma_lse[row]^2  = 1/3 sum_j (e56_j^2 + e448_j^2)
// with e_c,j = u w_j if c p_j >= 2^-6 else 2^-10 / (c sum p), V and O in output
// units. They are the standard deviations of the difference between the two
// results to first order.
void or_dense_attention_fp8pv(const or_dense_t* g, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                              const float* k_scale, const float* v, int32_t causal, double scale, int32_t smooth_v,
                              const int64_t* rows, int64_t nrows, const uint8_t* head_mask, double* out,
                              double* lse, double* sigma, double* sigma_lse) {
  const int32_t G = g->Hq / g->Hkv, d = g->d, Nk = g->Nk;
  const double sc = resolve_scale(scale, d);
  const Fp8V V = fp8_values(g, v, smooth_v);
  const int64_t nr = rows != nullptr ? nrows : g->Nq;
  const int64_t n_out = (int64_t)g->B * g->Nq * g->Hq * d;
  std::fill(out, out + n_out, 0.0);
  if (lse != nullptr) std::fill(lse, lse + (int64_t)g->B * g->Hq * g->Nq, -kInf);
  if (sigma != nullptr) std::fill(sigma, sigma + n_out, 0.0);
  if (sigma_lse != nullptr) std::fill(sigma_lse, sigma_lse + (int64_t)g->B * g->Hq * g->Nq, 0.0);
  const double u = std::ldexp(1.0, -4), sub = std::ldexp(1.0, -6), sub_err = std::ldexp(1.0, -10);
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int32_t b = 0; b < g->B; ++b)
    for (int32_t h = 0; h < g->Hq; ++h)
      for (int64_t r = 0; r < nr; ++r) {
        if (head_mask != nullptr && !head_mask[h]) continue;
        const int64_t i = rows != nullptr ? rows[r] : r;
        const int32_t kvh = h / G;
        std::vector<double> s(Nk);
        dense_scores(g, q_i8, q_scale, k_i8, k_scale, causal, sc, b, h, i, s.data());
        double m = -kInf;
        for (int32_t j = 0; j < Nk; ++j) m = std::max(m, s[j]);
        if (!(m > -kInf)) continue;                       // no visible key: zeros, lse -inf
        std::vector<double> p(Nk), p8(Nk);
        double l8 = 0.0, lp = 0.0;
        for (int32_t j = 0; j < Nk; ++j) {
          p[j] = std::exp(s[j] - m);
          p8[j] = p[j] > 0.0 ? e4m3_decode1(e4m3_encode1(448.0 * p[j])) : 0.0;
          l8 += p8[j];
          lp += p[j];
        }
        const int64_t orow = (((int64_t)b * g->Nq + i) * g->Hq + h) * d;
        const int64_t vrow = (int64_t)b * Nk * g->Hkv + kvh;   // token t: (vrow + t * Hkv) * d
        const float* svc = V.sv.data() + ((int64_t)b * g->Hkv + kvh) * d;
        const float* muc = V.mu.data() + ((int64_t)b * g->Hkv + kvh) * d;
        std::vector<double> o(d, 0.0), oe(d, 0.0);
        for (int32_t j = 0; j < Nk; ++j) {
          if (p[j] == 0.0) continue;
          const double* vj = V.v8.data() + (vrow + (int64_t)j * g->Hkv) * d;
          for (int32_t c = 0; c < d; ++c) {
            o[c] += p8[j] * vj[c];
            oe[c] += p[j] * vj[c];
          }
        }
        for (int32_t c = 0; c < d; ++c)
          out[orow + c] = o[c] / l8 * (double)svc[c] + (smooth_v ? (double)muc[c] : 0.0);
        const int64_t li = ((int64_t)b * g->Hq + h) * g->Nq + i;
        if (lse != nullptr) lse[li] = m + std::log(l8 / 448.0);
        if (sigma != nullptr || sigma_lse != nullptr) {
          std::vector<double> var(d, 0.0);
          double var_l = 0.0;
          for (int32_t j = 0; j < Nk; ++j) {
            if (p[j] == 0.0) continue;
            const double w = p[j] / lp;
            const double e56 = 56.0 * p[j] >= sub ? u * w : sub_err / (56.0 * lp);
            const double e448 = 448.0 * p[j] >= sub ? u * w : sub_err / (448.0 * lp);
            const double ee = e56 * e56 + e448 * e448;
            var_l += ee;
            const double* vj = V.v8.data() + (vrow + (int64_t)j * g->Hkv) * d;
            for (int32_t c = 0; c < d; ++c) {
              const double dv = (vj[c] - oe[c] / lp) * (double)svc[c];
              var[c] += dv * dv * ee;
            }
          }
          if (sigma != nullptr)
            for (int32_t c = 0; c < d; ++c) sigma[orow + c] = std::sqrt(var[c] / 3.0);
          if (sigma_lse != nullptr) sigma_lse[li] = std::sqrt(var_l / 3.0);
        }
      }
}

// A model of a tiled implementation, used only to check the tolerance
// model above against a realistic rounding pattern (it is not the
// definition): keys in tiles of `tile` in order; a reference m_t per row,
// moved to max(m, tile maximum) when the tile maximum exceeds it by more
// than `slack` (base 2) for any of the `group` consecutive rows that decide
// together (the rows of one query group); P8 = E4M3(448 * 2^-slack *
// exp(s - m_t)); O and l accumulate P8 and are rescaled by exp(m_old - m_new)
// when the reference moves. out and lse as or_dense_attention_fp8pv (all rows
// and heads).
void or_dense_attention_fp8pv_lazy(const or_dense_t* g, const int8_t* q_i8, const float* q_scale,
                                   const int8_t* k_i8, const float* k_scale, const float* v, int32_t causal,
                                   double scale, int32_t smooth_v, int32_t tile, double slack, int32_t group,
                                   double* out, double* lse) {
  const int32_t G = g->Hq / g->Hkv, d = g->d, Nk = g->Nk, Nq = g->Nq;
  const double sc = resolve_scale(scale, d);
  const Fp8V V = fp8_values(g, v, smooth_v);
  const double top = 448.0 * std::exp2(-slack), slack_e = slack * std::log(2.0);
  std::fill(out, out + (int64_t)g->B * Nq * g->Hq * d, 0.0);
  if (lse != nullptr) std::fill(lse, lse + (int64_t)g->B * g->Hq * Nq, -kInf);
  const int32_t ngroups = (Nq + group - 1) / group;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int32_t b = 0; b < g->B; ++b)
    for (int32_t h = 0; h < g->Hq; ++h)
      for (int32_t gi = 0; gi < ngroups; ++gi) {
        const int32_t kvh = h / G;
        const int32_t r0 = gi * group, r1 = std::min(r0 + group, Nq), nrw = r1 - r0;
        std::vector<double> s((size_t)nrw * Nk), m(nrw, -kInf), l(nrw, 0.0), o((size_t)nrw * d, 0.0);
        for (int32_t r = 0; r < nrw; ++r)
          dense_scores(g, q_i8, q_scale, k_i8, k_scale, causal, sc, b, h, r0 + r, s.data() + (int64_t)r * Nk);
        const int64_t vrow = (int64_t)b * Nk * g->Hkv + kvh;
        for (int32_t t0 = 0; t0 < Nk; t0 += tile) {
          const int32_t t1 = std::min(t0 + tile, Nk);
          std::vector<double> mt(nrw, -kInf);
          bool move = false;
          for (int32_t r = 0; r < nrw; ++r) {
            for (int32_t j = t0; j < t1; ++j) mt[r] = std::max(mt[r], s[(int64_t)r * Nk + j]);
            move = move || mt[r] > m[r] + slack_e;
          }
          for (int32_t r = 0; r < nrw; ++r) {
            const double m_new = move ? std::max(m[r], mt[r]) : m[r];
            if (!(m_new > -kInf)) continue;
            const double alpha = m[r] > -kInf ? std::exp(m[r] - m_new) : 0.0;
            l[r] *= alpha;
            for (int32_t c = 0; c < d; ++c) o[(int64_t)r * d + c] *= alpha;
            m[r] = m_new;
            for (int32_t j = t0; j < t1; ++j) {
              const double x = s[(int64_t)r * Nk + j];
              if (!(x > -kInf)) continue;
              const double p8 = e4m3_decode1(e4m3_encode1(top * std::exp(x - m_new)));
              l[r] += p8;
              const double* vj = V.v8.data() + (vrow + (int64_t)j * g->Hkv) * d;
              for (int32_t c = 0; c < d; ++c) o[(int64_t)r * d + c] += p8 * vj[c];
            }
          }
        }
        for (int32_t r = 0; r < nrw; ++r) {
          if (!(l[r] > 0.0)) continue;
          const int64_t orow = (((int64_t)b * Nq + r0 + r) * g->Hq + h) * d;
          const float* svc = V.sv.data() + ((int64_t)b * g->Hkv + kvh) * d;
          const float* muc = V.mu.data() + ((int64_t)b * g->Hkv + kvh) * d;
          for (int32_t c = 0; c < d; ++c)
            out[orow + c] = o[(int64_t)r * d + c] / l[r] * (double)svc[c] + (smooth_v ? (double)muc[c] : 0.0);
          if (lse != nullptr) lse[((int64_t)b * g->Hq + h) * Nq + r0 + r] = m[r] + std::log(l[r] / top);
        }
      }
}

}  // extern "C"
