// Helpers shared by the oracle's source files (oracle-internal; the GPU
// library neither includes nor links anything from here).
#ifndef QA_ORACLE_IMPL_H
#define QA_ORACLE_IMPL_H

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "oracle.h"

namespace orc {

constexpr double kInf = std::numeric_limits<double>::infinity();
constexpr int kBlock = 16;   // tokens per cache block

// One 16-bit storage pattern as the fp32 value it denotes (exact).
float widen1(uint16_t bits, int32_t dtype);

// Symmetric INT8 of one row of n fp32 values; returns the scale.
float quant_row(const float* x, int64_t n, int8_t* q);

// softmax_scale: a positive caller value is used as the fp32 number the
// GPU receives; otherwise 1/sqrt(d).
inline double resolve_scale(double scale, int32_t d) {
  return scale > 0.0 ? (double)(float)scale : 1.0 / std::sqrt((double)d);
}

// Two-pass softmax over n scores (masked keys carry -inf) and the product
// with n value rows of length d (row stride ld), in fp64. A row with no
// visible key gives zeros. Returns the maximum score (-inf if none).
double softmax_pv(const double* s, int64_t n, const double* v, int64_t ld, int32_t d, double* out);

// ln(sum_j exp(s_j)) as m + ln(sum_j exp(s_j - m)); -inf without a visible key.
double logsumexp(const double* s, int64_t n);

uint8_t e4m3_encode1(double x);
double e4m3_decode1(uint8_t c);

}  // namespace orc

#endif
