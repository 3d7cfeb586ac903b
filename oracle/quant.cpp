// Oracle: storage formats, per-row symmetric INT8 quantization, the paged
// KV-cache layout, rotary embedding ahead of quantization, and the E4M3
// codec. TEST INFRASTRUCTURE ONLY (see oracle.h).
//
// Quantization follows [QK-MMAC] §4 (scale = max|x| / 127, code =
// round(x / scale), done once per row), §2.1 (codes in [-127, 127]) and
// [SAGE-MACA]'s quantization-kernel table (round to nearest even). Every
// step is one IEEE fp32 operation; the build disables contraction
// (-ffp-contract=off) so no step is fused.
#include <algorithm>

#include "impl.h"

namespace orc {

float widen1(uint16_t bits, int32_t dtype) {
  if (dtype == OR_BF16) {
    // bf16 is the upper half of an IEEE binary32
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  // IEEE binary16: sign, 5 exponent bits (bias 15), 10 mantissa bits
  const int e = (bits >> 10) & 31, m = bits & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? std::numeric_limits<double>::quiet_NaN() : kInf;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return (float)((bits & 0x8000) ? -v : v);
}

float quant_row(const float* x, int64_t n, int8_t* q) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs(x[i]));
  const float s = amax / 127.0f;                 // one correctly rounded fp32 division
  for (int64_t i = 0; i < n; ++i) {
    if (!(s > 0.0f)) {                           // all-zero row: scale 0, codes 0
      q[i] = 0;
      continue;
    }
    const float r = x[i] / s;                    // one correctly rounded fp32 division
    float c = std::nearbyint(r);                 // round half to even (default mode)
    c = std::min(std::max(c, -127.0f), 127.0f);
    q[i] = (int8_t)c;
  }
  return s;
}

// ---- E4M3 (OCP 8-bit float "e4m3fn"): sign, 4 exponent bits (bias 7), 3
// mantissa bits; exponent 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN,
// there is no infinity, the largest finite value is 1.75 * 2^8 = 448.
double e4m3_decode1(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  const double mag = e == 0 ? m / 8.0 * std::ldexp(1.0, -6) : (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
  return (c & 0x80) ? -mag : mag;
}

// Nearest finite E4M3 value, ties to the code with an even mantissa;
// magnitudes above 448 give 448; the sign bit is kept (also for zero).
uint8_t e4m3_encode1(double x) {
  const double a = std::min(std::fabs(x), 448.0);
  // codes 0x00 .. 0x7E have increasing values; find the first value >= a
  int lo = 0, hi = 0x7E;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (e4m3_decode1((uint8_t)mid) >= a) hi = mid;
    else lo = mid + 1;
  }
  int code = lo;
  if (lo > 0) {
    const double dhi = e4m3_decode1((uint8_t)lo) - a, dlo = a - e4m3_decode1((uint8_t)(lo - 1));
    if (dlo < dhi || (dlo == dhi && (lo & 1) != 0)) code = lo - 1;
  }
  return (uint8_t)(std::signbit(x) ? (code | 0x80) : code);
}

}  // namespace orc

using namespace orc;

extern "C" {

void or_widen(const uint16_t* bits, int32_t dtype, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen1(bits[i], dtype);
}

// Nearest IEEE binary16 to each fp32 value, ties to an even mantissa;
// magnitudes from 65520 on overflow to infinity.
void or_f32_to_f16_bits(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    const float f = x[i];
    const uint16_t sign = std::signbit(f) ? 0x8000 : 0;
    const double a = std::fabs((double)f);
    if (std::isnan(f)) { out[i] = sign | 0x7E00; continue; }
    if (a >= 65520.0) { out[i] = sign | 0x7C00; continue; }
    if (a == 0.0) { out[i] = sign; continue; }
    int e2;
    std::frexp(a, &e2);                         // a = f * 2^e2, f in [0.5, 1)
    int E = std::max(e2 - 1, -14);              // exponent of a's binade (subnormals: -14)
    double n_ = std::nearbyint(a / std::ldexp(1.0, E - 10));   // exact quotient, then ties to even
    if (n_ == 2048.0) { n_ = 1024.0; E += 1; }
    uint16_t b;
    if (E == -14) b = (uint16_t)n_;             // subnormal, or the smallest binade (n_ >= 1024 sets the exponent)
    else b = (uint16_t)(((E + 15) << 10) | ((int)n_ - 1024));
    out[i] = sign | b;
  }
}

void or_e4m3_encode(const double* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode1(x[i]);
}

void or_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_decode1(codes[i]);
}

void or_quant_rows(const float* x, int64_t rows, int64_t n, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) s[r] = quant_row(x + r * n, n, q + r * n);
}

// [QK-MMAC] §1, §3: every token with a slot >= 0 is quantized per (token, KV
// head) and scattered into its page: block = slot / 16, offset = slot % 16,
//   k_cache[block][h][c][offset][j] = code of channel 16c + j
//   k_scale[block][h][offset]        = its scale
//   v_cache[block][h][i][offset]     = V value i (16-bit bits, or INT8 code
//                                      with v_scale[block][h][offset])
// Slots are distinct, so tokens are independent.
void or_write_kv(const float* k, const uint16_t* v_bits, int32_t v_dtype, int32_t v_int8, const int64_t* slots,
                 int64_t T, int32_t H, int32_t d, int8_t* k_cache, float* k_scale, void* v_cache, float* v_scale) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const int64_t slot = slots[t];
    if (slot < 0) continue;
    const int64_t blk = slot / kBlock, off = slot % kBlock;
    std::vector<int8_t> codes(d);
    std::vector<float> vrow(d);
    for (int32_t h = 0; h < H; ++h) {
      const int64_t bh = blk * H + h;
      const float s = quant_row(k + (t * H + h) * d, d, codes.data());
      for (int32_t i = 0; i < d; ++i) k_cache[((bh * (d / 16) + i / 16) * kBlock + off) * 16 + i % 16] = codes[i];
      k_scale[bh * kBlock + off] = s;
      const uint16_t* vr = v_bits + (t * H + h) * d;
      if (v_int8) {
        for (int32_t i = 0; i < d; ++i) vrow[i] = widen1(vr[i], v_dtype);
        const float sv = quant_row(vrow.data(), d, codes.data());
        for (int32_t i = 0; i < d; ++i) static_cast<int8_t*>(v_cache)[(bh * d + i) * kBlock + off] = codes[i];
        v_scale[bh * kBlock + off] = sv;
      } else {
        for (int32_t i = 0; i < d; ++i) static_cast<uint16_t*>(v_cache)[(bh * d + i) * kBlock + off] = vr[i];
      }
    }
  }
}

// [QK-MMAC] §3: logical token t of a sequence -> table entry t / 16 -> its
// physical block -> slot t % 16 of that page -> the head_dim chunks.
// Returns the sequence's first ctx tokens of KV head kvh: codes kq [ctx, d],
// scales sk [ctx], V [ctx, d] dequantized in fp64 (16-bit value, or code * sV).
void or_gather_kv(const int8_t* k_cache, const float* k_scale, const void* v_cache, const float* v_scale,
                  int32_t v_dtype, int32_t H, int32_t d, const int32_t* table_row, int32_t ctx, int32_t kvh,
                  int8_t* kq, float* sk, double* v) {
  for (int32_t t = 0; t < ctx; ++t) {
    const int64_t bh = (int64_t)table_row[t / kBlock] * H + kvh;
    const int off = t % kBlock;
    for (int32_t i = 0; i < d; ++i) kq[(int64_t)t * d + i] = k_cache[((bh * (d / 16) + i / 16) * kBlock + off) * 16 + i % 16];
    sk[t] = k_scale[bh * kBlock + off];
    for (int32_t i = 0; i < d; ++i) {
      const int64_t vi = (bh * d + i) * kBlock + off;
      v[(int64_t)t * d + i] = v_scale != nullptr
                                  ? (double)static_cast<const int8_t*>(v_cache)[vi] * (double)v_scale[bh * kBlock + off]
                                  : (double)widen1(static_cast<const uint16_t*>(v_cache)[vi], v_dtype);
    }
  }
}

// Rotary embedding ahead of quantization ([QK-MMAC] §4 names a RoPE/KV
// producer that quantizes the query; the pages give no rotary parameters).
// Readings: table row p holds cos(p w_i) in column i and sin(p w_i) in
// column rot/2 + i; "neox" pairs channel i with i + rot/2, otherwise 2i with
// 2i + 1; pair i uses frequency i; channels from rot on pass through. A pair
// (a, b) becomes (fl32(fl32(a cos) - fl32(b sin)), fl32(fl32(b cos) +
// fl32(a sin))) from the widened 16-bit inputs.
void or_apply_rope(const uint16_t* x_bits, int32_t dtype, int64_t T, int32_t H, int32_t d, const int64_t* pos,
                   const float* cos_sin, int32_t rot, int32_t neox, float* out) {
  const int32_t half = rot / 2;
  for (int64_t t = 0; t < T; ++t) {
    const float* cs = cos_sin + pos[t] * rot;
    for (int32_t h = 0; h < H; ++h) {
      const uint16_t* xr = x_bits + (t * H + h) * d;
      float* o = out + (t * H + h) * d;
      for (int32_t i = 0; i < d; ++i) o[i] = widen1(xr[i], dtype);
      for (int32_t i = 0; i < half; ++i) {
        const int32_t ia = neox ? i : 2 * i, ib = neox ? i + half : 2 * i + 1;
        const float a = widen1(xr[ia], dtype), b = widen1(xr[ib], dtype);
        const float c = cs[i], s = cs[half + i];
        const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        o[ia] = ac - bs;
        o[ib] = bc + as;
      }
    }
  }
}

}  // extern "C"
