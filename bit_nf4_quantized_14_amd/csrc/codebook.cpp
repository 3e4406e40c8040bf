// NF4 codebook for the HIP path, derived on the host in double precision.
//
// "Qlora Expert", Core Concept: NF4's 16 levels sit at quantiles of N(0,1).
// The inverse normal CDF is obtained by Newton's method on
// Phi(x) = erfc(-x / sqrt 2) / 2 (std::erfc), a route of its own; the
// resulting levels and midpoint thresholds travel to the kernels as kernel
// arguments.
#include <cmath>

#include "qlora_nf4.h"
#include "qn_internal.h"

namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_pdf(double x) {
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * 3.14159265358979323846);
}

// Quantile of N(0,1) for p in (1/2, 1): Newton on the CDF from a logistic
// start, iterated until the step stops shrinking.
double normal_quantile_upper(double p) {
  double x = std::log(p / (1.0 - p)) / 1.702;
  double prev_step = 1e300;
  for (int it = 0; it < 100; ++it) {
    const double step = (normal_cdf(x) - p) / normal_pdf(x);
    x -= step;
    const double a = std::fabs(step);
    if (a == 0.0 || a >= prev_step) break;
    prev_step = a;
  }
  return x;
}

}  // namespace

namespace qn {

void derive_codebook(float levels[16], float thresholds[15]) {
  const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  double v[16];
  // 7 negative levels (ascending), 0, 8 positive levels (ascending).
  for (int i = 0; i < 7; ++i) {
    const double p = delta + (0.5 - delta) * double(i) / 7.0;
    v[i] = -normal_quantile_upper(p);
  }
  v[7] = 0.0;
  for (int i = 0; i < 8; ++i) {
    const double p = delta + (0.5 - delta) * double(7 - i) / 8.0;
    v[8 + i] = normal_quantile_upper(p);
  }
  const double top = v[15];
  float lv[16];
  for (int j = 0; j < 16; ++j) lv[j] = static_cast<float>(v[j] / top);
  if (levels)
    for (int j = 0; j < 16; ++j) levels[j] = lv[j];
  if (thresholds)
    for (int j = 0; j < 15; ++j)
      thresholds[j] =
          static_cast<float>((double(lv[j]) + double(lv[j + 1])) / 2.0);
}

bool derive_variant_codebook(int code, float levels[16],
                             float thresholds[15]) {
  float lv[16];
  if (code == QN_CODE_NF4) {
    derive_codebook(lv, nullptr);
  } else if (code == QN_CODE_FP4) {
    // E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent 0 is
    // subnormal (0.5 * mantissa).  Sorted: the 7 negative nonzero values,
    // two zeros (both +0), the 7 positive values; divided by the top, 6.
    double pos[8];
    for (int b = 0; b < 8; ++b) {
      const int e = b >> 1, m = b & 1;
      pos[b] = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
    }
    for (int i = 0; i < 7; ++i) lv[i] = static_cast<float>(-pos[7 - i] / 6.0);
    lv[7] = 0.0f;
    lv[8] = 0.0f;
    for (int i = 1; i < 8; ++i) lv[8 + i] = static_cast<float>(pos[i] / 6.0);
  } else if (code == QN_CODE_INT4) {
    for (int j = 0; j < 16; ++j) lv[j] = static_cast<float>((j - 8) / 7.0);
  } else {
    return false;
  }
  if (levels)
    for (int j = 0; j < 16; ++j) levels[j] = lv[j];
  if (thresholds)
    for (int j = 0; j < 15; ++j)
      thresholds[j] =
          static_cast<float>((double(lv[j]) + double(lv[j + 1])) / 2.0);
  return true;
}

}  // namespace qn

extern "C" int nf4_codebook(float levels[16], float thresholds[15]) {
  qn::derive_codebook(levels, thresholds);
  return QN_OK;
}

extern "C" int qn_codebook(int32_t code, float levels[16],
                           float thresholds[15]) {
  return qn::derive_variant_codebook(code, levels, thresholds) ? QN_OK
                                                               : QN_EINVAL;
}
