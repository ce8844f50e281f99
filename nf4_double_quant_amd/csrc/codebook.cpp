// NF4 codebook, generated on the host when the library is loaded.
//
// "074｜QLoRA：把大模型放进显存，再用小适配器改变它" §二: NF4 uses 16 values
// inspired by normal-distribution quantiles, finer near zero, coarser in the
// tails, keeps an exact zero and is normalised by the block absmax.  Reading
// taken: 8 positive values Φ⁻¹(1/2 + j(p−1/2)/8), j = 1..8, 7 negative values
// −Φ⁻¹(1/2 + j(p−1/2)/7), j = 1..7, and 0, all divided by Φ⁻¹(p) with
// p = 1 − (1/32 + 1/30)/2 (the tail level of the QLoRA paper), computed in
// double and rounded to fp32 once.
//
// Φ⁻¹ here is Newton's method on Φ(x) = erfc(−x/√2)/2 in long double.
#include <cmath>

#include "common.h"

namespace qlora {
namespace {

long double normal_cdf(long double x) {
  return 0.5L * std::erfc(-x / std::sqrt(2.0L));
}

long double normal_pdf(long double x) {
  return std::exp(-0.5L * x * x) / std::sqrt(2.0L * 3.14159265358979323846264338327950288L);
}

double normal_quantile(double p) {
  long double x = 0.0L;
  for (int it = 0; it < 200; ++it) {
    long double step = (normal_cdf(x) - (long double)p) / normal_pdf(x);
    long double nx = x - step;
    if (nx == x) break;
    x = nx;
  }
  return (double)x;
}

Codebook build() {
  const double p_max = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  const double half_span = p_max - 0.5;
  const double z_max = normal_quantile(p_max);
  double vals[16];
  int k = 0;
  for (int j = 7; j >= 1; --j)  // most negative first
    vals[k++] = -normal_quantile(0.5 + half_span * ((double)j / 7.0)) / z_max;
  vals[k++] = 0.0;
  for (int j = 1; j <= 8; ++j)
    vals[k++] = normal_quantile(0.5 + half_span * ((double)j / 8.0)) / z_max;
  Codebook cb;
  for (int i = 0; i < 16; ++i) cb.v[i] = (float)vals[i];
  for (int i = 0; i < 15; ++i) cb.mid[i] = ((double)cb.v[i] + (double)cb.v[i + 1]) * 0.5;
  return cb;
}

}  // namespace

const Codebook& host_codebook() {
  static const Codebook cb = build();
  return cb;
}

}  // namespace qlora
