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
//
// The comparison tables of QLoRA-074 §四 (Table 2) go through the same
// kernels as other 16-entry tables in [-1, 1] (readings; the pages give no
// tables): int4 = (i − 8)/7 (absmax maps to 7; −8/7 is never nearest);
// FP4 E2M1 = sign, 2 exponent bits (bias 1, with subnormals), 1 mantissa
// bit, over 6; FP4 E3M0 = sign and 3 exponent bits, field 0 = zero, field e
// = 2^(e−7).  Both FP4 tables keep −0 and +0.
#include <cmath>
#include <cstring>

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

Codebook finish(const double (&vals)[16]) {
  Codebook cb;
  for (int i = 0; i < 16; ++i) cb.v[i] = (float)vals[i];
  for (int i = 0; i < 15; ++i) cb.mid[i] = ((double)cb.v[i] + (double)cb.v[i + 1]) * 0.5;
  return cb;
}

Codebook build_nf4() {
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
  return finish(vals);
}

Codebook build_int4() {
  double vals[16];
  for (int i = 0; i < 16; ++i) vals[i] = (double)(i - 8) / 7.0;
  return finish(vals);
}

// Ascending table of a 4-bit sign-magnitude format from the magnitudes of
// its 8 positive codes (ascending, starting at 0): −m7 .. −m1, −0, +0, m1 .. m7.
Codebook build_signed(const double (&mag)[8], double scale) {
  double vals[16];
  for (int i = 0; i < 8; ++i) vals[i] = -mag[7 - i] / scale;   // vals[7] = −0
  for (int i = 0; i < 8; ++i) vals[8 + i] = mag[i] / scale;
  return finish(vals);
}

Codebook build_e2m1() {
  double mag[8];
  for (int c = 0; c < 8; ++c) {
    const int e = c >> 1, m = c & 1;
    mag[c] = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  }
  return build_signed(mag, 6.0);
}

Codebook build_e3m0() {
  double mag[8];
  for (int e = 0; e < 8; ++e) mag[e] = e == 0 ? 0.0 : std::ldexp(1.0, e - 7);
  return build_signed(mag, 1.0);
}

// Number of midpoints strictly below x: the code of a weight with w/c1 = x.
int code_below(const Codebook& cb, double x) {
  int k = 0;
  for (int t = 0; t < 15; ++t) k += cb.mid[t] < x;
  return k;
}

EncodeGuide build_guide(const Codebook& cb) {
  constexpr double S = kGuideScale;
  uint8_t code[sizeof(EncodeGuide::packed)];
  for (size_t c = 0; c < sizeof(code); ++c)
    code[c] = (uint8_t)(c < (size_t)kGuideCells ? code_below(cb, ((double)c - S - 0.5) / S) : 15);
  bool ok = true;
  for (int c = 0; c + 1 < kGuideCells; ++c) ok = ok && code[c + 1] - code[c] <= 1;
  ok = ok && code_below(cb, 1.0) - code[kGuideCells - 1] <= 1;   // the last cell, up to x = 1
  for (int t = 0; t < 15; ++t) {
    const double e = cb.mid[t] * S + S + 0.5;   // exact: S is a power of two
    if (e > -1.0 && e < kGuideCells + 1.0) ok = ok && std::fabs(e - std::nearbyint(e)) > 1e-3;
  }
  EncodeGuide g;
  std::memcpy(g.packed, code, sizeof(code));
  g.zero_cell = -1;
  for (int c = 0; c < kGuideCells && ok; ++c)
    if (code[c] == 7) {
      g.zero_cell = c;
      break;
    }
  return g;
}

}  // namespace

const Codebook& host_codebook(int fmt) {
  static const Codebook tables[4] = {build_nf4(), build_int4(), build_e2m1(), build_e3m0()};
  return tables[fmt >= 0 && fmt < 4 ? fmt : 0];
}

const EncodeGuide& host_encode_guide(int fmt) {
  static const EncodeGuide guides[4] = {build_guide(host_codebook(0)), build_guide(host_codebook(1)),
                                        build_guide(host_codebook(2)), build_guide(host_codebook(3))};
  return guides[fmt >= 0 && fmt < 4 ? fmt : 0];
}

}  // namespace qlora
