// NF4 codebook, decision thresholds and the quantizer's bucket table (host code).
//
// The 16 levels come from N(0,1) quantiles with equal probability mass per bin,
// normalised to [-1, 1], with an exact zero obtained by giving the negative and
// positive halves different level counts ([QLoRA note] "2. NF4"; [Paper note]
// "关键设计 1", quantile-midpoint equation; [Digest] "数学公式与关键细节" item 1,
// "特点").  The printed midpoint formula has no index range; the reading used
// here: 7 negative levels, 0, 8 positive levels; each half samples the
// quantile function on an equally spaced probability grid from 1/2 to
// delta = 31/32 (the probability centre of the outermost of 16 equal-mass
// bins); both halves are divided by the quantile at delta so the ends are
// exactly -1 and +1; values are computed in double and rounded once to float.
//
// The quantile function here is a bisection on Phi(x) = erfc(-x / sqrt 2) / 2
// (libm erfc), run until the bracket stops shrinking.
//
// The FP4 table is the baseline 4-bit float of the pages' data-type comparison
// ([Digest] "6. 实验结果与分析", "核心结果分析" item 2), which gives no value set.
// Reading: the E2M1 float (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit)
// divided by 6 so that the block absmax maps to +-1 as for NF4; its two zeros give
// the ascending table -1 .. -1/12, 0, 0, 1/12 .. 1 (each value m / 6 computed in
// double and rounded once to float).  Thresholds and the bucket table follow the same
// rules as for NF4 (the threshold between the two zeros is 0: x = 0 takes code 7).

#include "../../include/qlora_nf4.h"
#include "qlora_internal.h"

#include <cmath>
#include <mutex>

namespace qlora {
namespace {

double phi(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double phi_inv(double p) {
  double lo = -40.0, hi = 40.0;
  for (;;) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) return mid;
    if (phi(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
}

void nf4_levels(float q[16]) {
  const double delta = 31.0 / 32.0;
  const double z = phi_inv(delta);
  double lv[16];
  // negative half: j = 7 .. 1 gives ascending values -1 .. q[6]
  for (int j = 7; j >= 1; --j) lv[7 - j] = -phi_inv(0.5 + j * (delta - 0.5) / 7.0) / z;
  lv[7] = 0.0;
  for (int j = 1; j <= 8; ++j) lv[7 + j] = phi_inv(0.5 + j * (delta - 0.5) / 8.0) / z;
  lv[0] = -1.0;
  lv[15] = 1.0;
  for (int i = 0; i < 16; ++i) q[i] = static_cast<float>(lv[i]);
}

void fp4_levels(float q[16]) {
  // E2M1 magnitudes in halves: 0, 1, 2, 3, 4, 6, 8, 12 (i.e. 0 .. 6)
  static const int halves[8] = {0, 1, 2, 3, 4, 6, 8, 12};
  for (int i = 0; i < 8; ++i) {
    const double v = halves[i] / 12.0;  // (halves / 2) / 6
    q[8 + i] = static_cast<float>(v);
    q[7 - i] = static_cast<float>(-v);
  }
  q[7] = 0.0f;  // the negative zero code decodes to +0 like the positive one
}

Codebook build(int quant_type) {
  Codebook cb{};
  if (quant_type == kQuantFP4)
    fp4_levels(cb.q);
  else
    nf4_levels(cb.q);

  // T[j] = largest float <= (q[j] + q[j+1]) / 2 (the double sum of two floats in
  // [-1, 1] is exact), so that for float x: x > T[j] <=> x > the exact midpoint;
  // an exact tie therefore goes to the lower code.
  for (int j = 0; j < 15; ++j) {
    double t = (static_cast<double>(cb.q[j]) + static_cast<double>(cb.q[j + 1])) * 0.5;
    float f = static_cast<float>(t);
    if (static_cast<double>(f) > t) f = std::nextafter(f, -INFINITY);
    cb.thr[j] = f;
  }

  // Bucket table for the quantizer: bucket i collects x with 64 x + 64 in [i, i+1)
  // (x in [-1, 1], i in 0..128).  Each bucket's window, widened by 2^-10 on both
  // sides to absorb the rounding of 64 x + 64, contains at most one threshold
  // (the thresholds are more than 0.07 apart).  code = base[i] + (x > bthr[i]),
  // where base[i] counts the thresholds below the window and bthr[i] is the one
  // threshold inside it (2.0 when none: never exceeded since |x| <= 1).
  cb.bucket_ok = true;
  const double eps = 1.0 / 1024.0;
  for (int i = 0; i < kBuckets; ++i) {
    double lo = (i - 64) / 64.0 - eps, hi = (i - 63) / 64.0 + eps;
    int base = 0, inside = 0;
    float t_in = 2.0f;
    for (int j = 0; j < 15; ++j) {
      double tj = cb.thr[j];
      if (tj < lo) {
        ++base;
      } else if (tj <= hi) {
        ++inside;
        t_in = cb.thr[j];
      }
    }
    if (inside > 1) cb.bucket_ok = false;
    cb.bucket_base[i] = base;
    cb.bucket_thr[i] = t_in;
  }
  return cb;
}

}  // namespace

const Codebook &codebook(int quant_type) {
  static std::once_flag once;
  static Codebook cb[2];
  std::call_once(once, [] {
    cb[0] = build(kQuantNF4);
    cb[1] = build(kQuantFP4);
  });
  return cb[quant_type == kQuantFP4 ? 1 : 0];
}

LevelTable level_table(int quant_type) {
  LevelTable lv;
  const Codebook &cb = codebook(quant_type);
  for (int i = 0; i < 16; ++i) lv.q[i] = cb.q[i];
  return lv;
}

}  // namespace qlora

extern "C" void qlora_nf4_codebook(float q[16], float thresholds[15]) {
  qlora_codebook(QLORA_QUANT_NF4, q, thresholds);
}

extern "C" int qlora_codebook(int quant_type, float q[16], float thresholds[15]) {
  if (quant_type != qlora::kQuantNF4 && quant_type != qlora::kQuantFP4) return QLORA_ERR_DTYPE;
  const qlora::Codebook &cb = qlora::codebook(quant_type);
  if (q)
    for (int i = 0; i < 16; ++i) q[i] = cb.q[i];
  if (thresholds)
    for (int j = 0; j < 15; ++j) thresholds[j] = cb.thr[j];
  return QLORA_OK;
}
