// NF4 codebook, computed by the library on the host.
//
// The pages name NF4 (bitsandbytes) as the base format but print no codebook.  The
// levels used here follow the NormalFloat construction of the QLoRA paper (Dettmers
// et al. 2023, section 3): with Phi the standard normal CDF and delta = 1 - (1/32 +
// 1/30)/2, the 8 positive levels are Phi^-1(1/2 + j (delta - 1/2) / 8) / Phi^-1(delta)
// for j = 1..8, the 7 negative levels are -Phi^-1(1/2 + j (delta - 1/2) / 7) /
// Phi^-1(delta) for j = 1..7, plus an exact zero; each is computed in double and
// rounded once to float.  Phi^-1 is found by bisection on Phi(x) = erfc(-x/sqrt 2)/2,
// which converges to the double nearest the root of the library erfc.
#include <math.h>

#include <algorithm>

#include "internal.hpp"

namespace msq {
namespace {

double phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

double inv_phi(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 400; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (phi(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  // pick whichever endpoint has the smaller residual
  return fabs(phi(lo) - p) <= fabs(phi(hi) - p) ? lo : hi;
}

struct Tables {
  Nf4Lut lut;
  Nf4Mid mid;
  Tables() {
    const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
    const double top = inv_phi(delta);
    double v[16];
    int n = 0;
    for (int j = 1; j <= 7; ++j) v[n++] = -inv_phi(0.5 + j * (delta - 0.5) / 7.0) / top;
    v[n++] = 0.0;
    for (int j = 1; j <= 8; ++j) v[n++] = inv_phi(0.5 + j * (delta - 0.5) / 8.0) / top;
    std::sort(v, v + 16);
    for (int c = 0; c < 16; ++c) lut.v[c] = (float)v[c];
    lut.v[0] = -1.0f;  // the normalisation makes the extremes exactly -1 and +1
    lut.v[15] = 1.0f;
    lut.v[7] = 0.0f;
    for (int i = 0; i < 15; ++i) mid.m[i] = ((double)lut.v[i] + (double)lut.v[i + 1]) * 0.5;
  }
};

const Tables& tables() {
  static const Tables t;
  return t;
}

}  // namespace

const Nf4Lut& nf4_lut() { return tables().lut; }
const Nf4Mid& nf4_mid() { return tables().mid; }

}  // namespace msq
