// Standard normal quantile for the statistical block cutoff of the BSA notes
// (design 2: p = mean + std * U(1 - k/n), U the normal quantile function).
//
// Method: M. J. Wichura, "Algorithm AS 241: The percentage points of the
// normal distribution", Applied Statistics 37 (1988) 477-484, the PPND16
// variant (about 16 correct digits): a rational function of degree 7 in
// r = 0.180625 - q^2 near the centre (|q| = |p - 1/2| <= 0.425), and two
// rational functions of degree 7 in r = sqrt(-ln(min(p, 1 - p))) in the
// tails (r <= 5 and r > 5), with the sign of q.
#include <cmath>
#include <limits>

#include "dbs_internal.h"

namespace dbs {
namespace {

// Coefficients of the published algorithm, constant term first.
constexpr double kCentreNum[8] = {3.3871328727963666080e0, 1.3314166789178437745e+2, 1.9715909503065514427e+3,
                                  1.3731693765509461125e+4, 4.5921953931549871457e+4, 6.7265770927008700853e+4,
                                  3.3430575583588128105e+4, 2.5090809287301226727e+3};
constexpr double kCentreDen[8] = {1.0, 4.2313330701600911252e+1, 6.8718700749205790830e+2,
                                  5.3941960214247511077e+3, 2.1213794301586595867e+4, 3.9307895800092710610e+4,
                                  2.8729085735721942674e+4, 5.2264952788528545610e+3};
constexpr double kNearNum[8] = {1.42343711074968357734e0, 4.63033784615654529590e0, 5.76949722146069140550e0,
                                3.64784832476320460504e0, 1.27045825245236838258e0, 2.41780725177450611770e-1,
                                2.27238449892691845833e-2, 7.74545014278341407640e-4};
constexpr double kNearDen[8] = {1.0, 2.05319162663775882187e0, 1.67638483018380384940e0, 6.89767334985100004550e-1,
                                1.48103976427480074590e-1, 1.51986665636164571966e-2, 5.47593808499534494600e-4,
                                1.05075007164441684324e-9};
constexpr double kFarNum[8] = {6.65790464350110377720e0, 5.46378491116411436990e0, 1.78482653991729133580e0,
                               2.96560571828504891230e-1, 2.65321895265761230930e-2, 1.24266094738807843860e-3,
                               2.71155556874348757815e-5, 2.01033439929228813265e-7};
constexpr double kFarDen[8] = {1.0, 5.99832206555887937690e-1, 1.36929880922735805310e-1, 1.48753612908506148525e-2,
                               7.86869131145613259100e-4, 1.84631831751005468180e-5, 1.42151175831644588870e-7,
                               2.04426310338993978564e-15};

double horner(const double (&c)[8], double x) {
  double v = c[7];
  for (int i = 6; i >= 0; --i) v = v * x + c[i];
  return v;
}

}  // namespace

double normal_quantile(double p) {
  if (!(p > 0.0 && p < 1.0)) {
    if (p == 0.0) return -std::numeric_limits<double>::infinity();
    if (p == 1.0) return std::numeric_limits<double>::infinity();
    return std::numeric_limits<double>::quiet_NaN();
  }
  const double q = p - 0.5;
  if (std::fabs(q) <= 0.425) {
    const double r = 0.180625 - q * q;
    return q * horner(kCentreNum, r) / horner(kCentreDen, r);
  }
  double r = std::sqrt(-std::log(q < 0.0 ? p : 1.0 - p));
  double x;
  if (r <= 5.0) {
    r -= 1.6;
    x = horner(kNearNum, r) / horner(kNearDen, r);
  } else {
    r -= 5.0;
    x = horner(kFarNum, r) / horner(kFarDen, r);
  }
  return q < 0.0 ? -x : x;
}

}  // namespace dbs
