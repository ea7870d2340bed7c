// Host-side codebook solver and codec set-up (fp64, no GPU calls).
//
// "Google presenta TurboQuant ..." (7minutos.es), "La mecánica geométrica de
// TurboQuant": each rotated coordinate of a unit vector follows a Beta law;
// the scalar quantizer minimising the MSE cost C(f_X, b) is found once per
// bit width and stored.  The density of one coordinate of a uniform point on
// S^{d-1} is f_d(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1], with
// C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).  The outer cells of the cost
// extend to -1 and +1, where f_d vanishes.
//
// Lloyd-Max alternates the two optimality conditions: thresholds at the
// midpoints of neighbouring centroids, centroids at the conditional means of
// their cells.  Cell masses and first moments are taken in closed form here:
//   P(X <= t)          = 1/2 + sgn(t)/2 * I_{t^2}(1/2, (d-1)/2)
//                        (X^2 follows Beta(1/2, (d-1)/2)),
//   int_a^b x f_d(x)dx = C_d / (d-1) * ((1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)),
// with the regularized incomplete beta I evaluated by its continued fraction
// (modified Lentz).

#include <cmath>
#include <cstring>

#include "tq.h"

namespace {

// Continued fraction of the incomplete beta function, modified Lentz.
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0;
  double d = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(d) < tiny) d = tiny;
  d = 1.0 / d;
  double h = d;
  for (int m = 1; m <= 100000; ++m) {
    const double m2 = 2.0 * m;
    // even step
    double num = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
    d = 1.0 + num * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    h *= d * c;
    // odd step
    num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
    d = 1.0 + num * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    const double delta = d * c;
    h *= delta;
    if (std::fabs(delta - 1.0) < 1e-17) break;
  }
  return h;
}

// ln Gamma(z + 1/2) - ln Gamma(z), z > 0, without the cancellation of two
// large lgamma values: shift z up to w >= 20 with the recurrence
// Gamma(w+1) = w Gamma(w), then take the difference of Stirling's series
// ln Gamma(w) = (w - 1/2) ln w - w + ln(2 pi)/2 + sum B_2k / (2k (2k-1) w^(2k-1)).
double log_gamma_ratio_half(double z) {
  double log_prod = 0.0;
  while (z < 20.0) {
    log_prod += std::log(z / (z + 0.5));
    z += 1.0;
  }
  const double w = z, v = z + 0.5;
  // (v - 1/2) ln v - v - ((w - 1/2) ln w - w) = w ln(1 + 1/(2w)) + ln(w)/2 - 1/2
  double r = w * std::log1p(0.5 / w) + 0.5 * std::log(w) - 0.5;
  static const double coef[] = {1.0 / 12.0, -1.0 / 360.0, 1.0 / 1260.0,
                                -1.0 / 1680.0, 1.0 / 1188.0,
                                -691.0 / 360360.0, 1.0 / 156.0};
  double pv = 1.0 / v, pw = 1.0 / w;
  const double v2 = pv * pv, w2 = pw * pw;
  for (double cf : coef) {
    r += cf * (pv - pw);
    pv *= v2;
    pw *= w2;
  }
  return r + log_prod;
}

// Regularized incomplete beta I_x(1/2, b), 0 <= x <= 1.
double inc_beta_half(double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double a = 0.5;
  // ln B(1/2, b) = ln Gamma(1/2) + ln Gamma(b) - ln Gamma(b + 1/2)
  const double log_beta = 0.5 * std::log(M_PI) - log_gamma_ratio_half(b);
  const double front = std::exp(a * std::log(x) + b * std::log1p(-x) - log_beta);
  if (x < (a + 1.0) / (a + b + 2.0)) return front * beta_cf(a, b, x) / a;
  return 1.0 - front * beta_cf(b, a, 1.0 - x) / b;
}

struct Coord {
  int d;
  double half_dm1;   // (d-1)/2
  double cd;         // C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2))
  explicit Coord(int dim) : d(dim), half_dm1(0.5 * (dim - 1)) {
    cd = std::exp(log_gamma_ratio_half(half_dm1)) / std::sqrt(M_PI);
  }
  double cdf(double t) const {
    if (t <= -1.0) return 0.0;
    if (t >= 1.0) return 1.0;
    const double i = inc_beta_half(half_dm1, t * t);
    return t >= 0.0 ? 0.5 + 0.5 * i : 0.5 - 0.5 * i;
  }
  // (1 - t^2)^((d-1)/2)
  double tail(double t) const {
    if (t <= -1.0 || t >= 1.0) return 0.0;
    return std::exp(half_dm1 * std::log1p(-t * t));
  }
  double first_moment(double a, double b) const {
    return cd / (d - 1.0) * (tail(a) - tail(b));
  }
};

}  // namespace

extern "C" const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_NOT_CONVERGED: return "codebook iteration did not converge";
    case TQ_ERR_HIP: return "HIP runtime error";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ_ERR_TOO_LARGE: return "request needs more than the library's fixed scratch";
    default: return "unknown status";
  }
}

extern "C" int tq_build_codebook(int d, int bits, double* centroids,
                                 double* thresholds) {
  if (d < 3 || bits < 1 || bits > 4 || centroids == nullptr ||
      (bits > 0 && thresholds == nullptr))
    return TQ_ERR_INVALID_ARG;
  const int n = 1 << bits;
  const Coord f(d);
  double c[TQ_MAX_LEVELS], t[TQ_MAX_LEVELS + 1];
  // start: evenly spaced over +-2.5 standard deviations (1/sqrt(d))
  const double span = std::fmin(0.9, 2.5 / std::sqrt((double)d));
  for (int k = 0; k < n; ++k) c[k] = -span + 2.0 * span * k / (n - 1);
  const int max_iter = 200000;
  double last_step = 1.0;
  int stalled = 0;
  for (int it = 0; it < max_iter; ++it) {
    t[0] = -1.0;
    for (int k = 1; k < n; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    t[n] = 1.0;
    double step = 0.0;
    double prev_cdf = f.cdf(t[0]);
    for (int k = 0; k < n; ++k) {
      const double next_cdf = f.cdf(t[k + 1]);
      const double mass = next_cdf - prev_cdf;
      prev_cdf = next_cdf;
      if (!(mass > 0.0)) return TQ_ERR_NOT_CONVERGED;
      const double nc = f.first_moment(t[k], t[k + 1]) / mass;
      step = std::fmax(step, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    // Converged once the update reaches the rounding level of the cell
    // integrals: either it vanishes, or it stops shrinking for 64 steps while
    // already below 1e-15.
    if (step == 0.0) break;
    if (step < last_step) {
      last_step = step;
      stalled = 0;
    } else if (++stalled >= 64 && last_step < 1e-15) {
      break;
    }
    if (it == max_iter - 1) return TQ_ERR_NOT_CONVERGED;
  }
  // f_d is even, so the optimum is symmetric; symmetrising removes the
  // rounding noise and puts the middle threshold exactly at 0.
  for (int k = 0; k < n / 2; ++k) {
    const double v = 0.5 * (c[n - 1 - k] - c[k]);
    c[k] = -v;
    c[n - 1 - k] = v;
  }
  for (int k = 0; k < n; ++k) centroids[k] = c[k];
  for (int k = 1; k < n; ++k) thresholds[k - 1] = 0.5 * (c[k - 1] + c[k]);
  return TQ_OK;
}

extern "C" int tq_codec_init(tq_codec* codec, int d, int mode, int bits,
                             const uint32_t* flip, const float* S) {
  if (codec == nullptr || flip == nullptr) return TQ_ERR_INVALID_ARG;
  if (d < 3 || d > TQ_MAX_D) return TQ_ERR_INVALID_ARG;
  if (mode != TQ_MSE && mode != TQ_PROD) return TQ_ERR_INVALID_ARG;
  const int code_bits = mode == TQ_PROD ? bits - 1 : bits;
  if (code_bits < 1 || code_bits > 4) return TQ_ERR_INVALID_ARG;
  if (mode == TQ_PROD && S == nullptr) return TQ_ERR_INVALID_ARG;
  double c[TQ_MAX_LEVELS], t[TQ_MAX_LEVELS];
  const int st = tq_build_codebook(d, code_bits, c, t);
  if (st != TQ_OK) return st;
  std::memset(codec, 0, sizeof(*codec));
  codec->d = d;
  codec->mode = mode;
  codec->bits = bits;
  codec->code_bits = code_bits;
  codec->m = mode == TQ_PROD ? d : 0;
  const int n = 1 << code_bits;
  for (int k = 0; k < n; ++k) codec->centroids[k] = (float)c[k];
  for (int k = 0; k + 1 < n; ++k) codec->thresholds[k] = (float)t[k];
  const int words = (d + 31) / 32;
  for (int w = 0; w < words; ++w) codec->flip[w] = flip[w];
  if (d % 32) codec->flip[words - 1] &= (1u << (d % 32)) - 1u;
  codec->S = mode == TQ_PROD ? S : nullptr;
  return TQ_OK;
}
