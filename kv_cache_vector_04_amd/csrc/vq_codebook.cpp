// FibQuant k = 2 codebook (host, fp64) and the vector codec struct.
//
// "FibQuant", "2.1 La Sorgente Canonica": a block of two consecutive rotated
// coordinates of a unit vector in d dimensions has the density
// (d-2)/(2 pi) (1 - |y|^2)^((d-4)/2) on the unit disk (|y|^2 ~ Beta(1, (d-2)/2)).
// "2.2 Costruzione del Codice", for N codewords:
//   - radius of codeword n by Bennett-Gersho companding (point density
//     ~ f^(1/2) for k = 2, whose mass inside r is 1 - (1 - r^2)^(d/4)):
//     r_n^2 = 1 - (1 - (n + 1/2)/N)^(4/d);
//   - angle on the planar Fibonacci spiral: n times the golden angle
//     pi (3 - sqrt 5), plus a restart phase;
//   - Lloyd refinement on an equal-probability polar quadrature of the
//     density (128 rings at the (i + 1/2)/128 quantiles of |y|^2, 256
//     angles), 40 iterations from each of the phases 0 and 1/2 golden angle,
//     the lower-MSE result kept.  Nearest-codeword ties go to the lower
//     index; a codeword with an empty cell stays where it is.

#include <cmath>
#include <cstdint>
#include <vector>

#include "tq.h"

namespace {

constexpr int kRings = 128;
constexpr int kAngles = 256;
constexpr int kLloydIters = 40;
constexpr double kRestartMargin = 1e-9;

struct Pt {
  double x, y;
};

int nearest_code(const Pt& p, const std::vector<Pt>& c) {
  int best = 0;
  double bd = INFINITY;
  for (size_t n = 0; n < c.size(); ++n) {
    const double dx = p.x - c[n].x, dy = p.y - c[n].y;
    const double dd = dx * dx + dy * dy;
    if (dd < bd) {
      bd = dd;
      best = (int)n;
    }
  }
  return best;
}

double code_mse(const std::vector<Pt>& pts, const std::vector<Pt>& c) {
  double s = 0.0;
  for (const Pt& p : pts) {
    const Pt& q = c[nearest_code(p, c)];
    s += (p.x - q.x) * (p.x - q.x) + (p.y - q.y) * (p.y - q.y);
  }
  return s / (double)pts.size();
}

}  // namespace

extern "C" int tq_build_vq_codebook(int d, int n_codes, double* codewords) {
  if (d < 6 || codewords == nullptr) return TQ_ERR_INVALID_ARG;
  if (n_codes < 2 || n_codes > TQ_VQ_MAX_CODES || (n_codes & (n_codes - 1))) return TQ_ERR_INVALID_ARG;
  const double golden = M_PI * (3.0 - std::sqrt(5.0));
  std::vector<Pt> pts;
  pts.reserve((size_t)kRings * kAngles);
  for (int i = 0; i < kRings; ++i) {
    const double q = (i + 0.5) / kRings;
    const double r = std::sqrt(1.0 - std::pow(1.0 - q, 2.0 / (d - 2)));
    for (int j = 0; j < kAngles; ++j) {
      const double th = 2.0 * M_PI * (j + 0.5) / kAngles;
      pts.push_back({r * std::cos(th), r * std::sin(th)});
    }
  }
  std::vector<Pt> best;
  double best_mse = INFINITY;
  const double phases[2] = {0.0, 0.5};
  std::vector<int> cell(pts.size());
  for (double ph : phases) {
    std::vector<Pt> c(n_codes);
    for (int n = 0; n < n_codes; ++n) {
      const double r = std::sqrt(1.0 - std::pow(1.0 - (n + 0.5) / n_codes, 4.0 / d));
      const double th = ph * golden + n * golden;
      c[n] = {r * std::cos(th), r * std::sin(th)};
    }
    for (int it = 0; it < kLloydIters; ++it) {
      for (size_t i = 0; i < pts.size(); ++i) cell[i] = nearest_code(pts[i], c);
      std::vector<double> sx(n_codes, 0.0), sy(n_codes, 0.0);
      std::vector<int64_t> cnt(n_codes, 0);
      for (size_t i = 0; i < pts.size(); ++i) {
        sx[cell[i]] += pts[i].x;
        sy[cell[i]] += pts[i].y;
        ++cnt[cell[i]];
      }
      for (int n = 0; n < n_codes; ++n)
        if (cnt[n] > 0) c[n] = {sx[n] / cnt[n], sy[n] / cnt[n]};
    }
    const double m = code_mse(pts, c);
    if (m < best_mse * (1.0 - kRestartMargin)) {
      best_mse = m;
      best = c;
    }
  }
  for (int n = 0; n < n_codes; ++n) {
    codewords[2 * n] = best[n].x;
    codewords[2 * n + 1] = best[n].y;
  }
  return TQ_OK;
}

extern "C" int tq_vq_codec_init(tq_vq_codec* codec, int d, int n_codes, const uint32_t* flip) {
  if (codec == nullptr || flip == nullptr) return TQ_ERR_INVALID_ARG;
  if (d <= 0 || d > TQ_MAX_D || d % 2) return TQ_ERR_INVALID_ARG;
  std::vector<double> cw(2 * (size_t)(n_codes > 0 ? n_codes : 1));
  const int st = tq_build_vq_codebook(d, n_codes, cw.data());
  if (st != TQ_OK) return st;
  *codec = tq_vq_codec{};
  codec->d = d;
  codec->n_codes = n_codes;
  int b = 0;
  while ((1 << b) < n_codes) ++b;
  codec->block_bits = b;
  for (int n = 0; n < 2 * n_codes; ++n) codec->codewords[n] = (float)cw[n];
  const int words = (d + 31) / 32;
  for (int w = 0; w < words; ++w) {
    uint32_t m = flip[w];
    if (w == words - 1 && d % 32) m &= (1u << (d % 32)) - 1u;
    codec->flip[w] = m;
  }
  return TQ_OK;
}
