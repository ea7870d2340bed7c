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

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
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
  *codec = tq_vq_codec{};   // search = NULL
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

// The nearest-codeword search table (layout in tq.h).  Each block
// coordinate is companded, u = x / (|x| + a), and the grid is uniform in u:
// cell i of an axis holds x in [x(u_i), x(u_i+1)) with u_i = 2 i / G - 1 and
// x(u) = a u / (1 - |u|), so cells are narrow where the codewords crowd
// (near 0) and the outermost ones reach the disk's edge (|x| <= 1).  The
// score of codeword c at a point p is s_c(p) = <p, c> - |c|^2 / 2; it is
// linear in p, so over a rectangle its extremes sit at the corners.  Every
// point of the widened cell has a best score of at least
// L = max_c min_corners s_c, so a codeword whose largest score on the cell is
// below L - slack can never be within slack of the best there: only the
// others are listed.  The slack (1e-5) covers the encoder's fp32 scores.
// Each cell edge is widened by 1e-5 plus 1e-6 dx/du at that edge: the
// encoder's fp32 u is within a few 1e-7 of the exact one, which moves an
// edge by that much times dx/du = a / (1 - |u|)^2 (large near |u| = 1).
namespace {

constexpr int kG = TQ_VQ_GRID;
constexpr int kCellCap = 48;              // a longer list: full search in that cell
constexpr int kOffsets = TQ_VQ_GRID * TQ_VQ_GRID + 8;

// edge i of an axis, moved outward by its widening (side -1: lower edge of
// a cell, +1: upper edge)
double cell_edge(double a, int i, int side) {
  const double u = 2.0 * i / kG - 1.0;
  if (i <= 0) return -1.001;
  if (i >= kG) return 1.001;
  const double x = a * u / (1.0 - std::fabs(u));
  const double dxdu = a / ((1.0 - std::fabs(u)) * (1.0 - std::fabs(u)));
  return std::max(-1.001, std::min(1.001, x + side * (1e-5 + 1e-6 * dxdu)));
}

// the candidate list of every cell for companding constant a
void fill_cells(double a, int n, const std::vector<double>& cx, const std::vector<double>& cy,
                const std::vector<double>& hq, std::vector<std::vector<uint8_t>>& cells) {
  constexpr double kSlack = 1e-5;
  std::vector<double> hi(n);
  cells.assign(kG * kG, {});
  for (int j = 0; j < kG; ++j)
    for (int i = 0; i < kG; ++i) {
      const double x0 = cell_edge(a, i, -1), x1 = cell_edge(a, i + 1, 1);
      const double y0 = cell_edge(a, j, -1), y1 = cell_edge(a, j + 1, 1);
      const double px[4] = {x0, x1, x0, x1}, py[4] = {y0, y0, y1, y1};
      double lo_best = -INFINITY;
      for (int k = 0; k < n; ++k) {
        double mn = INFINITY, mx = -INFINITY;
        for (int q = 0; q < 4; ++q) {
          const double sc = px[q] * cx[k] + py[q] * cy[k] + hq[k];
          mn = std::min(mn, sc);
          mx = std::max(mx, sc);
        }
        lo_best = std::max(lo_best, mn);
        hi[k] = mx;
      }
      std::vector<uint8_t>& lst = cells[j * kG + i];
      for (int k = 0; k < n; ++k)
        if (hi[k] >= lo_best - kSlack) lst.push_back((uint8_t)k);
      if ((int)lst.size() > kCellCap) lst.clear();      // empty: full search
    }
}

// lists longest first into full-search cells until the pool holds the rest
void fit_pool(std::vector<std::vector<uint8_t>>& cells) {
  size_t total = 0;
  for (const auto& l : cells) total += l.size();
  while (total > (size_t)TQ_VQ_ENTRIES) {
    size_t big = 0;
    for (size_t k = 1; k < cells.size(); ++k)
      if (cells[k].size() > cells[big].size()) big = k;
    total -= cells[big].size();
    cells[big].clear();
  }
}

int cell_of(double a, double x) {
  const double t = (x / (std::fabs(x) + a) + 1.0) * (kG / 2.0);
  return std::max(0, std::min(kG - 1, (int)std::floor(t)));
}

}  // namespace

extern "C" int tq_vq_search_build(const tq_vq_codec* c, void* table, size_t bytes) {
  if (c == nullptr || table == nullptr || bytes < (size_t)TQ_VQ_SEARCH_BYTES) return TQ_ERR_INVALID_ARG;
  const int n = c->n_codes, d = c->d;
  if (n < 2 || n > TQ_VQ_MAX_CODES || d < 6) return TQ_ERR_INVALID_ARG;
  std::vector<double> cx(n), cy(n), hq(n);
  for (int i = 0; i < n; ++i) {
    cx[i] = c->codewords[2 * i];
    cy[i] = c->codewords[2 * i + 1];
    hq[i] = -0.5 * (cx[i] * cx[i] + cy[i] * cy[i]);
  }
  // equal-weight points of the block density (rings at the Beta(1, (d-2)/2)
  // quantiles of |y|^2) to weigh the cells by how often blocks land there
  std::vector<double> qx, qy;
  for (int r = 0; r < 64; ++r) {
    const double rad = std::sqrt(1.0 - std::pow(1.0 - (r + 0.5) / 64.0, 2.0 / (d - 2)));
    for (int t = 0; t < 64; ++t) {
      const double th = 2.0 * M_PI * (t + 0.5) / 64.0;
      qx.push_back(rad * std::cos(th));
      qy.push_back(rad * std::sin(th));
    }
  }
  // the companding constant with the fewest expected codeword tests per
  // block (a full-search cell costs N), from multiples of the coordinate
  // scale 1 / sqrt(d)
  std::vector<std::vector<uint8_t>> cells;
  double best_a = 0.0, best_cost = INFINITY;
  for (int e = 0; e <= 12; ++e) {
    const double a = std::pow(2.0, 0.5 * e - 1.0) / std::sqrt((double)d);
    fill_cells(a, n, cx, cy, hq, cells);
    fit_pool(cells);
    double cost = 0.0;
    for (size_t p = 0; p < qx.size(); ++p) {
      const size_t k = cells[cell_of(a, qy[p]) * kG + cell_of(a, qx[p])].size();
      cost += k == 0 ? n : (double)k;
    }
    if (cost < best_cost) {
      best_cost = cost;
      best_a = a;
    }
  }
  fill_cells(best_a, n, cx, cy, hq, cells);
  fit_pool(cells);
  uint8_t* base = static_cast<uint8_t*>(table);
  std::fill(base, base + TQ_VQ_SEARCH_BYTES, (uint8_t)0);
  const float hdr_f[2] = {(float)best_a, (float)(kG / 2.0)};
  int32_t hdr_i[2] = {kG, 0};
  uint16_t* off = reinterpret_cast<uint16_t*>(base + 16);
  uint8_t* pool = base + 16 + 2 * kOffsets;
  int total = 0;
  for (int k = 0; k < kG * kG; ++k) {
    off[k] = (uint16_t)total;
    for (uint8_t v : cells[k]) pool[total++] = v;
  }
  for (int k = kG * kG; k < kOffsets; ++k) off[k] = (uint16_t)total;
  hdr_i[1] = total;
  std::memcpy(base, hdr_f, 8);
  std::memcpy(base + 8, hdr_i, 8);
  return TQ_OK;
}
