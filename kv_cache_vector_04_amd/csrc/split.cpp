// Outlier channel order for the split codec (host).
//
// "Google presenta TurboQuant", "Desempeño teórico y empírico": the outlier
// channels of a vector get more bits than the rest.  Which channels are the
// outliers is not stated there; here they are the d_hi channels of largest
// mean square over a calibration sample, ties to the lower channel index.
// The order lists them first and then the rest, each group ascending: the
// permutation a model applies once to the projection weights that produce
// K, V and the queries, so that the split codec's hi half sees them.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "tq.h"

extern "C" int tq_outlier_order(const float* x, int64_t n_rows, int d, int d_hi, int32_t* order) {
  if (x == nullptr || order == nullptr || n_rows <= 0 || d <= 0 || d_hi < 0 || d_hi > d)
    return TQ_ERR_INVALID_ARG;
  std::vector<double> ms(d, 0.0);
  for (int64_t r = 0; r < n_rows; ++r)
    for (int c = 0; c < d; ++c) {
      const double v = x[r * d + c];
      ms[c] += v * v;
    }
  // an inf or NaN sample has no defined order (and would break the sort)
  for (int c = 0; c < d; ++c)
    if (!std::isfinite(ms[c])) return TQ_ERR_INVALID_ARG;
  std::vector<int32_t> idx(d);
  std::iota(idx.begin(), idx.end(), 0);
  // larger mean square first; equal ones keep ascending channel order
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return ms[a] > ms[b]; });
  std::sort(idx.begin(), idx.begin() + d_hi);
  std::sort(idx.begin() + d_hi, idx.end());
  std::copy(idx.begin(), idx.end(), order);
  return TQ_OK;
}
