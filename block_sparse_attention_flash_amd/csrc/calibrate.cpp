// Host-side threshold calibration of the BLASST notes (section 3.2 and
// Algorithm 2): the best threshold follows lambda = a / L; per context
// length, pick from a threshold set the one whose measured sparsity is
// closest to the target, keep it when within the tolerance, then fit a line
// through the origin to the kept points (1 / L, lambda_best).
//
// The sparsities are measured by the caller with the attention kernels
// (fraction of visited blocks skipped); this file only selects and fits.

#include <cmath>
#include <cstdint>

#include "internal.h"

using namespace bsattn;

extern "C" {

bsattn_status bsattn_calibrate_threshold(double target, const int32_t* lengths, int32_t n_lengths,
                                         const double* lambdas, int32_t n_lambdas, const double* sparsity,
                                         double delta, double* a_out, int32_t* n_points_out) {
  clear_error();
  if (!lengths || !lambdas || !sparsity || !a_out || !n_points_out)
    return fail(BSATTN_ERR_INVALID_ARG, "lengths, lambdas, sparsity, a_out, n_points_out must be non-NULL");
  if (n_lengths < 1 || n_lambdas < 1) return fail(BSATTN_ERR_INVALID_ARG, "need at least one length and one lambda");
  if (!(target >= 0.0 && target <= 1.0)) return fail(BSATTN_ERR_INVALID_ARG, "target sparsity must lie in [0, 1]");
  if (!(delta > 0.0) || !std::isfinite(delta)) return fail(BSATTN_ERR_INVALID_ARG, "tolerance must be finite and > 0");
  for (int32_t k = 0; k < n_lengths; ++k)
    if (lengths[k] < 1) return fail(BSATTN_ERR_INVALID_ARG, "length %d is < 1", lengths[k]);
  for (int32_t i = 0; i < n_lambdas; ++i)
    if (!(lambdas[i] > 0.0 && lambdas[i] < 1.0))
      return fail(BSATTN_ERR_INVALID_ARG, "lambda[%d] must lie in (0, 1)", i);
  for (int64_t x = 0; x < (int64_t)n_lengths * n_lambdas; ++x)
    if (!(sparsity[x] >= 0.0 && sparsity[x] <= 1.0))
      return fail(BSATTN_ERR_INVALID_ARG, "sparsity entry %lld must lie in [0, 1]", (long long)x);

  double sxy = 0.0, sxx = 0.0;
  int32_t kept = 0;
  for (int32_t k = 0; k < n_lengths; ++k) {
    const double* row = sparsity + (int64_t)k * n_lambdas;
    double best = 0.0, min_gap = INFINITY;
    for (int32_t i = 0; i < n_lambdas; ++i) {  // strict: the first of equal gaps wins
      const double gap = std::fabs(row[i] - target);
      if (gap < min_gap) {
        min_gap = gap;
        best = lambdas[i];
      }
    }
    if (min_gap < delta) {  // strict, as printed
      const double x = 1.0 / (double)lengths[k];
      sxy += x * best;
      sxx += x * x;
      ++kept;
    }
  }
  *n_points_out = kept;
  *a_out = kept > 0 ? sxy / sxx : NAN;
  return BSATTN_OK;
}

}  // extern "C"
