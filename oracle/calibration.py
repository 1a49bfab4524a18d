"""Oracle for the BLASST threshold calibration (test infrastructure only).

Follows the BLASST notes, section 3.2 (inverse relation between the best
threshold and the context length, lambda = a / L) and its Algorithm 2 (the
calibration procedure): for every context length, the threshold of a given
set whose measured sparsity lies closest to the target is kept if it lies
within the tolerance; a line through the origin is then fitted to the kept
points (1 / L, lambda_best), and its slope is a.

Readings (the pages are silent):

1. Ties between thresholds of equal distance keep the first one of the set,
   in the set's order (the comparison in the procedure is strict).
2. "Within the tolerance" is a strict comparison as printed (gap < delta).
3. The regression is a least-squares line through the origin, since the
   calibration function has no intercept: a = sum(x * y) / sum(x * x) with
   x = 1 / L and y = lambda_best.
4. With no point kept the procedure has nothing to fit; the oracle returns
   None and the number of points, 0.

Sparsity is the fraction of visited key blocks that the rule skips.  The
oracle takes the measured sparsities as a table (it does not run attention);
tests fill that table from the attention oracle's skip sets.
"""

from __future__ import annotations

import numpy as np


def best_threshold(lambdas, sparsities, target: float):
    """The threshold whose sparsity lies closest to the target, and its gap.

    Walks the set in order and keeps a threshold only when its gap is strictly
    smaller than the best so far (Algorithm 2, inner loop)."""
    best, min_gap = None, float("inf")
    for lam, s in zip(lambdas, sparsities):
        gap = abs(float(s) - float(target))
        if gap < min_gap:
            best, min_gap = float(lam), gap
    return best, min_gap


def calibrate(target: float, lengths, lambdas, sparsity_table, delta: float):
    """Algorithm 2 on a measured table.

    sparsity_table[k][i] is the sparsity measured at context length
    lengths[k] with threshold lambdas[i].  Returns (a, points) where points
    is the list of kept (1 / L, lambda_best) pairs and a is the slope of the
    least-squares line through the origin (None without points)."""
    points = []
    for L, row in zip(lengths, sparsity_table):
        lam_best, min_gap = best_threshold(lambdas, row, target)
        if lam_best is not None and min_gap < delta:
            points.append((1.0 / float(L), lam_best))
    if not points:
        return None, points
    x = np.array([p[0] for p in points], dtype=np.float64)
    y = np.array([p[1] for p in points], dtype=np.float64)
    return float((x * y).sum() / (x * x).sum()), points


def block_sparsity(skip_sets) -> float:
    """Fraction of visited blocks skipped, over a collection of skip arrays."""
    skipped = sum(int(np.count_nonzero(s)) for s in skip_sets)
    visited = sum(int(np.size(s)) for s in skip_sets)
    return skipped / visited if visited else 0.0
