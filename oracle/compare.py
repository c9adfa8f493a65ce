"""Error metrics for comparing a result with the oracle. TEST INFRASTRUCTURE.

Per (batch, head) slice, the normwise infinity relative error
max_i |x_i - ref_i| / max_i |ref_i|. A per-element relative error is not used
for ``out`` or ``M``: their entries cross zero, where it is meaningless. ``z``
is positive everywhere, so its per-element relative error is meaningful and
equals the normwise one's worst case; callers pick ``elementwise=True`` for it.
"""

import numpy as np


def max_rel_err(x, ref, elementwise=False):
    """Normwise (or elementwise) relative error of one slice, ignoring NaN refs."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    keep = ~np.isnan(ref)
    if not keep.any():
        return 0.0
    x, ref = x[keep], ref[keep]
    if not np.all(np.isfinite(x)):
        return float("inf")
    err = np.abs(x - ref)
    if elementwise:
        return float(np.max(err / np.abs(ref)))
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(err))
    return float(np.max(err) / scale)


def slice_errors(x, ref, elementwise=False):
    """Worst relative error over the leading (batch, head) slices of a tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            worst = max(worst, max_rel_err(x[b, h], ref[b, h], elementwise))
    return worst
