"""ROOT-style soft-threshold split M = B + O, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[ROOT], "technical innovations of ROOT": the gradient is split into a robust
part B and an outlier part O with an l1 penalty on O, and only B is
orthogonalized.  The outlier part is the soft-threshold (l1 proximal step)
of M:

    O = sign(M) * max(|M| - lambda, 0),    B = M - O = clip(M, -lambda, lambda)

with lambda = 3 * median(|M|) (the heavy-tailed workload's definition).

Readings:

* the objective as printed has no factor 1/2 in front of the squared norm,
  which would make the literal threshold lambda/2; the split above (the
  usual proximal form, threshold lambda) is the one the workload defines;
* "median" of an even count: the lower median, the ceil(N/2)-th smallest
  |M| (1-based), taken over the stored values exactly.
"""

from __future__ import annotations

import numpy as np


def lower_median_abs(m: np.ndarray) -> float:
    """The ceil(N/2)-th smallest |m| (1-based) over all entries."""
    a = np.abs(np.asarray(m, dtype=np.float64)).ravel()
    if a.size == 0:
        raise ValueError("median of an empty matrix")
    k = (a.size + 1) // 2          # 1-based rank of the lower median
    return float(np.partition(a, k - 1)[k - 1])


def soft_threshold_split(m: np.ndarray, lam: float = None,
                         mult: float = 3.0):
    """Split m into (B, O, lambda) with O the soft-threshold of m.

    ``lam`` given: use it.  Otherwise lambda = mult * lower_median_abs(m).
    B = clip(m, -lambda, lambda) and O = sign(m) max(|m| - lambda, 0), both
    fp64; B + O equals m up to one fp64 rounding.
    """
    x = np.asarray(m, dtype=np.float64)
    if lam is None:
        lam = mult * lower_median_abs(x)
    lam = float(lam)
    o = np.sign(x) * np.maximum(np.abs(x) - lam, 0.0)
    b = np.clip(x, -lam, lam)
    return b, o, lam
