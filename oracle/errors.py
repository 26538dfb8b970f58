"""Error measure for comparing a computed tensor with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/seq.py``).

The acceptance measure is a max-normalised error over one output tensor (o, or
the final state):

    err(x, r) = max_i |x_i - r_i| / max_i |r_i|

with x upcast to float64.  An element-wise relative error is meaningless
where the reference is near zero, so the denominator is the largest magnitude
in the reference tensor.  Conventions for the corner cases:

* shapes must match exactly (no broadcasting): ValueError otherwise;
* an empty tensor has error 0;
* any non-finite value in x or in r gives +inf (never passes a tolerance);
* an all-zero reference gives the absolute error max |x_i|.

Pinned by hand-computed cases in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import numpy as np


def max_rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    if not (np.all(np.isfinite(x)) and np.all(np.isfinite(ref))):
        return float("inf")
    num = float(np.max(np.abs(x - ref)))
    den = float(np.max(np.abs(ref)))
    if den == 0.0:
        return num
    return num / den
