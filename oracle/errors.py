"""Error measure for comparing a computed tensor with the fp64 oracle.

The acceptance measure is a max-normalised error: max |x - r| / max |r| over
one output tensor (o or the final state), x upcast to float64.  An
element-wise relative error is meaningless where the reference is near zero,
so the denominator is the tensor's largest magnitude.
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
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(x - ref)))
    if den == 0.0:
        return num
    return num / den


def rel_fro(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(x - ref)) / (den if den else 1.0)
