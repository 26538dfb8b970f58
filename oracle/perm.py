"""fp64 token-by-token oracle of the delta rule with partial-permutation
transitions (the SFDA bounded-stack family).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP path.

The recurrence is the one of oracle/seq.py (state S in R^{d_v x d_k}, rows =
value channels, columns = key channels) with the key-axis transition D_t a 0/1
column-selection matrix given by a source map src_t:

    (S D_t)[:, j] = S[:, src_t[j]]   if 0 <= src_t[j] < d_k, else 0
    S_t = X_t + beta_t (w_t v_t - X_t k_t) k_t^T,   X_t = S_{t-1} D_t
    o_t = S_t q_t

An injective src_t is a partial permutation: channels move, and channels that
no source reaches start from zero.

Source: SFDA technical summary, "finite-state expressivity": the
kernel-compatible family with partial permutations in place of the phase
blocks realises a bounded stack (and with the delta correction, registers).
The page gives the family, not a construction; the stack used by the tests
(push = shift every cell one channel deeper, dropping the deepest, then write
the new top at channel 0; pop = shift one channel up; top = read channel 0) is
this module's reading of it.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def select_columns(S: np.ndarray, src: np.ndarray) -> np.ndarray:
    """X = S D for states S [..., d_v, d_k] and source maps src [..., d_k]
    (integers; values outside [0, d_k) give a zero column)."""
    dk = S.shape[-1]
    src = np.asarray(src)
    ok = (src >= 0) & (src < dk)
    idx = np.where(ok, src, 0)
    X = np.take_along_axis(S, np.broadcast_to(idx[..., None, :], S.shape), axis=-1)
    return np.where(ok[..., None, :], X, 0.0)


def forward(q, k, v, w, src, beta, S0=None):
    """q, k [B,T,H,d_k], v [B,T,H,d_v], w, beta [B,T,H], src [B,T,H,d_k] int,
    S0 [B,H,d_v,d_k] or None.  Returns (o [B,T,H,d_v], S_T [B,H,d_v,d_k])."""
    q, k, v, w, beta = map(_f64, (q, k, v, w, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        X = select_columns(S, src[:, t])
        y = np.einsum("bhvk,bhk->bhv", X, k[:, t])
        err = w[:, t][..., None] * v[:, t] - y
        S = X + beta[:, t][..., None, None] * err[..., :, None] * k[:, t][..., None, :]
        o[:, t] = np.einsum("bhvk,bhk->bhv", S, q[:, t])
    return o, S
