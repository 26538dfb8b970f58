"""fp64 token-by-token oracle of the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP path.

The recurrence (one head, state S in R^{d_v x d_k}, row i = value channel i,
column j = key channel j, so that S k ~ v):

    X_t = S_{t-1} D_t                                  (key-axis transition)
    S_t = X_t (I - beta_t k_t k_t^T) + w_t beta_t v_t k_t^T
        = X_t + beta_t (w_t v_t - X_t k_t) k_t^T
    o_t = S_t q_t

Sources (pages, not code):
  * CARVE technical summary, section 1 (fixed-size matrix state with d_v rows
    and d_k columns), section 2.2 (one scalar write gate per head and token),
    section 2.3 (the decay acts on the key axis only).
  * SFDA technical summary, "core architecture": the delta update with the
    transition applied before the rank-one erase, and the real form of the
    phase-decay diag(alpha e^{i theta}) as a direct sum of 2x2 rotation-decay
    blocks.  In this module's orientation that update is the transpose of the
    page's (its state is d_k x d_v with the transition on the left).
  * CARVE technical summary, section 2.1 (content-aware erase): the erase gate
    of chunk c is sigmoid(b_x + U_b m_c) with m_c the mean of the previous
    chunk's outputs; the limitations paragraph: no signal exists before the
    second chunk.

Readings taken where the pages leave a step open:
  * output after the update, o_t = S_t q_t (the SFDA/KDA convention);
  * beta scales both the erase and the write;
  * 2x2 blocks act on adjacent key channels (2j, 2j+1); the block for angle
    theta and magnitude gamma is gamma [[cos, -sin], [sin, cos]], applied on
    the right (S D);
  * content-aware: U_b is per head and factorised as a_h^T B_h with
    B_h in R^{r x d_v}, a_h in R^r; m_c is the mean over the previous ``chunk``
    tokens of this call's own outputs; the first chunk uses the carried mean
    (zero when none is given).

Everything is computed in float64 with numpy; loops run over tokens only.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def transition(S: np.ndarray, decay: str, alpha_t: np.ndarray,
               theta_t: Optional[np.ndarray]) -> np.ndarray:
    """X = S D_t for states S [..., d_v, d_k].

    diag: D_t = Diag(alpha_t), alpha_t [..., d_k]  (CARVE 2.3: key-axis decay).
    rot2: D_t = direct sum over j of gamma_j [[c_j, -s_j], [s_j, c_j]] on key
          channels (2j, 2j+1), gamma = alpha_t [..., d_k/2], c/s of theta_t
          (SFDA core architecture: 2x2 rotation-decay blocks).
    dihedral: as rot2, except that a block whose gamma has its sign bit set is
          the reflection |gamma| [[c, s], [s, -c]] = |gamma| R(theta) F with
          F = Diag(1, -1) (SFDA finite-state expressivity: with reflections
          the family realises dihedral phase-orientation memory).  Products
          of such blocks do not commute.
    """
    if decay == "diag":
        return S * alpha_t[..., None, :]
    if decay not in ("rot2", "dihedral"):
        raise ValueError(decay)
    c = np.cos(theta_t)[..., None, :]
    s = np.sin(theta_t)[..., None, :]
    g = np.abs(alpha_t)[..., None, :] if decay == "dihedral" else alpha_t[..., None, :]
    even = S[..., 0::2]
    odd = S[..., 1::2]
    X = np.empty_like(S)
    # (S D)[:, 2j]   = S[:, 2j] D[2j, 2j]   + S[:, 2j+1] D[2j+1, 2j]
    # (S D)[:, 2j+1] = S[:, 2j] D[2j, 2j+1] + S[:, 2j+1] D[2j+1, 2j+1]
    X[..., 0::2] = g * (c * even + s * odd)
    X[..., 1::2] = g * (-s * even + c * odd)
    if decay == "dihedral":
        refl = np.signbit(alpha_t)[..., None, :]
        X[..., 1::2] = np.where(refl, g * (s * even - c * odd), X[..., 1::2])
    return X


def delta_step(S, q_t, k_t, v_t, beta_t, w_t, alpha_t, theta_t=None, decay="diag"):
    """One token of the recurrence for a batch of states.

    S [..., d_v, d_k]; q_t, k_t [..., d_k]; v_t [..., d_v]; beta_t, w_t [...].
    Returns (S_t, o_t).
    """
    X = transition(S, decay, alpha_t, theta_t)
    y = np.matmul(X, k_t[..., :, None])[..., 0]                      # X k
    err = w_t[..., None] * v_t - y                                     # w v - X k
    S_new = X + beta_t[..., None, None] * err[..., :, None] * k_t[..., None, :]
    o = np.matmul(S_new, q_t[..., :, None])[..., 0]                    # S_t q_t
    return S_new, o


def forward(q, k, v, w, alpha, beta=None, theta=None, decay="diag", S0=None,
            beta_logit=None, ub_down=None, ub_up=None, chunk=None, m_carry=None,
            return_m=False):
    """Sequential fp64 forward over [B,T,H,...] inputs.

    Returns o [B,T,H,d_v] and S_T [B,H,d_v,d_k] (and the last chunk mean when
    ``return_m`` is set, for content-aware resume).
    """
    q, k, v, w, alpha = map(_f64, (q, k, v, w, alpha))
    beta, theta, S0 = _f64(beta), _f64(theta), _f64(S0)
    content = beta_logit is not None
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else S0.copy()
    o = np.empty((B, T, H, dv))
    if content:
        if chunk is None or chunk < 1:
            raise ValueError("content-aware erase needs the chunk length")
        bx = _f64(beta_logit)
        Bh = _f64(ub_down)                 # [H, r, dv]
        ah = _f64(ub_up)                   # [H, r]
        m = np.zeros((B, H, dv)) if m_carry is None else _f64(m_carry).copy()
        s_c = None
    for t in range(T):
        if content:
            if t % chunk == 0:
                if t >= chunk:
                    m = o[:, t - chunk:t].mean(axis=1)                  # [B,H,dv]
                proj = np.einsum("hrv,bhv->bhr", Bh, m)                  # B_h m
                s_c = np.einsum("hr,bhr->bh", ah, proj)                  # a_h^T (B_h m)
            beta_t = sigmoid(bx[:, t] + s_c)
        else:
            beta_t = beta[:, t]
        th = theta[:, t] if theta is not None else None
        S, o[:, t] = delta_step(S, q[:, t], k[:, t], v[:, t], beta_t, w[:, t],
                                alpha[:, t], th, decay)
    if content and return_m:
        if T % chunk == 0 and T >= chunk:
            m = o[:, T - chunk:T].mean(axis=1)
        return o, S, m
    return o, S


def decode_step(S, q, k, v, beta, w, alpha, theta=None, decay="diag"):
    """One token for N independent states [N,H,d_v,d_k]; returns (S', o)."""
    return delta_step(_f64(S), _f64(q), _f64(k), _f64(v), _f64(beta), _f64(w),
                      _f64(alpha), _f64(theta), decay)


# ----------------------------------------------------------------------------
# Gate activation and q/k normalisation inside the forward (CARVE technical
# summary, section 2.3: the decay activation is computed where it is used).
# ----------------------------------------------------------------------------
L2NORM_EPS = 1e-6   # q / sqrt(sum q^2 + eps): the pages give no epsilon; a reading


def softplus(x):
    """log(1 + e^x) in a form that neither overflows nor loses small values."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gated_decay(x, a):
    """Decay from its pre-activation: exp(-a_h softplus(x)), a_h per head.

    x [..., H, C] (C = d_k, or d_k/2 block magnitudes); a [H] with a_h >= 0."""
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    return np.exp(-a[:, None] * softplus(x))


def l2_normalise(x, eps=L2NORM_EPS):
    """x / sqrt(sum x^2 + eps) over the last axis (one token of one head)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def forward_gated(q_raw, k_raw, v, w, x, a, beta, theta=None, decay="diag", S0=None,
                  qk_l2norm=True):
    """The forward with the decay given as a pre-activation and, optionally, raw q
    and k normalised per token: forward(l2(q), l2(k), v, w, exp(-a softplus(x)))."""
    q = l2_normalise(q_raw) if qk_l2norm else _f64(q_raw)
    k = l2_normalise(k_raw) if qk_l2norm else _f64(k_raw)
    return forward(q, k, v, w, gated_decay(x, a), beta=beta, theta=theta, decay=decay, S0=S0)
