"""fp64 chunk-parallel (WY-form) reference of the gated delta-rule forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/seq.py``): used to pin the chunked
algebra against the token-by-token definition by brute force, and to expose
per-chunk intermediates.  It shares no code with the HIP path.

For one head and one chunk of n tokens (r = 1..n) starting from state S0,
with key-axis transitions D_r (d_k x d_k) and their running products
Gamma_r = D_1 ... D_r, the state after token r is

    S_r = S0 Gamma_r + sum_{i<=r} delta_i k_i^T Gamma_i^{-1} Gamma_r

(the product telescopes; no commutation is needed).  With the decayed forms

    K+_r = Gamma_r k_r,   Q+_r = Gamma_r q_r,   Kh_i = Gamma_i^{-T} k_i,
    K-_i = Gamma_n^T Kh_i

the per-token corrections delta solve one unit-lower-triangular system shared
by every value row (the WY form: CARVE technical summary, section 1.3 and
section 3 item 1 -- key-axis-only gating keeps one L x L system per chunk):

    A   = strict_lower(diag(beta) K+ Kh^T)
    Tm  = (I + A)^{-1}
    W   = Tm diag(beta) K+,      U = Tm diag(beta w) V
    Dlt = U - W S0^T                                   (rows = delta_r^T)
    O   = Q+ S0^T + lower_incl(Q+ Kh^T) Dlt
    S_n = S0 Gamma_n + Dlt^T K-

The last line is the exact affine chunk transfer S_n = S0 P + B with
P = Gamma_n - W^T K- and B = U^T K- (SFDA technical summary, main
contributions: the chunk write summary comes from the zero-initial-state
recursion; constructive chunk-WY theorem: the correction's rank grows only
inside a chunk).

Dense d_k x d_k matrices are used for Gamma so that the same code covers the
diagonal and the 2x2 rotation-decay transitions.  Sizes are meant to be tiny.
"""
from __future__ import annotations

import numpy as np

from . import seq


def transition_matrix(decay, alpha_t, theta_t, dk):
    """Dense D_t (d_k x d_k) such that seq.transition(S) == S @ D_t."""
    if decay == "diag":
        return np.diag(np.asarray(alpha_t, np.float64))
    theta_t = np.asarray(theta_t, np.float64)
    alpha_t = np.asarray(alpha_t, np.float64)
    D = np.zeros((dk, dk))
    for j in range(dk // 2):
        c, s, g = np.cos(theta_t[j]), np.sin(theta_t[j]), alpha_t[j]
        if decay == "dihedral" and np.signbit(g):   # reflection |g| R(theta) F, F = Diag(1, -1)
            g = -g
            D[2 * j, 2 * j] = g * c
            D[2 * j, 2 * j + 1] = g * s
            D[2 * j + 1, 2 * j] = g * s
            D[2 * j + 1, 2 * j + 1] = -g * c
            continue
        D[2 * j, 2 * j] = g * c
        D[2 * j, 2 * j + 1] = -g * s
        D[2 * j + 1, 2 * j] = g * s
        D[2 * j + 1, 2 * j + 1] = g * c
    return D


def chunk_head(q, k, v, w, alpha, beta, theta=None, decay="diag", S0=None,
               chunk=16, keep=False, beta_fn=None):
    """One head: q,k [T,dk], v [T,dv], w,beta [T], alpha [T,dk|dk/2].

    ``beta_fn(c, O_prev)`` (content-aware) returns the chunk's beta [n] from
    the previous chunk's outputs (None for chunk 0).  Returns (o, S_T, stages).
    """
    q, k, v, w, alpha = (np.asarray(x, np.float64) for x in (q, k, v, w, alpha))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.empty((T, dv))
    stages = []
    O_prev = None
    for ci, c0 in enumerate(range(0, T, chunk)):
        idx = np.arange(c0, min(c0 + chunk, T))
        n = len(idx)
        if beta_fn is not None:
            b = np.asarray(beta_fn(ci, O_prev), np.float64)
        else:
            b = np.asarray(beta, np.float64)[idx]
        Gam = []
        G = np.eye(dk)
        for t in idx:
            th = None if theta is None else np.asarray(theta[t], np.float64)
            G = G @ transition_matrix(decay, alpha[t], th, dk)
            Gam.append(G)
        Kp = np.stack([Gam[r] @ k[idx[r]] for r in range(n)])
        Qp = np.stack([Gam[r] @ q[idx[r]] for r in range(n)])
        Kh = np.stack([np.linalg.solve(Gam[r].T, k[idx[r]]) for r in range(n)])
        GL = Gam[-1]
        Km = Kh @ GL                                    # rows: (GL^T Kh_i)^T
        A = np.tril(b[:, None] * (Kp @ Kh.T), -1)
        Mqk = np.tril(Qp @ Kh.T)
        Tm = np.linalg.inv(np.eye(n) + A)
        W = Tm @ (b[:, None] * Kp)
        U = Tm @ ((b * w[idx])[:, None] * v[idx])
        Dlt = U - W @ S.T
        O = Qp @ S.T + Mqk @ Dlt
        if keep:
            stages.append(dict(S_start=S.copy(), Kp=Kp, Qp=Qp, Kh=Kh, Km=Km, A=A,
                               Mqk=Mqk, T=Tm, W=W, U=U, Delta=Dlt, O=O, GL=GL,
                               beta=b))
        S = S @ GL + Dlt.T @ Km
        o[idx] = O
        O_prev = O
    return o, S, stages


def forward(q, k, v, w, alpha, beta=None, theta=None, decay="diag", S0=None,
            chunk=16, beta_logit=None, ub_down=None, ub_up=None, m_carry=None):
    """Chunked forward over [B,T,H,...] inputs, head by head (tiny sizes)."""
    q = np.asarray(q, np.float64)
    B, T, H, dk = q.shape
    dv = np.shape(v)[-1]
    o = np.empty((B, T, H, dv))
    S_out = np.empty((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            beta_fn = None
            if beta_logit is not None:
                Bh = np.asarray(ub_down, np.float64)[h]
                ah = np.asarray(ub_up, np.float64)[h]
                bx = np.asarray(beta_logit, np.float64)[b, :, h]
                m0 = (np.zeros(dv) if m_carry is None
                      else np.asarray(m_carry, np.float64)[b, h])

                def beta_fn(ci, O_prev, Bh=Bh, ah=ah, bx=bx, m0=m0):
                    m = m0 if O_prev is None else O_prev.mean(axis=0)
                    s_c = ah @ (Bh @ m)
                    lo = ci * chunk
                    return seq.sigmoid(bx[lo:lo + chunk] + s_c)
            o[b, :, h], S_out[b, h], _ = chunk_head(
                q[b, :, h], np.asarray(k)[b, :, h], np.asarray(v)[b, :, h],
                np.asarray(w)[b, :, h], np.asarray(alpha)[b, :, h],
                None if beta is None else np.asarray(beta)[b, :, h],
                None if theta is None else np.asarray(theta)[b, :, h],
                decay, None if S0 is None else np.asarray(S0)[b, h], chunk,
                beta_fn=beta_fn)
    return o, S_out
