"""fp64 gradients of the gated delta-rule forward: reverse mode through the
token recurrence, and the same gradients from the chunk (WY) algebra.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests use it.  It shares no code with the HIP path.

The forward is ``oracle.seq.forward`` (plain erase), per token

    X_t = S_{t-1} D_t,   e_t = w_t v_t - X_t k_t,
    S_t = X_t + beta_t e_t k_t^T,   o_t = S_t q_t,

with D_t = Diag(alpha_t) or the 2x2 rotation-decay blocks
gamma [[cos, -sin], [sin, cos]] (SFDA technical summary, core architecture;
CARVE technical summary, section 2.3: every gate on the key axis).  The
published throughput is that of training (CARVE technical summary, results),
and section 3 item 5 (theorem 5) bounds the gradient norm; these functions give
the gradients that training needs, for a scalar loss
L = sum(dO * o) + sum(dS_T * S_T), with respect to q, k, v, w, beta, the
transition (alpha, or gamma and theta) and S_0.

``backward_seq`` walks the tokens backwards (the plain definition of reverse
mode; pinned by central finite differences in the tests).  ``backward_gated``
adds the chain rule through the gated forward's decay activation
exp(-a_h softplus(x)) and per-token q/k normalisation (``oracle.seq.forward_gated``;
also pinned by finite differences).  ``backward_chunk``
obtains the same gradients from the chunk form that a chunk-parallel kernel
evaluates: per chunk, the WY factors are rebuilt from the chunk's start state,
and the adjoint runs through those matrix expressions in reverse.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle import seq as _seq
from oracle.seq import transition


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _transition_adjoint(S_prev, dX, alpha_t, theta_t, decay):
    """Given X = S_prev D and dL/dX, return (dL/dS_prev, dL/dalpha, dL/dtheta)."""
    if decay == "diag":
        dS = dX * alpha_t[..., None, :]
        dalpha = np.sum(dX * S_prev, axis=-2)
        return dS, dalpha, None
    c = np.cos(theta_t)[..., None, :]
    s = np.sin(theta_t)[..., None, :]
    g = alpha_t[..., None, :]
    Se, So = S_prev[..., 0::2], S_prev[..., 1::2]
    dXe, dXo = dX[..., 0::2], dX[..., 1::2]
    # X_e = g (c Se + s So),  X_o = g (-s Se + c So)
    dS = np.empty_like(S_prev)
    dS[..., 0::2] = g * (c * dXe - s * dXo)
    dS[..., 1::2] = g * (s * dXe + c * dXo)
    dgamma = np.sum(dXe * (c * Se + s * So) + dXo * (-s * Se + c * So), axis=-2)
    # d/dtheta of (c, s) is (-s, c)
    dtheta = np.sum(g * (dXe * (-s * Se + c * So) + dXo * (-c * Se - s * So)), axis=-2)
    return dS, dgamma, dtheta


def backward_seq(q, k, v, w, alpha, beta, dO, dS_T=None, theta=None, decay="diag", S0=None):
    """Gradients of L = sum(dO o) + sum(dS_T S_T) by reverse mode over tokens.

    Shapes as in ``oracle.seq.forward`` ([B,T,H,...]); dO [B,T,H,d_v],
    dS_T [B,H,d_v,d_k] or None.  Returns a dict with dq, dk, dv, dw, dbeta,
    dalpha (d_k, or d_k/2 block magnitudes), dtheta (rot2) and dS0.
    """
    q, k, v, w, alpha, beta, dO = map(_f64, (q, k, v, w, alpha, beta, dO))
    theta, S0, dS_T = _f64(theta), _f64(S0), _f64(dS_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else S0.copy()
    # forward, keeping S_{t-1} and X_t of every token
    S_prev = np.empty((T, B, H, dv, dk))
    Xs = np.empty((T, B, H, dv, dk))
    for t in range(T):
        S_prev[t] = S
        th = None if theta is None else theta[:, t]
        X = transition(S, decay, alpha[:, t], th)
        e = w[:, t, :, None] * v[:, t] - np.matmul(X, k[:, t, :, :, None])[..., 0]
        S = X + beta[:, t, :, None, None] * e[..., :, None] * k[:, t, :, None, :]
        Xs[t] = X
    G = np.zeros((B, H, dv, dk)) if dS_T is None else dS_T.copy()
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dw", w),
                                              ("dbeta", beta), ("dalpha", alpha))}
    if theta is not None:
        out["dtheta"] = np.zeros_like(theta)
    for t in range(T - 1, -1, -1):
        X = Xs[t]
        kt, qt, vt = k[:, t], q[:, t], v[:, t]
        bt, wt = beta[:, t], w[:, t]
        e = wt[..., None] * vt - np.matmul(X, kt[..., :, None])[..., 0]
        S_t = X + bt[..., None, None] * e[..., :, None] * kt[..., None, :]
        # o_t = S_t q_t
        G = G + dO[:, t, :, :, None] * qt[..., None, :]
        out["dq"][:, t] = np.matmul(np.swapaxes(S_t, -1, -2), dO[:, t, :, :, None])[..., 0]
        # S_t = X + beta e k^T
        Gk = np.matmul(G, kt[..., :, None])[..., 0]                     # G k  [.., dv]
        out["dbeta"][:, t] = np.sum(e * Gk, axis=-1)
        de = bt[..., None] * Gk
        dk_t = bt[..., None] * np.matmul(np.swapaxes(G, -1, -2), e[..., :, None])[..., 0]
        # e = w v - X k
        out["dw"][:, t] = np.sum(de * vt, axis=-1)
        out["dv"][:, t] = wt[..., None] * de
        dX = G - de[..., :, None] * kt[..., None, :]
        dk_t = dk_t - np.matmul(np.swapaxes(X, -1, -2), de[..., :, None])[..., 0]
        out["dk"][:, t] = dk_t
        th = None if theta is None else theta[:, t]
        G, da, dth = _transition_adjoint(S_prev[t], dX, alpha[:, t], th, decay)
        out["dalpha"][:, t] = da
        if theta is not None:
            out["dtheta"][:, t] = dth
    out["dS0"] = G
    return out


# ----------------------------------------------------------------------------
# Chunk form.  For one chunk of L tokens with start state S (one head), let
# P_r = D_1 D_2 ... D_r (the chunk's transitions up to token r, as right
# factors: with no writes the state would be S P_r), and, as columns per token,
#     Kp_r = P_r k_r,   Qp_r = P_r q_r,   Kh_r = P_r^{-T} k_r.
# With delta vectors d_r = beta_r (w_r v_r - S_{r-1} D_r k_r) the recurrence
# unrolls to
#     S_r = (S + sum_{s<=r} d_s Kh_s^T) P_r,
# so the deltas (rows of Dl) solve the unit lower-triangular system
#     (I + Diag(beta) N) Dl = Diag(beta) (Diag(w) V - Kp S^T),
#     N_rs = Kp_r . Kh_s for s < r,
# and  O = Qp S^T + M Dl  with  M_rs = Qp_r . Kh_s for s <= r,
#      S_end = (S + Dl^T Kh) P_L.
# ----------------------------------------------------------------------------

def _chunk_mats(alpha_c, theta_c, decay, dk):
    """Cumulative transitions P_r = D_1 ... D_r (r = 1..L) of one chunk as dense
    [L, dk, dk] arrays (S P_r is S after r transitions), built by applying
    ``transition`` to the identity so that the convention is the oracle's own."""
    L = alpha_c.shape[0]
    P = np.empty((L, dk, dk))
    M = np.eye(dk)
    for r in range(L):
        th = None if theta_c is None else theta_c[r]
        M = transition(M, decay, alpha_c[r], th)   # M <- M D_r: rows act as states
        P[r] = M
    return P


def _forward_chunk_one(S, qc, kc, vc, wc, bc, P):
    """Chunk form for one head and one chunk: returns (O [L,dv], S_end, parts)."""
    L = qc.shape[0]
    Kp = np.einsum("rij,rj->ri", P, kc)                     # P_r k_r
    Qp = np.einsum("rij,rj->ri", P, qc)                     # P_r q_r
    Pinv = np.linalg.inv(P)
    Kh = np.einsum("rji,rj->ri", Pinv, kc)                  # P_r^{-T} k_r
    N = np.tril(Kp @ Kh.T, -1)                              # N_rs = Kp_r . Kh_s, s < r
    A = np.eye(L) + bc[:, None] * N
    R = bc[:, None] * (wc[:, None] * vc - Kp @ S.T)         # [L, dv]
    Dl = np.linalg.solve(A, R)                              # deltas, rows = tokens
    M = np.tril(Qp @ Kh.T)                                  # s <= r
    O = Qp @ S.T + M @ Dl
    S_end = (S + Dl.T @ Kh) @ P[-1]
    return O, S_end, dict(Kp=Kp, Qp=Qp, Kh=Kh, Pinv=Pinv, N=N, A=A, R=R, Dl=Dl, M=M)


def forward_chunk(q, k, v, w, alpha, beta, theta=None, decay="diag", S0=None, chunk=16):
    """The forward in chunk form (fp64, dense matrices): same result as
    ``oracle.seq.forward`` up to rounding."""
    q, k, v, w, alpha, beta = map(_f64, (q, k, v, w, alpha, beta))
    theta, S0 = _f64(theta), _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    O = np.empty((B, T, H, dv))
    S_out = np.empty((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else S0[b, h].copy()
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                P = _chunk_mats(alpha[b, c0:c1, h], None if theta is None else theta[b, c0:c1, h],
                                decay, dk)
                Oc, S, _ = _forward_chunk_one(S, q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h],
                                              w[b, c0:c1, h], beta[b, c0:c1, h], P)
                O[b, c0:c1, h] = Oc
            S_out[b, h] = S
    return O, S_out


def _dP_to_transition(dP, P, alpha_c, theta_c, decay):
    """Pull a gradient on the cumulative products P_r (r = 1..L) back to the
    per-token transitions: P_r = P_{r-1} D_r as right factors."""
    L = P.shape[0]
    dk = P.shape[1]
    da = np.zeros_like(alpha_c)
    dth = None if theta_c is None else np.zeros_like(theta_c)
    G = np.zeros((dk, dk))
    for r in range(L - 1, -1, -1):
        G = G + dP[r]
        Pprev = np.eye(dk) if r == 0 else P[r - 1]
        th = None if theta_c is None else theta_c[r]
        G, dar, dthr = _transition_adjoint(Pprev, G, alpha_c[r], th, decay)
        da[r] = dar
        if theta_c is not None:
            dth[r] = dthr
    return da, dth


def backward_chunk(q, k, v, w, alpha, beta, dO, dS_T=None, theta=None, decay="diag", S0=None,
                   chunk=16):
    """The gradients of ``backward_seq`` from the chunk form: chunk start states
    from a forward pass, then chunks in reverse, each rebuilding its WY factors
    and running the adjoint of its matrix expressions."""
    q, k, v, w, alpha, beta, dO = map(_f64, (q, k, v, w, alpha, beta, dO))
    theta, S0, dS_T = _f64(theta), _f64(S0), _f64(dS_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dw", w),
                                              ("dbeta", beta), ("dalpha", alpha))}
    if theta is not None:
        out["dtheta"] = np.zeros_like(theta)
    out["dS0"] = np.zeros((B, H, dv, dk))
    starts = list(range(0, T, chunk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else S0[b, h].copy()
            S_start, Ps = [], []
            for c0 in starts:
                c1 = min(T, c0 + chunk)
                P = _chunk_mats(alpha[b, c0:c1, h], None if theta is None else theta[b, c0:c1, h],
                                decay, dk)
                S_start.append(S)
                Ps.append(P)
                _, S, _ = _forward_chunk_one(S, q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h],
                                             w[b, c0:c1, h], beta[b, c0:c1, h], P)
            G = np.zeros((dv, dk)) if dS_T is None else dS_T[b, h].copy()   # dL/dS_end
            for ci in range(len(starts) - 1, -1, -1):
                c0 = starts[ci]
                c1 = min(T, c0 + chunk)
                sl = slice(c0, c1)
                qc, kc, vc = q[b, sl, h], k[b, sl, h], v[b, sl, h]
                wc, bc = w[b, sl, h], beta[b, sl, h]
                S, P = S_start[ci], Ps[ci]
                _, _, f = _forward_chunk_one(S, qc, kc, vc, wc, bc, P)
                Kp, Qp, Kh, Pinv, A, R, Dl, M = (f[n] for n in ("Kp", "Qp", "Kh", "Pinv", "A", "R",
                                                                "Dl", "M"))
                dOc = dO[b, sl, h]
                PL = P[-1]
                # S_end = (S + Dl^T Kh) PL  and  O = Qp S^T + M Dl
                Y = S + Dl.T @ Kh
                dY = G @ PL.T
                dPL = Y.T @ G
                dS = dY + dOc.T @ Qp
                dQp = dOc @ S
                dM = np.tril(dOc @ Dl.T)
                dDl = M.T @ dOc + Kh @ dY.T
                dKh = Dl @ dY
                # M = tril(Qp Kh^T)
                dQp = dQp + dM @ Kh
                dKh = dKh + dM.T @ Qp
                # Dl = A^{-1} R
                dR = np.linalg.solve(A.T, dDl)
                dA = -dR @ Dl.T
                # A = I + Diag(b) tril(Kp Kh^T, -1)
                Nfull = Kp @ Kh.T
                dN = np.tril(bc[:, None] * dA, -1)
                dbc = np.sum(np.tril(dA, -1) * np.tril(Nfull, -1), axis=1)
                dKp = dN @ Kh
                dKh = dKh + dN.T @ Kp
                # R = Diag(b) (Diag(w) V - Kp S^T)
                inner = wc[:, None] * vc - Kp @ S.T
                dbc = dbc + np.sum(dR * inner, axis=1)
                dinner = bc[:, None] * dR
                dwc = np.sum(dinner * vc, axis=1)
                dvc = wc[:, None] * dinner
                dKp = dKp - dinner @ S
                dS = dS - dinner.T @ Kp
                # Kp_r = P_r k_r, Qp_r = P_r q_r, Kh_r = P_r^{-T} k_r
                dkc = np.einsum("rij,ri->rj", P, dKp) + np.einsum("rji,ri->rj", Pinv, dKh)
                dqc = np.einsum("rij,ri->rj", P, dQp)
                dP = np.einsum("ri,rj->rij", dKp, kc) + np.einsum("ri,rj->rij", dQp, qc)
                # Kh_r = Pinv_r^T k_r: dPinv_r = k_r dKh_r^T; dP = -P^{-T} dPinv P^{-T}
                dPinv = np.einsum("rj,ri->rji", kc, dKh)
                dP = dP - np.einsum("rji,rjk,rlk->ril", Pinv, dPinv, Pinv)   # -P^-T dPinv P^-T
                dP[-1] = dP[-1] + dPL
                da, dth = _dP_to_transition(dP, P, alpha[b, sl, h],
                                            None if theta is None else theta[b, sl, h], decay)
                out["dq"][b, sl, h] = dqc
                out["dk"][b, sl, h] = dkc
                out["dv"][b, sl, h] = dvc
                out["dw"][b, sl, h] = dwc
                out["dbeta"][b, sl, h] = dbc
                out["dalpha"][b, sl, h] = da
                if theta is not None:
                    out["dtheta"][b, sl, h] = dth
                G = dS
            out["dS0"][b, h] = G
    return out


def backward_gated(q_raw, k_raw, v, w, x, a, beta, dO, dS_T=None, theta=None, decay="diag",
                   S0=None, qk_l2norm=True):
    """Gradients of ``oracle.seq.forward_gated`` for the same scalar loss.

    The forward is ``forward(l2(q_raw), l2(k_raw), v, w, exp(-a_h softplus(x)))``
    (CARVE technical summary, section 2.3: the decay activation computed where
    it is used), with l2(y) = y / sqrt(sum y^2 + eps) per token when
    ``qk_l2norm``.  Its gradients are ``backward_seq``'s at the activated,
    normalised inputs, carried back by the chain rule:
      d decay / dx = -a_h sigmoid(x) decay,  d decay / da_h = -softplus(x) decay,
      dL/dy = (g - u (u . g)) / n  with n = sqrt(sum y^2 + eps), u = y / n,
        g = dL/dl2(y).
    Returns dq, dk (of the raw inputs), dv, dw, dbeta, dx, da [H], dtheta
    (rot2) and dS0.
    """
    x64, a64 = np.asarray(x, dtype=np.float64), np.asarray(a, dtype=np.float64)
    alpha = _seq.gated_decay(x64, a64)
    if qk_l2norm:
        q, k = _seq.l2_normalise(q_raw), _seq.l2_normalise(k_raw)
    else:
        q, k = _f64(q_raw), _f64(k_raw)
    g = backward_seq(q, k, v, w, alpha, beta, dO, dS_T, theta=theta, decay=decay, S0=S0)
    out = {n: t for n, t in g.items() if n != "dalpha"}
    gd = g["dalpha"] * alpha                        # dL/d(decay) times the decay
    out["dx"] = gd * (-a64[:, None]) * _seq.sigmoid(x64)
    out["da"] = np.sum(gd * -_seq.softplus(x64), axis=(0, 1, 3))
    if qk_l2norm:
        for name, raw in (("dq", q_raw), ("dk", k_raw)):
            y = _f64(raw)
            n = np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + _seq.L2NORM_EPS)
            u = y / n
            gn = out[name]
            out[name] = (gn - u * np.sum(u * gn, axis=-1, keepdims=True)) / n
    return out
