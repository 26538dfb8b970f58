"""fp64 token-by-token oracle of the Raven routing slot memory.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP path.

The recurrence (one head; M slots; a key state S^k in R^{M x d_k} and a value
state S^v in R^{M x d_v}, one row per slot):

    m_t    = sigmoid(z_t)                    router scores, z_t in R^M
    sel_t  = the K slots with the largest z_t (ties: the lower slot index)
    r_t[i] = m_t[i] / sum_{j in sel_t} m_t[j]  for i in sel_t, else 0
    lam_t[i] = exp(a_t r_t[i])  for i in sel_t, else exactly 1 (frozen slot)
    S^k_t[i] = lam_t[i] S^k_{t-1}[i] + (1 - lam_t[i]) k_t
    S^v_t[i] = lam_t[i] S^v_{t-1}[i] + (1 - lam_t[i]) v_t
    p_t    = softmax_i(scale * S^k_t[i] . q_t)
    o_t    = sum_i p_t[i] S^v_t[i]

Sources (pages, not code):
  * Raven technical summary, section 2.1 (routing slot memories): a state of M
    independent slots, a routing vector that sets each slot's write strength,
    and the two extremes it spans -- a dense router (a state-space model) and
    a one-hot, time-indexed router with full replacement (sliding-window
    attention).
  * Raven technical summary, section 2.2: separate key and value slot states
    as in sliding-window attention; sigmoid scores of the input, only the top
    K kept and the kept ones normalised (the DeepSeek-MoE router); the
    selective decay exp(a_t r_t) applied to the selected slots only, with an
    input-dependent scalar a_t, so that an unselected slot is frozen; no
    short convolution.

Readings taken where the page leaves a step open:
  * the router's input projection is outside this operation: z_t = W x_t
    arrives as given logits (the kernel's input);
  * the value state follows the same selective-decay update as the key state,
    with v_t in place of k_t;
  * the read-out is attention over the slots, softmax(scale S^k_t q_t) applied
    to S^v_t, taken after the update -- the form under which the one-hot
    router with full replacement is exactly sliding-window attention;
  * an unselected slot's factor is exactly 1 (not exp(a_t * 0) evaluated), and
    a_t is finite and <= 0;
  * ties among equal router logits go to the lower slot index.

Everything is computed in float64 with numpy; loops run over tokens only.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def route(z: np.ndarray, topk: int):
    """Router of one token for a batch of heads: z [..., M] -> (sel, r).

    sel [..., M] bool: the top-K slots by z (a stable sort of -z keeps equal
    logits in slot order, so the lower index wins a tie); r [..., M]: the
    sigmoid scores of the selected slots divided by their sum, 0 elsewhere.
    """
    z = _f64(z)
    M = z.shape[-1]
    if not 1 <= topk <= M:
        raise ValueError("topk must be in [1, M]")
    order = np.argsort(-z, axis=-1, kind="stable")
    sel = np.zeros(z.shape, dtype=bool)
    np.put_along_axis(sel, order[..., :topk], True, axis=-1)
    m = 1.0 / (1.0 + np.exp(-z))
    gm = np.where(sel, m, 0.0)
    r = gm / np.sum(gm, axis=-1, keepdims=True)
    return sel, r


def step(Sk, Sv, q_t, k_t, v_t, z_t, a_t, topk: int, scale: float):
    """One token for a batch of heads.

    Sk [..., M, d_k], Sv [..., M, d_v]; q_t, k_t [..., d_k]; v_t [..., d_v];
    z_t [..., M]; a_t [...].  Returns (Sk_t, Sv_t, o_t).
    """
    sel, r = route(z_t, topk)
    lam = np.where(sel, np.exp(a_t[..., None] * r), 1.0)[..., None]   # [..., M, 1]
    Sk = lam * Sk + (1.0 - lam) * k_t[..., None, :]
    Sv = lam * Sv + (1.0 - lam) * v_t[..., None, :]
    logits = scale * np.einsum("...md,...d->...m", Sk, q_t)
    logits = logits - np.max(logits, axis=-1, keepdims=True)
    p = np.exp(logits)
    p = p / np.sum(p, axis=-1, keepdims=True)
    o = np.einsum("...m,...md->...d", p, Sv)
    return Sk, Sv, o


def forward(q, k, v, z, a, topk: int, scale: float, Sk0=None, Sv0=None):
    """Whole sequences: q, k [B,T,H,d_k], v [B,T,H,d_v], z [B,T,H,M],
    a [B,T,H]; Sk0 [B,H,M,d_k], Sv0 [B,H,M,d_v] or None (zero).

    Returns (o [B,T,H,d_v], Sk_T [B,H,M,d_k], Sv_T [B,H,M,d_v]), float64.
    """
    q, k, v, z, a = map(_f64, (q, k, v, z, a))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    M = z.shape[-1]
    Sk = np.zeros((B, H, M, dk)) if Sk0 is None else _f64(Sk0).copy()
    Sv = np.zeros((B, H, M, dv)) if Sv0 is None else _f64(Sv0).copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        Sk, Sv, o[:, t] = step(Sk, Sv, q[:, t], k[:, t], v[:, t], z[:, t], a[:, t],
                               topk, scale)
    return o, Sk, Sv
