"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test names the fact it checks.  Plausible mistakes each fail at least one:
a dropped or misplaced decay (closed form under beta = 0, hand examples), the
erase/decay order or sign (exact read-back), the state orientation (read-back,
linear attention), o from S_{t-1} instead of S_t (linear attention, hand
examples), beta missing from the write (hand example), a wrong rotation sign or
pairing (hand example, theta = 0 reduction, cyclic counter), a stale-by-zero
or wrong-window content signal (hand example, chunk-0 and short-sequence
checks), and any error in the chunked algebra (brute-force equality).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import chunk as ochunk
from oracle import seq
from synth.gen import Workload, generate

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _small(decay="diag", B=2, H=3, T=40, dk=8, dv=6, chunk=16, seed=11, content=False):
    wl = Workload("t", B, H, T, dk, dv, chunk, "f32", decay, content, seed, rank=4)
    return generate(wl, ub_std=1.0 if content else 0.02)


def _run(x, **kw):
    args = dict(q=x.q, k=x.k, v=x.v, w=x.w, alpha=x.alpha, beta=x.beta, theta=x.theta,
                decay=x.wl.decay, S0=x.S0)
    if x.wl.content:
        args.update(beta_logit=x.beta_logit, ub_down=x.ub_down, ub_up=x.ub_up,
                    chunk=x.wl.chunk)
    args.update(kw)
    return seq.forward(**args)


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _as_bth(a, extra=True):
    """[T, ...] fixture arrays -> [1, T, 1, ...]."""
    a = np.asarray(a, np.float64)
    return a[None, :, None] if extra else a[None, :, None]


# ---------------------------------------------------------------- hand examples
def test_hand_diag():
    g = _load("hand_diag.json")
    o, S = seq.forward(_as_bth(g["q"]), _as_bth(g["k"]), _as_bth(g["v"]), _as_bth(g["w"]),
                       _as_bth(g["alpha"]), beta=_as_bth(g["beta"]), decay="diag",
                       S0=np.asarray(g["S0"])[None, None])
    np.testing.assert_allclose(o[0, :, 0], g["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], g["S_T"], rtol=0, atol=1e-15)


def test_hand_rot2():
    g = _load("hand_rot2.json")
    o, S = seq.forward(_as_bth(g["q"]), _as_bth(g["k"]), _as_bth(g["v"]), _as_bth(g["w"]),
                       _as_bth(g["alpha"]), beta=_as_bth(g["beta"]),
                       theta=_as_bth(g["theta"]), decay="rot2",
                       S0=np.asarray(g["S0"])[None, None])
    np.testing.assert_allclose(o[0, :, 0], g["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], g["S_T"], rtol=0, atol=1e-15)


def test_hand_content():
    g = _load("hand_content.json")
    o, S = seq.forward(_as_bth(g["q"]), _as_bth(g["k"]), _as_bth(g["v"]), _as_bth(g["w"]),
                       _as_bth(g["alpha"]), decay="diag",
                       beta_logit=_as_bth(g["beta_logit"]),
                       ub_down=np.asarray(g["ub_down"]), ub_up=np.asarray(g["ub_up"]),
                       chunk=g["chunk"])
    np.testing.assert_allclose(o[0, :, 0], g["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], g["S_T"], rtol=0, atol=1e-14)


def test_hand_examples_chunked():
    """The chunked reference reproduces the hand examples too."""
    for name, decay in (("hand_diag.json", "diag"), ("hand_rot2.json", "rot2")):
        g = _load(name)
        o, S, _ = ochunk.chunk_head(np.asarray(g["q"]), np.asarray(g["k"]), np.asarray(g["v"]),
                                    np.asarray(g["w"]), np.asarray(g["alpha"]),
                                    np.asarray(g["beta"]),
                                    None if decay == "diag" else np.asarray(g["theta"]),
                                    decay, np.asarray(g["S0"]), chunk=2)
        np.testing.assert_allclose(o, g["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(S, g["S_T"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_p1_identity_transition_no_erase(decay):
    """alpha = 1 (theta = 0) and beta = 0 leave the state unchanged; o_t = S0 q_t."""
    x = _small(decay)
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((2, 3, 6, 8))
    alpha = np.ones_like(x.alpha)
    theta = None if decay == "diag" else np.zeros_like(x.theta)
    o, S = seq.forward(x.q, x.k, x.v, x.w, alpha, beta=np.zeros_like(x.beta), theta=theta,
                       decay=decay, S0=S0)
    assert np.array_equal(S, S0)
    ref = np.einsum("bhvk,bthk->bthv", S0, x.q.astype(np.float64))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_p2_exact_readback(decay):
    """beta = w = 1 and unit k: the updated state maps k_t exactly to v_t, any S, any decay."""
    x = _small(decay)
    k = x.k.astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    one = np.ones_like(x.w, dtype=np.float64)
    rng = np.random.default_rng(7)
    S = rng.standard_normal((2, 3, 6, 8))
    for t in range(x.wl.T):
        th = None if x.theta is None else x.theta[:, t]
        S, _ = seq.delta_step(S, x.q[:, t].astype(np.float64), k[:, t],
                              x.v[:, t].astype(np.float64), one[:, t], one[:, t],
                              x.alpha[:, t].astype(np.float64),
                              None if th is None else th.astype(np.float64), decay)
        back = np.einsum("bhvk,bhk->bhv", S, k[:, t])
        np.testing.assert_allclose(back, x.v[:, t], rtol=0, atol=1e-13)


def test_p3_rotation_norm_and_mod5_counter():
    """Pure rotation (gamma = 1, beta = 0) keeps ||S||_F; constant theta = 2 pi / 5
    returns the state to S0 every 5 tokens (the constructed cyclic counter of the
    SFDA results section)."""
    B, T, H, dk, dv = 1, 8192, 2, 8, 4
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((B, H, dv, dk))
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    zeros = np.zeros((B, T, H))
    ones = np.ones((B, T, H, dk // 2))
    theta = rng.uniform(-math.pi, math.pi, (B, T, H, dk // 2))
    _, S = seq.forward(q, k, v, zeros, ones, beta=zeros, theta=theta, decay="rot2", S0=S0)
    np.testing.assert_allclose(np.linalg.norm(S, axis=(-2, -1)),
                               np.linalg.norm(S0, axis=(-2, -1)), rtol=1e-11)
    theta5 = np.full((B, 5 * 40, H, dk // 2), 2 * math.pi / 5)
    S = S0
    for n in range(40):
        _, S = seq.forward(q[:, :5], k[:, :5], v[:, :5], zeros[:, :5], ones[:, :5],
                           beta=zeros[:, :5], theta=theta5[:, 5 * n:5 * n + 5],
                           decay="rot2", S0=S)
        np.testing.assert_allclose(S, S0, rtol=0, atol=1e-11)
    # and not before: after 1..4 steps the state differs
    _, S1 = seq.forward(q[:, :2], k[:, :2], v[:, :2], zeros[:, :2], ones[:, :2],
                        beta=zeros[:, :2], theta=theta5[:, :2], decay="rot2", S0=S0)
    assert np.max(np.abs(S1 - S0)) > 0.1


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_p4_no_erase_closed_form(decay):
    """beta = 0: S_t = S0 Gamma_t and o_t = S0 Gamma_t q_t (products of the transitions)."""
    x = _small(decay, B=1, H=2, T=24)
    rng = np.random.default_rng(9)
    S0 = rng.standard_normal((1, 2, 6, 8))
    o, S = seq.forward(x.q, x.k, x.v, x.w, x.alpha, beta=np.zeros_like(x.beta),
                       theta=x.theta, decay=decay, S0=S0)
    for h in range(2):
        G = np.eye(8)
        for t in range(24):
            th = None if x.theta is None else x.theta[0, t, h]
            G = G @ ochunk.transition_matrix(decay, x.alpha[0, t, h], th, 8)
            np.testing.assert_allclose(o[0, t, h], S0[0, h] @ G @ x.q[0, t, h],
                                       rtol=0, atol=1e-13)
        np.testing.assert_allclose(S[0, 0 + h], S0[0, h] @ G, rtol=0, atol=1e-13)
    # the dense transition agrees with the closed-form per-channel decay
    if decay == "diag":
        lam = np.cumsum(np.log(x.alpha[0, :, 0].astype(np.float64)), axis=0)[-1]
        np.testing.assert_allclose(S[0, 0], S0[0, 0] * np.exp(lam)[None, :], rtol=1e-12)


def test_p5_linear_attention():
    """alpha = 1, beta = w = 1, orthonormal keys, S0 = 0: causal linear attention,
    o_t = sum_{i<=t} (k_i . q_t) v_i and S_t = sum_{i<=t} v_i k_i^T (the plain
    delta rule the CARVE family contains)."""
    T, dk, dv = 12, 16, 5
    rng = np.random.default_rng(1)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, :, None]                       # orthonormal rows
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    one = np.ones((1, T, 1))
    o, S = seq.forward(q, k, v, one, np.ones((1, T, 1, dk)), beta=one, decay="diag")
    for t in range(T):
        ref = sum((k[0, i, 0] @ q[0, t, 0]) * v[0, i, 0] for i in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], v[0, :, 0].T @ k[0, :, 0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_p6_affine_in_state_and_values(decay):
    """The map (S0, V) -> (o, S_T) is linear for fixed gates: o(S0, V) = o(S0, 0) + o(0, V)
    (exact affine chunk transfer, SFDA main contributions)."""
    x = _small(decay)
    rng = np.random.default_rng(2)
    S0 = rng.standard_normal((2, 3, 6, 8))
    o1, S1 = _run(x, S0=S0)
    o2, S2 = _run(x, S0=S0, v=np.zeros_like(x.v))
    o3, S3 = _run(x, S0=None)
    np.testing.assert_allclose(o1, o2 + o3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S1, S2 + S3, rtol=0, atol=1e-12)


def test_p7_reductions():
    """rot2 with theta = 0 equals diag with both channels of a block decayed by gamma
    (SFDA with zero phase is KDA); w = 1 and alpha = 1 give the plain delta rule."""
    x = _small("rot2")
    o_r, S_r = seq.forward(x.q, x.k, x.v, x.w, x.alpha, beta=x.beta,
                           theta=np.zeros_like(x.theta), decay="rot2")
    alpha_d = np.repeat(x.alpha, 2, axis=-1)
    o_d, S_d = seq.forward(x.q, x.k, x.v, x.w, alpha_d, beta=x.beta, decay="diag")
    np.testing.assert_allclose(o_r, o_d, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_r, S_d, rtol=0, atol=1e-13)
    # plain delta rule written out: S <- S - beta (S k - v) k^T
    y = _small("diag", B=1, H=1)
    one = np.ones_like(y.w)
    o, S = seq.forward(y.q, y.k, y.v, one, np.ones_like(y.alpha), beta=y.beta)
    Sp = np.zeros((6, 8))
    for t in range(y.wl.T):
        kt, vt, bt = y.k[0, t, 0].astype(np.float64), y.v[0, t, 0], y.beta[0, t, 0]
        Sp = Sp - bt * np.outer(Sp @ kt - vt, kt)
        np.testing.assert_allclose(o[0, t, 0], Sp @ y.q[0, t, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], Sp, rtol=0, atol=1e-13)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
@pytest.mark.parametrize("L", [1, 2, 4, 16])
def test_p8_chunked_equals_sequential(decay, L):
    """Brute force: the chunk-WY algebra (per-chunk triangular solve + affine transfer)
    equals the token recurrence, T % L != 0 and S0 != 0 included.  The SFDA results
    section reports residuals of 1e-10 to 1e-15 for the same comparison."""
    x = _small(decay, T=37)
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((2, 3, 6, 8))
    o_s, S_s = _run(x, S0=S0)
    o_c, S_c = ochunk.forward(x.q, x.k, x.v, x.w, x.alpha, beta=x.beta, theta=x.theta,
                              decay=decay, S0=S0, chunk=L)
    np.testing.assert_allclose(o_c, o_s, rtol=0, atol=1e-10)
    np.testing.assert_allclose(S_c, S_s, rtol=0, atol=1e-10)


def test_p8_chunked_content_aware():
    x = _small("diag", T=64, chunk=16, content=True)
    o_s, S_s = _run(x)
    o_c, S_c = ochunk.forward(x.q, x.k, x.v, x.w, x.alpha, decay="diag", chunk=16,
                              beta_logit=x.beta_logit, ub_down=x.ub_down, ub_up=x.ub_up)
    np.testing.assert_allclose(o_c, o_s, rtol=0, atol=1e-10)
    np.testing.assert_allclose(S_c, S_s, rtol=0, atol=1e-10)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_p9_norm_bound(decay):
    """||S_t||_F <= ||D_t||_2 ||S_{t-1}||_F + w beta ||v|| ||k|| for beta in [0, 2], ||k|| = 1
    (a quantitative form of the bounded-state statement, CARVE section 3, Thm 4)."""
    x = _small(decay, B=1, H=2, T=64)
    k = x.k.astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    rng = np.random.default_rng(8)
    beta = rng.uniform(0, 2, x.beta.shape)
    S = rng.standard_normal((1, 2, 6, 8))
    for t in range(64):
        th = None if x.theta is None else x.theta[:, t].astype(np.float64)
        Sn, _ = seq.delta_step(S, x.q[:, t].astype(np.float64), k[:, t],
                               x.v[:, t].astype(np.float64), beta[:, t],
                               x.w[:, t].astype(np.float64), x.alpha[:, t].astype(np.float64),
                               th, decay)
        dnorm = np.max(x.alpha[:, t], axis=-1)          # ||D_t||_2 (block magnitude)
        bound = (dnorm * np.linalg.norm(S, axis=(-2, -1))
                 + x.w[:, t] * beta[:, t] * np.linalg.norm(x.v[:, t], axis=-1))
        assert np.all(np.linalg.norm(Sn, axis=(-2, -1)) <= bound * (1 + 1e-12))
        S = Sn


def test_p10_content_aware_special_cases():
    """U_b = 0 is erase = sigmoid(b_x); T <= L gives no content signal (no previous
    chunk); chunk 0 never depends on U_b (CARVE section 2.1 and limitations)."""
    x = _small("diag", T=64, chunk=16, content=True)
    o, S = _run(x, ub_down=np.zeros_like(x.ub_down))
    o0, S0_ = seq.forward(x.q, x.k, x.v, x.w, x.alpha, beta=seq.sigmoid(x.beta_logit.astype(np.float64)))
    np.testing.assert_array_equal(o, o0)
    np.testing.assert_array_equal(S, S0_)
    # T <= L: no signal at all
    y = _small("diag", T=16, chunk=16, content=True)
    o1, _ = _run(y)
    o2, _ = seq.forward(y.q, y.k, y.v, y.w, y.alpha, beta=seq.sigmoid(y.beta_logit.astype(np.float64)))
    np.testing.assert_array_equal(o1, o2)
    # chunk 0 unaffected, later chunks affected (stress scale)
    o3, _ = _run(x)
    np.testing.assert_array_equal(o3[:, :16], o0[:, :16])
    assert np.max(np.abs(o3[:, 16:] - o0[:, 16:])) > 1e-3


def test_p10_content_signal_is_previous_chunk_mean():
    """Decompose the content-aware run: chunk c's erase gate equals sigmoid(b_x + a^T B m)
    with m the mean of chunk c-1's outputs, replayed through the plain path."""
    x = _small("diag", B=1, H=2, T=48, chunk=16, content=True)
    o, S = _run(x)
    beta = np.empty_like(x.beta_logit, dtype=np.float64)
    m = np.zeros((1, 2, 6))
    Sr = None
    for c in range(3):
        sl = slice(16 * c, 16 * c + 16)
        if c:
            m = o[:, 16 * (c - 1):16 * c].mean(axis=1)
        s = np.stack([x.ub_up[h] @ (x.ub_down[h] @ m[0, h]) for h in range(2)])
        beta[:, sl] = seq.sigmoid(x.beta_logit[:, sl] + s[None, None, :])
        oc, Sr = seq.forward(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.w[:, sl], x.alpha[:, sl],
                             beta=beta[:, sl], S0=Sr)
        np.testing.assert_allclose(oc, o[:, sl], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sr, S, rtol=0, atol=1e-13)


@pytest.mark.parametrize("content", [False, True])
def test_p11_resume(content):
    """fwd(T1) then fwd(T2, S0 = S_T1, carried mean) equals fwd(T1 + T2)."""
    x = _small("diag", T=64, chunk=16, content=content)
    if content:
        o, S = _run(x)
        o1, S1, m1 = _run(x, q=x.q[:, :32], k=x.k[:, :32], v=x.v[:, :32], w=x.w[:, :32],
                          alpha=x.alpha[:, :32], beta_logit=x.beta_logit[:, :32],
                          return_m=True)
        o2, S2 = _run(x, q=x.q[:, 32:], k=x.k[:, 32:], v=x.v[:, 32:], w=x.w[:, 32:],
                      alpha=x.alpha[:, 32:], beta_logit=x.beta_logit[:, 32:], S0=S1,
                      m_carry=m1)
    else:
        o, S = _run(x)
        sl1, sl2 = slice(0, 23), slice(23, 64)
        o1, S1 = _run(x, q=x.q[:, sl1], k=x.k[:, sl1], v=x.v[:, sl1], w=x.w[:, sl1],
                      alpha=x.alpha[:, sl1], beta=x.beta[:, sl1])
        o2, S2 = _run(x, q=x.q[:, sl2], k=x.k[:, sl2], v=x.v[:, sl2], w=x.w[:, sl2],
                      alpha=x.alpha[:, sl2], beta=x.beta[:, sl2], S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-13)


def test_decode_step_is_one_token():
    """The decode oracle is one token of the recurrence on each of N states."""
    x = _small("rot2", B=3, H=2, T=1)
    rng = np.random.default_rng(6)
    S0 = rng.standard_normal((3, 2, 6, 8))
    o, S = seq.forward(x.q, x.k, x.v, x.w, x.alpha, beta=x.beta, theta=x.theta,
                       decay="rot2", S0=S0)
    S1, o1 = seq.decode_step(S0, x.q[:, 0], x.k[:, 0], x.v[:, 0], x.beta[:, 0], x.w[:, 0],
                             x.alpha[:, 0], x.theta[:, 0], "rot2")
    np.testing.assert_array_equal(S1, S)
    np.testing.assert_array_equal(o1, o[:, 0])


def test_generator_deterministic_and_bf16_exact():
    from synth.gen import WORKLOADS, bf16_round
    a = generate(WORKLOADS["small"], T=64)
    b = generate(WORKLOADS["small"], T=64)
    for f in ("q", "k", "v", "beta", "w", "alpha"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    # bf16 tensors are exactly representable, q/k unit norm to bf16 accuracy
    np.testing.assert_array_equal(bf16_round(a.q), a.q)
    n = np.linalg.norm(a.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all((a.alpha > 0) & (a.alpha <= 1)) and np.all((a.beta > 0) & (a.beta < 1))


def test_bf16_rounding_ties_to_even():
    from synth.gen import bf16_bits
    # 1 + 2^-8 is halfway between two bf16 neighbours -> rounds to even (1.0);
    # 1 + 3*2^-8 is halfway -> rounds up to the even neighbour 1 + 2^-6... (0x3F82)
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    bits = bf16_bits(vals)
    assert list(bits[:4]) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


# ---------------------------------------------------------------- error measure
def test_max_rel_err_hand_cases():
    """The parity measure is max|x - r| / max|r| over the whole tensor (hand values)."""
    from oracle.errors import max_rel_err
    # errors 0.1 and 0.5, reference magnitudes 4 and 2: 0.5 / 4.  (An element-wise
    # relative error would give 0.25, a mean 0.1, a relative Frobenius norm 0.114.)
    assert max_rel_err([4.1, 1.5], [4.0, 2.0]) == pytest.approx(0.125, abs=1e-15)
    # the sign of x and of the difference both count: |-1 - 1| / 1
    assert max_rel_err([-1.0], [1.0]) == 2.0
    assert max_rel_err([[0.0, -3.0]], [[0.0, 3.0]]) == 2.0
    # all-zero reference: the absolute error
    assert max_rel_err([0.0, -0.25], [0.0, 0.0]) == 0.25
    assert max_rel_err([0.0], [0.0]) == 0.0
    # identical tensors and the empty tensor
    assert max_rel_err(np.arange(6.0).reshape(2, 3), np.arange(6.0).reshape(2, 3)) == 0.0
    assert max_rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
    # non-finite values never pass a tolerance
    assert max_rel_err([np.nan, 1.0], [1.0, 1.0]) == math.inf
    assert max_rel_err([np.inf], [1.0]) == math.inf
    assert max_rel_err([1.0], [np.nan]) == math.inf
    # no broadcasting: a shape mismatch is an error
    with pytest.raises(ValueError):
        max_rel_err(np.zeros((2, 3)), np.zeros((3,)))
    with pytest.raises(ValueError):
        max_rel_err(np.zeros((2, 1)), np.zeros((2, 2)))
    # float32 input is upcast before subtracting: 1 + 2^-23 vs 1 is not zero
    assert max_rel_err(np.float32([1 + 2 ** -23]), [1.0]) == pytest.approx(2 ** -23, rel=1e-12)


# ---------------------------------------------------------------- strong decay
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_pure_reset_register(decay):
    """alpha = 0 (or a zero-magnitude rotation block), beta = w = 1, unit keys: the
    state forgets everything and holds exactly the last write, S_t = v_t k_t^T, so
    o_t = v_t (k_t . q_t) -- the reset/register construction of the SFDA page
    (finite-state expressivity, with delta correction)."""
    x = _small(decay, T=20)
    k = x.k.astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    ones = np.ones_like(x.w)
    zero_a = np.zeros_like(x.alpha)
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((2, 3, 6, 8))
    o, S = seq.forward(x.q, k, x.v, ones, zero_a, beta=ones, theta=x.theta, decay=decay, S0=S0)
    q = x.q.astype(np.float64)
    v = x.v.astype(np.float64)
    o_ref = v * np.sum(k * q, axis=-1)[..., None]
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    S_ref = v[:, -1, :, :, None] * k[:, -1, :, None, :]
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-14)


def test_strong_decay_closed_form():
    """beta = 0 with per-token decays far below the fp32 range of a running product
    (alpha in [1e-3, 0.01], cumulative log-decay below -150 within 32 tokens): the
    oracle still gives S_t = S_0 Gamma_t exactly (fp64 has the range)."""
    x = _small("diag", T=48)
    rng = np.random.default_rng(4)
    a = rng.uniform(1e-3, 0.01, size=x.alpha.shape)
    S0 = rng.standard_normal((2, 3, 6, 8))
    o, S = seq.forward(x.q, x.k, x.v, x.w, a, beta=np.zeros_like(x.w), S0=S0)
    G = np.cumprod(a, axis=1)                                   # [B,T,H,dk]
    lg = np.log(G[:, 31])
    assert lg.max() < -150                         # every channel leaves fp32's range
    q = x.q.astype(np.float64)
    o_ref = np.einsum("bhvk,bthk,bthk->bthv", S0, G, q)
    scale = np.einsum("bhvk,bthk,bthk->bthv", np.abs(S0), G, np.abs(q))   # sum of |terms|
    assert np.all(np.abs(o - o_ref) <= 1e-13 * scale)
    np.testing.assert_allclose(S, S0 * G[:, -1, :, None, :], rtol=1e-12, atol=0)


# ---------------------------------------------------------------- gated forward
def test_gated_decay_closed_forms():
    """softplus(0) = ln 2, so a = 1 gives a decay of exactly 1/2; a = 0 gives 1 for
    any x; x -> -inf gives 1; x = 50 gives e^{-50 a} (softplus(x) = x + log1p(e^-x));
    x = 1000 does not overflow: e^{-1000 a}."""
    x = np.array([[0.0, 0.0], [-1000.0, 50.0], [1000.0, 3.0]])
    d = seq.gated_decay(x[None], np.array([1.0, 0.0, 0.1]))[0]
    assert d[0, 0] == 0.5 and d[0, 1] == 0.5
    assert d[1, 0] == 1.0 and d[1, 1] == 1.0          # a = 0
    assert d[2, 0] == pytest.approx(np.exp(-100.0), rel=1e-13)
    assert d[2, 1] == pytest.approx(np.exp(-0.1 * (3.0 + np.log1p(np.exp(-3.0)))), rel=1e-15)
    d50 = seq.gated_decay(np.array([[[50.0]]]), np.array([0.1]))
    assert d50[0, 0, 0] == pytest.approx(np.exp(-5.0), rel=1e-14)
    assert seq.gated_decay(np.array([[[-1000.0]]]), np.array([3.0]))[0, 0, 0] == 1.0


def test_l2_normalise_hand_values():
    """(3, 4) -> (0.6, 0.8) up to the epsilon; scale-invariant; a zero vector stays
    zero (the epsilon keeps it finite)."""
    v = seq.l2_normalise(np.array([3.0, 4.0, 0.0]), eps=0.0)
    assert list(v) == [0.6, 0.8, 0.0]
    v = seq.l2_normalise(np.array([3.0, 4.0]))
    np.testing.assert_allclose(v, [0.6, 0.8], rtol=1e-7)
    np.testing.assert_array_equal(seq.l2_normalise(np.zeros(4)), np.zeros(4))


def test_forward_gated_matches_explicit_inputs():
    """With x = 0 and a = 1 (decay exactly 1/2) and raw keys/queries that are
    multiples of unit vectors, the gated forward equals the plain forward on the
    unit vectors and alpha = 1/2 -- values fixed without the activation's formula."""
    rng = np.random.default_rng(8)
    B, T, H, dk, dv = 2, 12, 3, 8, 6
    qu = rng.standard_normal((B, T, H, dk)); qu /= np.linalg.norm(qu, axis=-1, keepdims=True)
    ku = rng.standard_normal((B, T, H, dk)); ku /= np.linalg.norm(ku, axis=-1, keepdims=True)
    sq = rng.uniform(0.5, 4.0, (B, T, H, 1)); sk = rng.uniform(0.5, 4.0, (B, T, H, 1))
    v = rng.standard_normal((B, T, H, dv))
    w = rng.uniform(0, 1, (B, T, H)); beta = rng.uniform(0, 1, (B, T, H))
    o1, S1 = seq.forward_gated(qu * sq, ku * sk, v, w, np.zeros((B, T, H, dk)), np.ones(H), beta)
    o2, S2 = seq.forward(qu, ku, v, w, np.full((B, T, H, dk), 0.5), beta=beta)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-6)   # eps = 1e-6 against norms >= 0.5
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-6)
    # rotation blocks: the pre-activation drives the block magnitude
    x = np.zeros((B, T, H, dk // 2))
    th = rng.uniform(-np.pi, np.pi, (B, T, H, dk // 2))
    o1, _ = seq.forward_gated(qu * sq, ku * sk, v, w, x, np.ones(H), beta, theta=th, decay="rot2")
    o2, _ = seq.forward(qu, ku, v, w, np.full((B, T, H, dk // 2), 0.5), beta=beta, theta=th,
                        decay="rot2")
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-6)


# ----------------------------------------------------------------------------
# Reflection blocks (dihedral memory; SFDA technical summary, finite-state
# expressivity: "with reflections" the family realises dihedral phase-
# orientation memory).  Pinned against the group law of D_n, not the matrices.
# ----------------------------------------------------------------------------
def _dihedral_apply(a_b_seq, n):
    """Fold (a, b) pairs (rotation index, reflection bit) by the D_n law
    (a1, b1)(a2, b2) = (a1 + (-1)^b1 a2 mod n, b1 xor b2), left to right."""
    a, b = 0, 0
    for a2, b2 in a_b_seq:
        a, b = (a + (-a2 if b else a2)) % n, b ^ b2
    return a, b


def _dihedral_matrix(a, b, n):
    """M(a, b) = R(2 pi a / n) F^b acting on the right of a row pair, with
    R(phi) = [[cos, -sin], [sin, cos]] and F = Diag(1, -1)."""
    ph = 2 * np.pi * a / n
    R = np.array([[np.cos(ph), -np.sin(ph)], [np.sin(ph), np.cos(ph)]])
    return R @ (np.diag([1.0, -1.0]) if b else np.eye(2))


@pytest.mark.parametrize("n", [3, 5, 8])
def test_dihedral_memory_follows_the_group_law(n):
    """With beta = 0 the state of each key pair is S0 times the product of the
    tokens' D_n elements; the oracle must agree with the group law folded by
    hand (a wrong reflection matrix or a swapped product order fails for the
    non-abelian D_n, n >= 3)."""
    rng = np.random.default_rng(n)
    B, T, H, dk, dv = 1, 40, 1, 6, 3
    a_idx = rng.integers(0, n, (T, dk // 2))
    b_bit = rng.integers(0, 2, (T, dk // 2))
    theta = (2 * np.pi * a_idx / n)[None, :, None, :]
    gam = np.where(b_bit == 1, -1.0, 1.0)[None, :, None, :]
    S0 = rng.standard_normal((B, H, dv, dk))
    z = np.zeros((B, T, H))
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    _, S = seq.forward(q, k, v, z, gam, beta=z, theta=theta, decay="dihedral", S0=S0)
    for j in range(dk // 2):
        a, b = _dihedral_apply(list(zip(a_idx[:, j], b_bit[:, j])), n)
        want = S0[0, 0][:, 2 * j:2 * j + 2] @ _dihedral_matrix(a, b, n)
        assert np.allclose(S[0, 0][:, 2 * j:2 * j + 2], want, atol=1e-12)


def test_dihedral_reflection_is_an_involution_and_does_not_commute():
    """Two equal reflections give |gamma|^2 S0; a rotation then a reflection
    differs from the reverse order."""
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((1, 1, 2, 2))
    z = np.zeros((1, 2, 1))
    qkv = rng.standard_normal((1, 2, 1, 2))

    def run(gam, th):
        g = np.asarray(gam, np.float64).reshape(1, 2, 1, 1)
        t = np.asarray(th, np.float64).reshape(1, 2, 1, 1)
        return seq.forward(qkv, qkv, qkv, z, g, beta=z, theta=t, decay="dihedral", S0=S0)[1]
    assert np.allclose(run([-0.5, -0.5], [0.7, 0.7]), 0.25 * S0, atol=1e-14)
    a = run([0.9, -0.9], [0.7, 0.2])
    b = run([-0.9, 0.9], [0.2, 0.7])
    assert not np.allclose(a, b)


@pytest.mark.parametrize("L", [1, 3, 8, 16])
def test_dihedral_chunked_equals_sequential(L):
    """Brute force: the chunk-WY algebra with dense, non-commuting transition
    products equals the token recurrence (random magnitudes, angles and
    reflection signs, writes on, ragged tail, S0 != 0)."""
    from oracle import chunk
    rng = np.random.default_rng(10 + L)
    B, T, H, dk, dv = 2, 21, 2, 4, 3
    q = rng.standard_normal((B, T, H, dk)) * 0.5
    k = rng.standard_normal((B, T, H, dk)) * 0.5
    v = rng.standard_normal((B, T, H, dv))
    w = rng.uniform(0.2, 1.0, (B, T, H))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    gam = rng.uniform(0.7, 1.0, (B, T, H, dk // 2)) * np.where(rng.uniform(size=(B, T, H, dk // 2)) < 0.5, -1, 1)
    theta = rng.uniform(-np.pi, np.pi, (B, T, H, dk // 2))
    S0 = rng.standard_normal((B, H, dv, dk)) * 0.3
    o1, S1 = seq.forward(q, k, v, w, gam, beta=beta, theta=theta, decay="dihedral", S0=S0)
    o2, S2 = chunk.forward(q, k, v, w, gam, beta=beta, theta=theta, decay="dihedral", S0=S0, chunk=L)
    assert np.max(np.abs(o1 - o2)) < 1e-10 and np.max(np.abs(S1 - S2)) < 1e-10
