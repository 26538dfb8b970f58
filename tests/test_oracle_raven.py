"""Pins of the Raven slot-memory oracle (oracle/raven.py), CPU only.

Each pin is a special case the Raven page names or a closed form that does not
go through the oracle's own slot arithmetic:

* the one-hot, time-indexed router with full replacement (Raven technical
  summary, section 2.1) is sliding-window attention over the last M tokens --
  checked against attention written directly over the token window;
* the dense router with equal logits (all M slots selected, r = 1/M each; the
  state-space-model end of section 2.1) keeps every slot equal, so the output
  is the exponential moving average h_t = lam_t h_{t-1} + (1 - lam_t) v_t
  with lam_t = exp(a_t / M);
* a = 0 freezes every slot (section 2.2): the output is attention over the
  initial state for every token, and the states come back bitwise;
* the router: top-K with ties to the lower slot index, normalised sigmoid
  gates, and unselected slots untouched (bitwise);
* one token from a zero state with full replacement: o has a closed form.
"""
import math

import numpy as np
import pytest

from oracle import raven


def _rand(shape, rng):
    return rng.standard_normal(shape)


def test_router_top_k_ties_and_normalisation():
    z = np.array([0.0, 1.0, 1.0, 0.5])
    sel, r = raven.route(z, 2)
    assert sel.tolist() == [False, True, True, False]
    assert np.allclose(r, [0.0, 0.5, 0.5, 0.0], rtol=0, atol=1e-15)
    sel, r = raven.route(z, 1)                      # tie: the lower index wins
    assert sel.tolist() == [False, True, False, False] and r[1] == 1.0
    sel, r = raven.route(z, 3)
    s = 1 / (1 + math.exp(-1.0))
    h = 1 / (1 + math.exp(-0.5))
    assert sel.tolist() == [False, True, True, True]
    assert np.allclose(r, [0.0, s / (2 * s + h), s / (2 * s + h), h / (2 * s + h)], atol=1e-15)
    # batched: each row routed on its own
    sel, r = raven.route(np.array([[3.0, -1.0, 2.0], [-5.0, -5.0, -6.0]]), 1)
    assert sel.tolist() == [[True, False, False], [True, False, False]]
    with pytest.raises(ValueError):
        raven.route(z, 0)


def test_one_hot_full_replacement_is_sliding_window_attention():
    """K = 1 with slot t mod M on top, a = -1e30 (exp(a r) = 0): after M tokens
    the slots hold exactly the last M keys and values, and o_t is softmax
    attention of q_t over tokens t-M+1 .. t."""
    rng = np.random.default_rng(0)
    B, T, H, M, d = 2, 23, 3, 5, 4
    q, k, v = (_rand((B, T, H, d), rng) for _ in range(3))
    z = np.full((B, T, H, M), -3.0)
    for t in range(T):
        z[:, t, :, t % M] = 3.0
    a = np.full((B, T, H), -1e30)
    scale = 0.7
    o, Sk, Sv = raven.forward(q, k, v, z, a, 1, scale)
    for t in range(M - 1, T):
        win = slice(t - M + 1, t + 1)
        s = scale * np.einsum("bhd,bshd->bhs", q[:, t], k[:, win])
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        want = np.einsum("bhs,bshd->bhd", p, v[:, win])
        assert np.max(np.abs(o[:, t] - want)) < 1e-12, t
    for j in range(M):                       # slot j holds the last token t with t % M == j
        t = max(tt for tt in range(T) if tt % M == j)
        assert np.array_equal(Sk[:, :, j], k[:, t]) and np.array_equal(Sv[:, :, j], v[:, t])


def test_dense_equal_router_is_an_exponential_moving_average():
    """K = M and z = 0: r = 1/M on every slot, all slots stay equal (zero start),
    the softmax is uniform, and o_t = h_t with h_t = lam h_{t-1} + (1-lam) v_t,
    lam = exp(a_t / M)."""
    rng = np.random.default_rng(1)
    B, T, H, M, d = 1, 17, 2, 4, 3
    q, k, v = (_rand((B, T, H, d), rng) for _ in range(3))
    z = np.zeros((B, T, H, M))
    a = -rng.uniform(0.1, 3.0, (B, T, H))
    o, Sk, Sv = raven.forward(q, k, v, z, a, M, 1.0)
    h = np.zeros((B, H, d))
    hk = np.zeros((B, H, d))
    for t in range(T):
        lam = np.exp(a[:, t] / M)[..., None]
        h = lam * h + (1 - lam) * v[:, t]
        hk = lam * hk + (1 - lam) * k[:, t]
        assert np.max(np.abs(o[:, t] - h)) < 1e-12, t
    assert np.max(np.abs(Sv - h[:, :, None, :])) < 1e-12
    assert np.max(np.abs(Sk - hk[:, :, None, :])) < 1e-12


def test_zero_rate_freezes_every_slot():
    """a = 0: exp(a r) = 1 for every slot, nothing is written; o_t is attention
    of q_t over the initial slots, and the states come back unchanged."""
    rng = np.random.default_rng(2)
    B, T, H, M, d = 2, 9, 2, 6, 5
    q, k, v = (_rand((B, T, H, d), rng) for _ in range(3))
    z = _rand((B, T, H, M), rng)
    Sk0, Sv0 = _rand((B, H, M, d), rng), _rand((B, H, M, d), rng)
    o, Sk, Sv = raven.forward(q, k, v, z, np.zeros((B, T, H)), 3, 0.5, Sk0, Sv0)
    assert np.array_equal(Sk, Sk0) and np.array_equal(Sv, Sv0)
    s = 0.5 * np.einsum("bhmd,bthd->bthm", Sk0, q)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    want = np.einsum("bthm,bhmd->bthd", p, Sv0)
    assert np.max(np.abs(o - want)) < 1e-12


def test_unselected_slots_are_untouched():
    """Slots that the router never selects keep their initial rows bitwise,
    while selected ones change."""
    rng = np.random.default_rng(3)
    B, T, H, M, d = 1, 12, 1, 8, 4
    q, k, v = (_rand((B, T, H, d), rng) for _ in range(3))
    z = _rand((B, T, H, M), rng)
    z[..., 5:] = -50.0                        # slots 5..7 never reach the top 2
    Sk0, Sv0 = _rand((B, H, M, d), rng), _rand((B, H, M, d), rng)
    _, Sk, Sv = raven.forward(q, k, v, z, -np.ones((B, T, H)), 2, 1.0, Sk0, Sv0)
    assert np.array_equal(Sk[..., 5:, :], Sk0[..., 5:, :])
    assert np.array_equal(Sv[..., 5:, :], Sv0[..., 5:, :])
    assert not np.allclose(Sk[..., :5, :], Sk0[..., :5, :])


def test_single_token_full_replacement_closed_form():
    """T = 1 from zero slots, K = 1, a = -1e30: slot j* becomes (k, v), every
    other slot stays zero, so o = e^(s k.q) v / (e^(s k.q) + M - 1); the read-out
    sees the state after the update."""
    rng = np.random.default_rng(4)
    M, d, s = 7, 5, 0.9
    q, k, v = (_rand((1, 1, 1, d), rng) for _ in range(3))
    z = np.zeros((1, 1, 1, M))
    z[..., 4] = 1.0
    o, Sk, Sv = raven.forward(q, k, v, z, np.full((1, 1, 1), -1e30), 1, s)
    e = math.exp(s * float(np.dot(k[0, 0, 0], q[0, 0, 0])))
    assert np.allclose(o[0, 0, 0], e * v[0, 0, 0] / (e + M - 1), rtol=0, atol=1e-14)
    assert np.array_equal(Sk[0, 0, 4], k[0, 0, 0]) and not np.any(Sk[0, 0, :4])


def test_partial_decay_mixes_old_and_new():
    """One selected slot with r = 1 and a = ln(0.25): the slot becomes
    0.25 * old + 0.75 * new, exactly."""
    Sk0 = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    Sv0 = np.array([[[[5.0], [6.0]]]])
    k = np.array([[[[10.0, 20.0]]]])
    v = np.array([[[[7.0]]]])
    q = np.zeros((1, 1, 1, 2))
    z = np.array([[[[0.0, 1.0]]]])
    _, Sk, Sv = raven.forward(q, k, v, z, np.full((1, 1, 1), math.log(0.25)), 1, 1.0, Sk0, Sv0)
    assert np.allclose(Sk[0, 0], [[1.0, 2.0], [0.25 * 3 + 7.5, 0.25 * 4 + 15.0]], atol=1e-14)
    assert np.allclose(Sv[0, 0], [[5.0], [0.25 * 6 + 0.75 * 7]], atol=1e-14)
