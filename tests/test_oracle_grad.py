"""Pins of the fp64 gradient oracle (oracle/grad.py), CPU only.

* backward_seq against central finite differences of oracle.seq.forward, on
  every element of every input, both transition forms;
* closed forms: with beta = 0 nothing is written, so v and w get exactly zero
  gradient; one token from a zero state gives dv = beta w (k . q) dO;
* the chunk form: forward_chunk equals seq.forward, and backward_chunk equals
  backward_seq for chunk lengths 1, 3, 4 and whole-sequence, ragged tails
  included.
"""
import numpy as np
import pytest

from oracle import grad, seq

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(decay, B=1, T=5, H=2, d=4, seed=0, zero_beta=False):
    rng = np.random.default_rng(seed)
    C = d if decay == "diag" else d // 2
    x = dict(
        q=rng.standard_normal((B, T, H, d)),
        k=rng.standard_normal((B, T, H, d)) * 0.5,
        v=rng.standard_normal((B, T, H, d)),
        w=rng.uniform(0.2, 1.0, (B, T, H)),
        beta=np.zeros((B, T, H)) if zero_beta else rng.uniform(0.1, 0.9, (B, T, H)),
        alpha=rng.uniform(0.5, 1.0, (B, T, H, C)),
        theta=None if decay == "diag" else rng.uniform(-3.0, 3.0, (B, T, H, C)),
        S0=rng.standard_normal((B, H, d, d)) * 0.3,
    )
    dO = rng.standard_normal((B, T, H, d))
    dS = rng.standard_normal((B, H, d, d))
    return x, dO, dS


def _loss(x, dO, dS, decay):
    o, S = seq.forward(x["q"], x["k"], x["v"], x["w"], x["alpha"], beta=x["beta"],
                       theta=x["theta"], decay=decay, S0=x["S0"])
    return float(np.sum(dO * o) + np.sum(dS * S))


NAMES = {"q": "dq", "k": "dk", "v": "dv", "w": "dw", "beta": "dbeta", "alpha": "dalpha",
         "theta": "dtheta", "S0": "dS0"}


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_backward_seq_matches_finite_differences(decay):
    """Every partial derivative against a central difference (h = 1e-5; the
    truncation error is O(h^2) ~ 1e-10 for these smooth polynomials)."""
    x, dO, dS = _case(decay)
    g = grad.backward_seq(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, dS,
                          theta=x["theta"], decay=decay, S0=x["S0"])
    h = 1e-5
    for name, gname in NAMES.items():
        if x[name] is None:
            continue
        fd = np.empty_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = dict(x)
            xm = dict(x)
            xp[name] = x[name].copy()
            xm[name] = x[name].copy()
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (_loss(xp, dO, dS, decay) - _loss(xm, dO, dS, decay)) / (2 * h)
        err = np.max(np.abs(fd - g[gname]) / np.maximum(1.0, np.abs(fd)))
        assert err < 1e-7, (decay, name, err)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_no_write_gives_zero_value_gradients(decay):
    """beta = 0: the state only decays, o_t = S0 P_t q_t, so dv = dw = 0 exactly
    and dk = 0 (k enters only through the erase and the write)."""
    x, dO, dS = _case(decay, zero_beta=True, seed=3)
    g = grad.backward_seq(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, dS,
                          theta=x["theta"], decay=decay, S0=x["S0"])
    assert np.all(g["dv"] == 0) and np.all(g["dw"] == 0) and np.all(g["dk"] == 0)
    assert np.any(g["dbeta"] != 0) and np.any(g["dq"] != 0)


def test_single_token_from_zero_state():
    """T = 1, S0 = 0: S_1 = beta w v k^T and o = beta w (k . q) v, so
    dv = beta w (k . q) dO + beta w (dS k), dq = beta w (v . dO) k."""
    x, dO, dS = _case("diag", T=1, H=1, seed=5)
    x["S0"] = np.zeros_like(x["S0"])
    g = grad.backward_seq(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, dS,
                          decay="diag", S0=x["S0"])
    b, w = x["beta"][0, 0, 0], x["w"][0, 0, 0]
    k, q, v, do = x["k"][0, 0, 0], x["q"][0, 0, 0], x["v"][0, 0, 0], dO[0, 0, 0]
    dv_ref = b * w * np.dot(k, q) * do + b * w * (dS[0, 0] @ k)
    dq_ref = b * w * np.dot(v, do) * k
    assert np.allclose(g["dv"][0, 0, 0], dv_ref, rtol=1e-13, atol=1e-14)
    assert np.allclose(g["dq"][0, 0, 0], dq_ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
@pytest.mark.parametrize("chunk", [1, 3, 4, 64])
def test_chunk_form_matches_sequential(decay, chunk):
    """forward_chunk = seq.forward and backward_chunk = backward_seq (T = 11:
    ragged last chunk for 3 and 4; one chunk for 64)."""
    x, dO, dS = _case(decay, B=2, T=11, H=2, d=4, seed=7)
    o1, S1 = seq.forward(x["q"], x["k"], x["v"], x["w"], x["alpha"], beta=x["beta"],
                         theta=x["theta"], decay=decay, S0=x["S0"])
    o2, S2 = grad.forward_chunk(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"],
                                theta=x["theta"], decay=decay, S0=x["S0"], chunk=chunk)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(S1 - S2)) < 1e-12
    g1 = grad.backward_seq(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, dS,
                           theta=x["theta"], decay=decay, S0=x["S0"])
    g2 = grad.backward_chunk(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, dS,
                             theta=x["theta"], decay=decay, S0=x["S0"], chunk=chunk)
    assert set(g1) == set(g2)
    for n in g1:
        scale = max(1.0, float(np.max(np.abs(g1[n]))))
        assert np.max(np.abs(g1[n] - g2[n])) / scale < 1e-11, (n, chunk)


def test_chunk_backward_without_final_state_gradient():
    """dS_T = None (loss on the outputs only) and S0 = None."""
    x, dO, _ = _case("rot2", B=1, T=9, H=1, d=4, seed=11)
    g1 = grad.backward_seq(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, None,
                           theta=x["theta"], decay="rot2")
    g2 = grad.backward_chunk(x["q"], x["k"], x["v"], x["w"], x["alpha"], x["beta"], dO, None,
                             theta=x["theta"], decay="rot2", chunk=4)
    for n in g1:
        assert np.max(np.abs(g1[n] - g2[n])) < 1e-11, n


def _gated_case(decay, B=1, T=5, H=2, d=4, seed=11):
    rng = np.random.default_rng(seed)
    C = d if decay == "diag" else d // 2
    x = dict(
        q=rng.standard_normal((B, T, H, d)),
        k=rng.standard_normal((B, T, H, d)),
        v=rng.standard_normal((B, T, H, d)),
        w=rng.uniform(0.2, 1.0, (B, T, H)),
        beta=rng.uniform(0.1, 0.9, (B, T, H)),
        x=rng.standard_normal((B, T, H, C)),
        a=rng.uniform(0.3, 1.5, (H,)),
        theta=None if decay == "diag" else rng.uniform(-3.0, 3.0, (B, T, H, C)),
        S0=rng.standard_normal((B, H, d, d)) * 0.3,
    )
    return x, rng.standard_normal((B, T, H, d)), rng.standard_normal((B, H, d, d))


GATED_NAMES = {"q": "dq", "k": "dk", "v": "dv", "w": "dw", "beta": "dbeta", "x": "dx", "a": "da",
               "theta": "dtheta", "S0": "dS0"}


@pytest.mark.parametrize("qk_l2norm", [True, False])
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_backward_gated_matches_finite_differences(decay, qk_l2norm):
    """backward_gated (chain rule through exp(-a softplus(x)) and the per-token
    q/k normalisation) against central differences of seq.forward_gated, every
    element of every input, the per-head scale a included."""
    x, dO, dS = _gated_case(decay, seed=11 + qk_l2norm)

    def loss(y):
        o, S = seq.forward_gated(y["q"], y["k"], y["v"], y["w"], y["x"], y["a"], y["beta"],
                                 theta=y["theta"], decay=decay, S0=y["S0"], qk_l2norm=qk_l2norm)
        return float(np.sum(dO * o) + np.sum(dS * S))

    g = grad.backward_gated(x["q"], x["k"], x["v"], x["w"], x["x"], x["a"], x["beta"], dO, dS,
                            theta=x["theta"], decay=decay, S0=x["S0"], qk_l2norm=qk_l2norm)
    assert set(g) == {n for k, n in GATED_NAMES.items() if x[k] is not None}
    h = 1e-5
    for name, gname in GATED_NAMES.items():
        if x[name] is None:
            continue
        fd = np.empty_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp, xm = dict(x), dict(x)
            xp[name], xm[name] = x[name].copy(), x[name].copy()
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        err = np.max(np.abs(fd - g[gname]) / np.maximum(1.0, np.abs(fd)))
        assert err < 1e-7, (decay, qk_l2norm, name, err)


def test_backward_gated_without_gate_or_norm_is_backward_seq():
    """a = 0 makes every decay 1 (and dx = 0); without normalisation the q, k, v,
    w, beta and S0 gradients are backward_seq's with alpha = 1, and da is the
    alpha gradient weighted by -softplus(x)."""
    x, dO, dS = _gated_case("diag", seed=21)
    a0 = np.zeros_like(x["a"])
    g = grad.backward_gated(x["q"], x["k"], x["v"], x["w"], x["x"], a0, x["beta"], dO, dS,
                            S0=x["S0"], qk_l2norm=False)
    ones = np.ones_like(x["x"])
    r = grad.backward_seq(x["q"], x["k"], x["v"], x["w"], ones, x["beta"], dO, dS, S0=x["S0"])
    for n in ("dq", "dk", "dv", "dw", "dbeta", "dS0"):
        assert np.array_equal(g[n], r[n]), n
    assert np.all(g["dx"] == 0)
    assert np.allclose(g["da"], np.sum(r["dalpha"] * -seq.softplus(x["x"]), axis=(0, 1, 3)),
                       rtol=1e-14, atol=0)
