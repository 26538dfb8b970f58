"""Parity of the gated forward (decay activation and q/k normalisation in the
kernel) with the fp64 oracle, through gdr_chunk_fwd_gated.

The oracle is oracle.seq.forward_gated: the same sequential definition as the
plain forward, fed with exp(-a_h softplus(x)) and with q, k divided by
sqrt(sum of squares + 1e-6), all in fp64 from the same bf16 inputs.  Each case
checks every output of every head against the bf16 bar of test_gpu_parity.py.
"""
import dataclasses

import numpy as np
import pytest

from _gpu import TOL, dev, random_state
from oracle import seq
from oracle.errors import max_rel_err
from synth.gen import WORKLOADS, Workload, bf16_round, generate_gated

pytestmark = pytest.mark.gpu


def _wl(decay, dk, B=2, H=3, T=300, seed=81):
    return Workload("gated", B, H, T, dk, dk, 64, "bf16", decay, False, seed,
                    decay_scale=0.1 if decay == "diag" else 0.05)


def _spread_a(x):
    """Per-head scales that differ (0.5 .. 1.5 times the recipe's), so a head
    reading another head's a_h shows."""
    H = x.a.shape[0]
    return dataclasses.replace(x, a=(x.a * np.linspace(0.5, 1.5, H)).astype(np.float32))


def _prenormalised(x):
    """q, k already L2-normalised (then rounded to bf16): the inputs of a call
    with qk_l2norm off, whose keys must have unit scale for a stable erase."""
    return dataclasses.replace(x, q=bf16_round(seq.l2_normalise(x.q).astype(np.float32)),
                               k=bf16_round(seq.l2_normalise(x.k).astype(np.float32)))


def run_gated(x, qk_l2norm=True, S0=None, chunk=64):
    import torch
    import recurrent_state_memory_amd as gdr
    bf = torch.bfloat16
    o, S = gdr.gdr_chunk_fwd_gated(
        dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.x, bf), dev(x.a), dev(x.w), dev(x.beta),
        theta=dev(x.theta), qk_l2norm=qk_l2norm, S0=dev(S0), chunk=chunk)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def oracle_gated(x, qk_l2norm=True, S0=None):
    return seq.forward_gated(x.q, x.k, x.v, x.w, x.x, x.a, x.beta, theta=x.theta,
                             decay=x.wl.decay, S0=S0, qk_l2norm=qk_l2norm)


def check(x, qk_l2norm=True, S0=None, what="", chunk=64):
    o, S = run_gated(x, qk_l2norm, S0, chunk)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)), what
    o_r, S_r = oracle_gated(x, qk_l2norm, S0)
    eo, es = max_rel_err(o, o_r), max_rel_err(S, S_r)
    print(f"{what}: err(o) = {eo:.3e}  err(S) = {es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (what, eo, es)
    return o, S


@pytest.mark.parametrize("qk_l2norm", [True, False])
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_gated_forward(decay, dk, qk_l2norm):
    """Ragged tail (T = 300), non-zero S0, a different a_h per head."""
    x = _spread_a(generate_gated(_wl(decay, dk, seed=81 + dk)))
    if not qk_l2norm:
        x = _prenormalised(x)
    S0 = random_state(2, 3, dk, dk, 4)
    check(x, qk_l2norm, S0, f"gated {decay}/d{dk}/l2norm={qk_l2norm}")


@pytest.mark.parametrize("T", [1, 31, 33, 64, 97])
def test_gated_short_sequences(T):
    """Fewer tokens than one pipeline fill (the three-chunk unroll's tails)."""
    x = _spread_a(generate_gated(_wl("diag", 128, T=T, seed=90 + T)))
    check(x, True, None, f"gated short T={T}")


@pytest.mark.parametrize("chunk", [16, 32, 128])
def test_gated_chunk_argument(chunk):
    """The chunk argument sets no arithmetic of the plain-erase path: same
    result for every supported value."""
    x = _spread_a(generate_gated(_wl("rot2", 128, T=200, seed=95)))
    check(x, True, None, f"gated chunk={chunk}", chunk=chunk)


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_gated_strong_decay(decay):
    """Pre-activations that make the decay tiny or exactly zero: x = +60 on
    every 41st token, which with a_h = 5 (head 0) gives exp(-300) = 0 in fp32,
    a reset; a_h = 5 and a_h = 40 (heads 0 and 2) push whole chunks out of the
    split form's range, so they take the token path, with the normalisation
    applied there too; head 1 keeps the recipe's scale (fast path)."""
    x = generate_gated(_wl(decay, 128, T=260, seed=97))
    xx = x.x.copy()
    xx[:, 7::41] = 60.0
    a = x.a.copy()
    a[0] = 5.0
    a[2] = 40.0
    x = dataclasses.replace(x, x=bf16_round(xx), a=a.astype(np.float32))
    S0 = random_state(2, 3, 128, 128, 6)
    check(x, True, S0, f"gated strong {decay}")


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_gated_layer_grid(decay):
    """The full-size layer launch shape (B = 8, H = 16, d = 128: 64 value
    channels per workgroup) on a 512-token prefix: every head."""
    wl = WORKLOADS["layer"] if decay == "diag" else WORKLOADS["rot"].replace(B=8)
    x = _spread_a(generate_gated(wl, T=512))
    check(x, True, None, f"gated layer grid {decay}")


def test_gated_matches_plain_on_activated_inputs():
    """The gated call equals the plain forward fed with the activated decay and
    the normalised q, k (both computed here in fp32 numpy, rounded as the
    plain path takes them): a consistency check between the two entry points."""
    import torch
    import recurrent_state_memory_amd as gdr
    x = _spread_a(generate_gated(_wl("diag", 128, T=256, seed=99)))
    o_g, S_g = run_gated(x, True)
    xf = x.x.astype(np.float64)
    sp = np.maximum(xf, 0) + np.log1p(np.exp(-np.abs(xf)))
    alpha = np.exp(-x.a[:, None].astype(np.float64) * sp).astype(np.float32)
    nrm = lambda t: (t / np.sqrt((t.astype(np.float64) ** 2).sum(-1, keepdims=True) + 1e-6))
    bf = torch.bfloat16
    o_p, S_p = gdr.gdr_chunk_fwd(dev(nrm(x.q), bf), dev(nrm(x.k), bf), dev(x.v, bf), dev(alpha),
                                 dev(x.w), dev(x.beta))
    torch.cuda.synchronize()
    assert max_rel_err(o_g, o_p.float().cpu().numpy()) <= TOL["bf16"]
    assert max_rel_err(S_g, S_p.cpu().numpy()) <= TOL["bf16"]
