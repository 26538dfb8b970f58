"""Parity of the gated backward (gdr_chunk_bwd_gated: gradients through the
decay activation exp(-a_h softplus(x)) and the per-token q/k normalisation)
with the fp64 oracle ``oracle.grad.backward_gated``, which is pinned by finite
differences on the CPU.  Every gradient of every head is compared, with the
bf16 bar of the other backward tests.
"""
import dataclasses

import numpy as np
import pytest

from _gpu import TOL, dev, random_state
from oracle import grad
from oracle.errors import max_rel_err
from synth.gen import WORKLOADS, bf16_round, generate_gated
from test_gpu_gated import _prenormalised, _spread_a, _wl

pytestmark = pytest.mark.gpu

NAMES = {"q": "dq", "k": "dk", "v": "dv", "w": "dw", "beta": "dbeta", "x": "dx", "a": "da",
         "theta": "dtheta", "S0": "dS0"}


def _upstream(x, seed):
    rng = np.random.default_rng(seed)
    B, T, H, dv = x.v.shape
    dO = bf16_round(rng.standard_normal((B, T, H, dv)).astype(np.float32))
    dS = (rng.standard_normal((B, H, dv, x.k.shape[-1])) / 8).astype(np.float32)
    return dO, dS


def check(x, dO, dS=None, S0=None, qk_l2norm=True, what=""):
    import torch
    import recurrent_state_memory_amd as gdr
    bf = torch.bfloat16
    got = gdr.gdr_chunk_bwd_gated(dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.x, bf),
                                  dev(x.a), dev(x.w), dev(x.beta), dev(dO, bf),
                                  theta=dev(x.theta), qk_l2norm=qk_l2norm, S0=dev(S0),
                                  grad_S=dev(dS))
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in got.items()}
    ref = grad.backward_gated(x.q, x.k, x.v, x.w, x.x, x.a, x.beta, dO, dS, theta=x.theta,
                              decay=x.wl.decay, S0=S0, qk_l2norm=qk_l2norm)
    errs = {}
    for name, rname in NAMES.items():
        if name not in got:
            continue
        assert np.all(np.isfinite(got[name])), (what, name)
        errs[name] = max_rel_err(got[name], ref[rname])
    print(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if v > TOL["bf16"]}
    assert not bad, (what, bad)


@pytest.mark.parametrize("qk_l2norm", [True, False])
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_bwd_gated(decay, dk, qk_l2norm):
    """Ragged tail (T = 100), S0 and grad_S set, a different a_h per head."""
    x = _spread_a(generate_gated(_wl(decay, dk, B=2, H=3, T=100, seed=171 + dk)))
    if not qk_l2norm:
        x = _prenormalised(x)
    dO, dS = _upstream(x, 9)
    S0 = random_state(2, 3, dk, dk, 10)
    check(x, dO, dS, S0, qk_l2norm, f"bwd gated {decay}/d{dk}/l2norm={qk_l2norm}")


@pytest.mark.parametrize("T", [1, 33])
def test_bwd_gated_short(T):
    """Fewer tokens than one block, and one block plus a token; no S0, no grad_S."""
    x = generate_gated(_wl("diag", 128, B=1, H=2, T=T, seed=181 + T))
    dO, _ = _upstream(x, 11)
    check(x, dO, what=f"bwd gated short T={T}")


def test_bwd_gated_strong_decay():
    """Large a_h and pre-activations drive some blocks' decay products below
    e^-40: those heads take the backward's token path."""
    x = _spread_a(generate_gated(_wl("diag", 128, B=1, H=3, T=130, seed=191)))
    x = dataclasses.replace(x, a=(x.a * 40.0).astype(np.float32))
    dO, dS = _upstream(x, 12)
    check(x, dO, dS, what="bwd gated strong decay")


def test_bwd_gated_layer_grid():
    """The layer's head count and width (B = 8, H = 16, d = 128) on a 128-token
    prefix: every gradient of every head, the per-head scale's sum over 1024
    token rows included."""
    x = generate_gated(WORKLOADS["layer"], T=128)
    dO, dS = _upstream(x, 13)
    check(x, dO, dS, what="bwd gated layer grid")
