"""Parity of the HIP backward (gdr_chunk_bwd) with the fp64 gradient oracle.

The oracle is oracle.grad.backward_seq (reverse mode through the token
recurrence, pinned by finite differences in test_oracle_grad.py), run on the
same bf16-rounded inputs and upstream gradients.  Every gradient of every head
is compared with the max-normalised error of test_gpu_parity.py; the bar is
the bf16 one (the backward's block-start states come from the forward's bf16
matrix products).
"""
import dataclasses

import numpy as np
import pytest

from _gpu import TOL, dev, random_state
from oracle import grad
from oracle.errors import max_rel_err
from synth.gen import WORKLOADS, Workload, bf16_round, generate

pytestmark = pytest.mark.gpu


def _wl(decay, dk, B=2, H=2, T=100, seed=121):
    return Workload("bwd", B, H, T, dk, dk, 64, "bf16", decay, False, seed,
                    decay_scale=0.1 if decay == "diag" else 0.05)


def run_bwd(x, dO, S0=None, dS=None):
    import torch
    import recurrent_state_memory_amd as gdr
    bf = torch.bfloat16
    g = gdr.gdr_chunk_bwd(dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.alpha), dev(x.w),
                          dev(x.beta), dev(dO, bf), theta=dev(x.theta), S0=dev(S0),
                          grad_S=dev(dS))
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}


def oracle_bwd(x, dO, S0=None, dS=None):
    return grad.backward_seq(x.q, x.k, x.v, x.w, x.alpha, x.beta, dO, dS, theta=x.theta,
                             decay=x.wl.decay, S0=S0)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "w": "dw", "beta": "dbeta", "alpha": "dalpha",
         "theta": "dtheta", "S0": "dS0"}


def check(x, dO, S0=None, dS=None, what="", tol=None):
    tol = TOL["bf16"] if tol is None else tol
    got = run_bwd(x, dO, S0, dS)
    ref = oracle_bwd(x, dO, S0, dS)
    errs = {}
    for name, rname in NAMES.items():
        if name not in got:
            continue
        assert np.all(np.isfinite(got[name])), (what, name)
        errs[name] = max_rel_err(got[name], ref[rname])
    print(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, (what, bad)


def _upstream(x, seed):
    rng = np.random.default_rng(seed)
    B, T, H, dv = x.v.shape
    dO = bf16_round(rng.standard_normal((B, T, H, dv)).astype(np.float32))
    dS = (rng.standard_normal((B, H, dv, x.k.shape[-1])) / 8).astype(np.float32)
    return dO, dS


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_bwd(decay, dk):
    """Ragged tail (T = 100: three full blocks and 4 tokens), S0 and grad_S set."""
    x = generate(_wl(decay, dk, seed=121 + dk))
    dO, dS = _upstream(x, 5)
    S0 = random_state(2, 2, dk, dk, 8)
    check(x, dO, S0, dS, f"bwd {decay}/d{dk}")


@pytest.mark.parametrize("T", [1, 31, 32, 33])
def test_bwd_short(T):
    """Fewer tokens than one block, exactly one, one plus a token; no S0, no
    grad_S."""
    x = generate(_wl("diag", 128, T=T, seed=130 + T))
    dO, _ = _upstream(x, 6)
    check(x, dO, None, None, f"bwd short T={T}")


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_bwd_layer_grid(decay):
    """The layer's head count and width (B = 8, H = 16, d = 128) on a 256-token
    prefix: every gradient of every head."""
    wl = WORKLOADS["layer"] if decay == "diag" else WORKLOADS["rot"].replace(B=8)
    x = generate(wl, T=256)
    dO, dS = _upstream(x, 7)
    check(x, dO, None, dS, f"bwd layer grid {decay}")
