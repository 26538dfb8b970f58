"""Parity of the HIP path with the fp64 oracle under strong forgetting.

Per-token decays far below the synthetic recipe's push a chunk's running
product Gamma_L out of fp32's range; the split form (Gamma_r, Gamma_r^{-1})
would overflow there, so such chunks must take the kernels' token path.  These
cases mix both paths inside one sequence:

* ``uniform``: alpha (or the rotation magnitude gamma) ~ U(1e-3, 0.05) on every
  token and channel -- every chunk on the token path;
* ``bursts``: the recipe's mild decay, except runs of strong decay in a few
  channels of chosen chunks -- fast and token chunks alternate;
* ``reset``: exact zeros (alpha = 0) on every 37th token in a third of the
  channels, and 1e-40 (an fp32 subnormal) on every 53rd token elsewhere;
* ``cum150``: all channels at alpha = e^-5 over one whole 64-token stretch
  (cumulative log-decay below -150 inside any 32-token block).

Plus the pure reset of the SFDA page's register construction (finite-state
expressivity, with delta correction): alpha = 0, beta = w = 1, where the state
holds exactly the last write.  Tolerances as in test_gpu_parity.py.
"""
import dataclasses

import numpy as np
import pytest

from _gpu import TOL, compare_heads, dev, io_dtype, oracle_heads, random_state, run_gpu
from oracle import seq
from oracle.errors import max_rel_err
from synth.gen import Workload, generate

pytestmark = pytest.mark.gpu


def _wl(io, decay, dk, B=2, H=3, T=200, chunk=64, content=False, seed=51):
    return Workload("strong", B, H, T, dk, dk, chunk, io, decay, content, seed,
                    decay_scale=0.1 if decay == "diag" else 0.05)


def strong_transition(a, pattern, chunk, seed):
    """Apply a strong-decay pattern to a [B,T,H,C] decay array (C = d_k or d_k/2)."""
    rng = np.random.default_rng(seed)
    a = a.copy()
    B, T, H, C = a.shape
    if pattern == "uniform":
        a[:] = rng.uniform(1e-3, 0.05, a.shape)
    elif pattern == "bursts":
        # strong runs in a quarter of the channels of every other chunk
        for c0 in range(0, T, 2 * chunk):
            t1 = min(T, c0 + chunk)
            ch = rng.choice(C, size=max(1, C // 4), replace=False)
            sub = a[:, c0:t1][..., ch]
            a[:, c0:t1, :, ch] = rng.uniform(1e-3, 0.05, sub.shape).astype(np.float32)
    elif pattern == "reset":
        third = np.arange(C) < C // 3
        a[:, 5::37, :, third] = 0.0
        a[:, 11::53, :, ~third] = np.float32(1e-40)
    elif pattern == "cum150":
        t0 = min(chunk // 2, T - 1)
        a[:, t0:t0 + 64] = np.float32(np.exp(-5.0))
    else:
        raise ValueError(pattern)
    return a.astype(np.float32)


@pytest.mark.parametrize("pattern", ["uniform", "bursts", "reset", "cum150"])
@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("decay", ["diag", "rot2"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_strong_decay(io, decay, dk, pattern):
    """Both chunked kernels (bf16 d in {64, 128}: pipelined; fp32 or d = 32:
    sequential stages) against the oracle, ragged tail, non-zero S0."""
    chunk = 32 if io == "f32" and dk == 128 else 64
    x = generate(_wl(io, decay, dk, T=4 * chunk + 9, chunk=chunk, seed=51 + dk))
    x = dataclasses.replace(x, alpha=strong_transition(x.alpha, pattern, chunk, seed=dk))
    S0 = random_state(2, 3, dk, dk, 9)
    o, S = run_gpu(x, S0=S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    compare_heads(o, S, oracle_heads(x, S0=S0), TOL[io], f"strong {pattern} {io}/{decay}/d{dk}")


@pytest.mark.parametrize("io,dk,chunk", [("bf16", 128, 128), ("bf16", 64, 32), ("bf16", 128, 16),
                                         ("f32", 64, 64), ("f32", 128, 16)])
@pytest.mark.parametrize("pattern", ["bursts", "reset"])
def test_strong_decay_content_aware(io, dk, chunk, pattern):
    """Content-aware erase (projection std 1.0) with strong-decay chunks: the window
    means must come out of the token path too."""
    wl = _wl(io, "diag", dk, B=2, H=2, T=4 * chunk + 7, chunk=chunk, content=True, seed=61)
    x = generate(wl, ub_std=1.0)
    x = dataclasses.replace(x, alpha=strong_transition(x.alpha, pattern, 32, seed=7))
    o, S = run_gpu(x)
    compare_heads(o, S, oracle_heads(x), TOL[io], f"strong content {pattern} {io}/d{dk}/L{chunk}")


@pytest.mark.parametrize("decay", ["diag", "rot2"])
@pytest.mark.parametrize("io,dk", [("bf16", 128), ("bf16", 64), ("f32", 128), ("bf16", 32)])
def test_pure_reset(io, decay, dk):
    """alpha = 0 (rotation magnitude 0), beta = w = 1: the state is exactly the last
    write v_t k_t^T, whatever S0 was (SFDA register/reset construction)."""
    x = generate(_wl(io, decay, dk, T=150, chunk=64, seed=71))
    ones = np.ones_like(x.w)
    x = dataclasses.replace(x, alpha=np.zeros_like(x.alpha), beta=ones, w=ones)
    S0 = random_state(2, 3, dk, dk, 3)
    o, S = run_gpu(x, S0=S0)
    compare_heads(o, S, oracle_heads(x, S0=S0), TOL[io], f"pure reset {io}/{decay}/d{dk}")
    # closed form: with a zero transition the erase acts on nothing, so
    # S_t = v_t k_t^T and o_t = v_t (k_t . q_t) exactly, for any key norm
    k, q, v = (a.astype(np.float64) for a in (x.k, x.q, x.v))
    o_ref = v * np.sum(k * q, axis=-1)[..., None]
    S_ref = v[:, -1, :, :, None] * k[:, -1, :, None, :]
    assert max_rel_err(o, o_ref) <= TOL[io]
    assert max_rel_err(S, S_ref) <= TOL[io]


def test_strong_decay_full_layer_grid():
    """The full-size layer launch (B=8, H=16, d=128, bf16, 64 value channels per
    workgroup) on a 1024-token prefix with strong-decay bursts: every head."""
    from synth.gen import WORKLOADS
    x = generate(WORKLOADS["layer"], T=1024)
    x = dataclasses.replace(x, alpha=strong_transition(x.alpha, "bursts", 64, seed=5))
    o, S = run_gpu(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    compare_heads(o, S, oracle_heads(x), TOL["bf16"], "strong layer grid")


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_decode_reset(decay):
    """Decode with a zero transition and beta = w = 1 keeps exactly v k^T."""
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import generate_decode
    d = generate_decode(_wl("bf16", decay, 128), N=5, rng=np.random.default_rng(2))
    S = dev(d.S)
    one = np.ones_like(d.beta)
    o = gdr.gdr_step_decode(S, dev(d.q, torch.bfloat16), dev(d.k, torch.bfloat16),
                            dev(d.v, torch.bfloat16), dev(np.zeros_like(d.alpha)), dev(one),
                            dev(one), theta=dev(d.theta))
    torch.cuda.synchronize()
    S_r, o_r = seq.decode_step(d.S, d.q, d.k, d.v, one, one, np.zeros_like(d.alpha), d.theta, decay)
    assert max_rel_err(S.cpu().numpy(), S_r) <= TOL["bf16"]
    assert max_rel_err(o.float().cpu().numpy(), o_r) <= TOL["bf16"]
