"""Parity of the reflection-block transition (GDR_DECAY_DIHEDRAL) with the fp64
oracle.

The SFDA page's finite-state expressivity result adds reflections to the 2x2
rotation-decay blocks so that the family realises dihedral memory; a block
whose gamma has its sign bit set is |gamma| R(theta) F, F = Diag(1, -1).  The
pipelined forward and the decode step take it; these tests check:

* ragged lengths, S0, both head widths, every head (max-normalised bf16 bar
  of test_gpu_parity.py);
* the dihedral workload's full size (4 x 16 heads, 8192 tokens, d = 128) in
  the launch the benchmark times, on sampled heads the oracle runs one by one;
* the group law: with beta = 0 and |gamma| = 1 the state of each key pair is
  S0 times the D_n element folded by integer arithmetic (no oracle involved),
  to fp32 accuracy -- a swapped product order or a wrong reflection fails;
* strong forgetting (every chunk on the kernel's token path) and exact zeros;
* the decode step, alone and chained against the chunked forward.
"""
import numpy as np
import pytest

from _gpu import TOL, compare_heads, dev, io_dtype, oracle_heads, random_state, run_gpu
from oracle import seq
from oracle.errors import max_rel_err
from synth.gen import WORKLOADS, Workload, generate, generate_decode
from test_gpu_strong_decay import strong_transition

pytestmark = pytest.mark.gpu


def _wl(dk, B=2, H=3, T=200, chunk=64, seed=71, io="bf16"):
    return Workload("dihedral-test", B, H, T, dk, dk, chunk, io, "dihedral", False, seed,
                    decay_scale=0.05)


def run_refl(x, S0=None):
    """gdr_chunk_fwd with reflections on (the shared helper passes rot2)."""
    import torch
    import recurrent_state_memory_amd as gdr
    bf = torch.bfloat16
    o, S = gdr.gdr_chunk_fwd(dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.alpha),
                             dev(x.w), dev(x.beta), theta=dev(x.theta), S0=dev(S0),
                             chunk=x.wl.chunk, reflections=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("T", [1, 31, 33, 200])
def test_dihedral_ragged(dk, T):
    """Fewer tokens than one block, a block and a token, several blocks plus a
    ragged tail; S0 set; every head."""
    x = generate(_wl(dk, T=T, seed=71 + T + dk))
    assert np.any(np.signbit(x.alpha)) and np.any(~np.signbit(x.alpha))
    S0 = random_state(2, 3, dk, dk, 17)
    o, S = run_refl(x, S0)
    compare_heads(o, S, oracle_heads(x, S0=S0), TOL["bf16"], f"dihedral d{dk} T={T}")


def test_dihedral_differs_from_rotation():
    """The same inputs read as plain rotations (sign ignored by taking |gamma|)
    give another state: the reflection bit is not dropped on the way in."""
    x = generate(_wl(128, T=96, seed=80))
    o_r, S_r = run_refl(x)
    import dataclasses
    y = dataclasses.replace(x, alpha=np.abs(x.alpha).astype(np.float32))
    o_p, S_p = run_gpu(y)                     # rot2 launch on |gamma|
    assert max_rel_err(S_r, S_p) > 0.1


def test_dihedral_layer_grid():
    """The dihedral workload's head grid (B = 4, H = 16, d = 128) on a
    512-token prefix: every head."""
    x = generate(WORKLOADS["dihedral"], T=512)
    o, S = run_refl(x)
    compare_heads(o, S, oracle_heads(x), TOL["bf16"], "dihedral layer grid")


def test_dihedral_full_size_sampled_heads():
    """4 x 16 heads of 8192 tokens, d = 128, as timed; the oracle runs three
    heads (first, last and one in the middle) on the full length."""
    x = generate(WORKLOADS["dihedral"])
    o, S = run_refl(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    heads = [(0, 0), (1, 7), (3, 15)]
    compare_heads(o, S, oracle_heads(x, heads=heads), TOL["bf16"], "dihedral full size")


def _fold(a_idx, b_bit, n):
    """D_n law (a1, b1)(a2, b2) = (a1 + (-1)^b1 a2 mod n, b1 xor b2), folded
    left to right over the token axis (integers only)."""
    a = np.zeros(a_idx.shape[1:], np.int64)
    b = np.zeros(a_idx.shape[1:], np.int64)
    for t in range(a_idx.shape[0]):
        a = (a + np.where(b == 1, -a_idx[t], a_idx[t])) % n
        b = b ^ b_bit[t]
    return a, b


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("n", [3, 6])
def test_dihedral_group_law(dk, n):
    """beta = w = 0, gamma = +-1, theta = 2 pi a / n: S_T[:, pair j] =
    S0[:, pair j] R(2 pi a_j / n) F^(b_j) with (a_j, b_j) the D_n product of
    the tokens' elements; fp32 transition arithmetic over 150 tokens."""
    import torch
    import recurrent_state_memory_amd as gdr
    rng = np.random.default_rng(200 + n + dk)
    B, T, H = 2, 150, 3
    a_idx = rng.integers(0, n, (T, B, H, dk // 2))
    b_bit = rng.integers(0, 2, (T, B, H, dk // 2))
    theta = (2 * np.pi * a_idx / n).transpose(1, 0, 2, 3).astype(np.float32)
    gam = np.where(b_bit == 1, -1.0, 1.0).transpose(1, 0, 2, 3).astype(np.float32)
    S0 = random_state(B, H, dk, dk, 3)
    bf = torch.bfloat16
    qkv = rng.standard_normal((B, T, H, dk)).astype(np.float32) / np.sqrt(dk)
    z = np.zeros((B, T, H), np.float32)
    _, S = gdr.gdr_chunk_fwd(dev(qkv, bf), dev(qkv, bf), dev(qkv, bf), dev(gam), dev(z),
                             dev(z), theta=dev(theta), S0=dev(S0), reflections=True)
    torch.cuda.synchronize()
    S = S.cpu().numpy()
    a, b = _fold(a_idx, b_bit, n)                       # [B, H, dk/2]
    ph = 2 * np.pi * a / n
    c, s = np.cos(ph), np.sin(ph)
    sg = np.where(b == 1, -1.0, 1.0)
    # [x, y] R(ph) F^b = [x c + y s, (-x s + y c) sg]
    x0, y0 = S0[..., 0::2].astype(np.float64), S0[..., 1::2].astype(np.float64)
    want = np.empty_like(S0, dtype=np.float64)
    want[..., 0::2] = x0 * c[:, :, None, :] + y0 * s[:, :, None, :]
    want[..., 1::2] = (-x0 * s[:, :, None, :] + y0 * c[:, :, None, :]) * sg[:, :, None, :]
    err = max_rel_err(S, want)
    print(f"group law D_{n} d{dk}: err = {err:.2e}", flush=True)
    assert err < 1e-4


@pytest.mark.parametrize("pattern", ["uniform", "bursts", "reset", "cum150"])
@pytest.mark.parametrize("dk", [64, 128])
def test_dihedral_strong_decay(dk, pattern):
    """Strong forgetting with the reflection signs kept: the token path and the
    fast path mixed inside one sequence (patterns of test_gpu_strong_decay.py;
    'reset' has exact zeros of either sign)."""
    x = generate(_wl(dk, T=200, seed=90 + dk))
    mag = strong_transition(np.abs(x.alpha), pattern, 64, seed=dk)
    import dataclasses
    x = dataclasses.replace(x, alpha=np.where(np.signbit(x.alpha), -mag, mag).astype(np.float32))
    S0 = random_state(2, 3, dk, dk, 5)
    o, S = run_refl(x, S0)
    compare_heads(o, S, oracle_heads(x, S0=S0), TOL["bf16"], f"dihedral strong {pattern} d{dk}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk", [32, 64, 128])
def test_dihedral_decode(io, dk):
    import torch
    import recurrent_state_memory_amd as gdr
    wl = _wl(dk, io=io)
    d = generate_decode(wl, N=7, rng=np.random.default_rng(300 + dk))
    assert np.any(np.signbit(d.alpha))
    iot = io_dtype(io)
    S = dev(d.S)
    o = gdr.gdr_step_decode(S, dev(d.q, iot), dev(d.k, iot), dev(d.v, iot), dev(d.alpha),
                            dev(d.beta), dev(d.w), theta=dev(d.theta), reflections=True)
    torch.cuda.synchronize()
    S_r, o_r = seq.decode_step(d.S, d.q, d.k, d.v, d.beta, d.w, d.alpha, d.theta, "dihedral")
    eo = max_rel_err(o.float().cpu().numpy(), o_r)
    es = max_rel_err(S.cpu().numpy(), S_r)
    print(f"dihedral decode {io} d{dk}: err(o) = {eo:.2e} err(S) = {es:.2e}", flush=True)
    assert eo <= TOL[io] and es <= TOL[io]


def test_dihedral_decode_chain_equals_chunk_fwd():
    """T decode steps from S0 reproduce the chunked forward with reflections."""
    import torch
    import recurrent_state_memory_amd as gdr
    x = generate(_wl(128, B=2, H=2, T=40, seed=95))
    S0 = random_state(2, 2, 128, 128, 95)
    o_c, S_c = run_refl(x, S0)
    bf = torch.bfloat16
    S = dev(S0)
    outs = []
    for t in range(x.wl.T):
        sl = (slice(None), t)
        outs.append(gdr.gdr_step_decode(
            S, dev(x.q[sl], bf), dev(x.k[sl], bf), dev(x.v[sl], bf), dev(x.alpha[sl]),
            dev(x.beta[sl]), dev(x.w[sl]), theta=dev(x.theta[sl]), reflections=True).float())
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1).cpu().numpy()
    assert max_rel_err(o_d, o_c) <= TOL["bf16"]
    assert max_rel_err(S.cpu().numpy(), S_c) <= TOL["bf16"]
