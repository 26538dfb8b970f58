"""Parity of the partial-permutation forward (gdr_perm_fwd) with the fp64 oracle
(oracle/perm.py, pinned in test_oracle_perm.py by a simulated bounded stack).

Both sides read the same bf16 q, k, v and fp32 gates; the kernel keeps the
state and all arithmetic in fp32, so the bars are o <= 2e-2 (bf16 output) and
the state <= 1e-4 (max |x - ref| / max |ref| per tensor).

Cases: random stack moves with ragged lengths, both key widths, value widths
32 .. 256, a start state and in place; random partial permutations and maps
with repeated or out-of-range sources; maps one channel away from the identity
or a stack shift; the stack construction read back exactly
(push = shift down then write channel 0, pop = shift up, top = channel 0); the
workload's 128 heads on a prefix and at full size on sampled heads; a bitwise
rerun.
"""
import numpy as np
import pytest

from _gpu import dev, random_state
from oracle import perm
from oracle.errors import max_rel_err
from synth.gen import PERM_WORKLOADS, Workload, generate_perm, stack_moves

pytestmark = pytest.mark.gpu

TOL_O, TOL_S = 2e-2, 1e-4


def _wl(dk, dv=None, B=2, H=3, T=100, seed=500):
    return Workload("perm-test", B, H, T, dk, dv or dk, 64, "bf16", "perm", False, seed)


def run(x, S0=None, src=None, inplace=False, beta=None, q=None, k=None, v=None):
    import torch
    import recurrent_state_memory_amd as gdr
    bf = torch.bfloat16
    s0 = dev(S0)
    srcd = torch.from_numpy(np.ascontiguousarray(x.src if src is None else src)).to("cuda")
    o, S = gdr.gdr_perm_fwd(dev(x.q if q is None else q, bf), dev(x.k if k is None else k, bf),
                            dev(x.v if v is None else v, bf), dev(x.w),
                            srcd, dev(x.beta if beta is None else beta), S0=s0,
                            S_out=s0 if inplace else None)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def check(got, ref, what):
    eo, es = max_rel_err(got[0], ref[0]), max_rel_err(got[1], ref[1])
    print(f"{what}: err(o) = {eo:.2e} err(S) = {es:.2e}", flush=True)
    assert np.all(np.isfinite(got[0])) and eo <= TOL_O and es <= TOL_S, (what, eo, es)


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 100])
def test_perm_stack_moves_ragged(dk, T):
    x = generate_perm(_wl(dk, T=T, seed=500 + T + dk))
    S0 = random_state(2, 3, dk, dk, T)
    check(run(x, S0), perm.forward(x.q, x.k, x.v, x.w, x.src, x.beta, S0), f"perm d{dk} T={T}")


@pytest.mark.parametrize("dv", [32, 96, 256])
def test_perm_value_widths(dv):
    x = generate_perm(_wl(128, dv=dv, T=70, seed=510 + dv))
    check(run(x), perm.forward(x.q, x.k, x.v, x.w, x.src, x.beta), f"perm dv={dv}")


def test_perm_general_maps():
    """Random partial permutations, maps with repeated sources, and sources
    outside [0, dk) (zero columns)."""
    x = generate_perm(_wl(128, T=90, seed=520))
    rng = np.random.default_rng(521)
    B, T, H, dk = x.src.shape
    src = np.empty_like(x.src)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                kind = (b + t + h) % 3
                if kind == 0:     # partial permutation: a permutation with some drops
                    m = rng.permutation(dk)
                    m[rng.uniform(size=dk) < 0.1] = -1
                elif kind == 1:   # repeated sources
                    m = rng.integers(0, dk, dk)
                else:             # out of range both ways
                    m = rng.integers(-300, 300, dk)
                src[b, t, h] = m.astype(np.int16)
    S0 = random_state(B, H, dk, dk, 9)
    check(run(x, S0, src=src), perm.forward(x.q, x.k, x.v, x.w, src, x.beta, S0),
          "perm general maps")


@pytest.mark.parametrize("dk", [64, 128])
def test_perm_near_structured_maps(dk):
    """Maps one channel away from the identity, push or pop (which take the
    register path when exact) must take the general path; an out-of-range
    source where a shift empties a channel is still that shift."""
    x = generate_perm(_wl(dk, T=96, seed=560 + dk))
    rng = np.random.default_rng(561 + dk)
    B, T, H, _ = x.src.shape
    j = np.arange(dk)
    push, pop = np.where(j >= 1, j - 1, -1), np.where(j + 1 < dk, j + 1, -1)
    src = np.empty_like(x.src)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                kind = rng.integers(0, 7)
                m = [j, push, pop][kind % 3].copy()
                if kind in (3, 4, 5):            # one channel altered
                    c = rng.integers(0, dk)
                    m[c] = (m[c] + rng.integers(1, dk)) % dk if rng.uniform() < 0.7 else -1
                elif kind == 6:                   # push / pop with another "none" value
                    m = (push if rng.uniform() < 0.5 else pop).copy()
                    m[m < 0] = rng.choice([-7, dk, 300])
                src[b, t, h] = m.astype(np.int16)
    S0 = random_state(B, H, dk, dk, 11)
    check(run(x, S0, src=src), perm.forward(x.q, x.k, x.v, x.w, src, x.beta, S0),
          f"perm near-structured maps d{dk}")


def test_perm_bounded_stack_exact():
    """The stack construction with exact small integers: o reads the top exactly
    (bitwise) and the state holds the whole bounded stack."""
    rng = np.random.default_rng(530)
    B, T, H, dk, dv = 1, 160, 2, 64, 32
    op = np.where(rng.uniform(size=(B, T, H)) < 0.6, 0, rng.integers(1, 3, (B, T, H)))
    src = stack_moves(op, dk)
    e0 = np.zeros(dk, np.float32)
    e0[0] = 1.0
    q = np.broadcast_to(e0, (B, T, H, dk)).copy()
    v = rng.integers(1, 100, (B, T, H, dv)).astype(np.float32)
    beta = (op == 0).astype(np.float32)
    w = np.ones((B, T, H), np.float32)
    x = generate_perm(_wl(dk, dv=dv, B=B, H=H, T=T, seed=531))
    x.w = w
    o, S = run(x, src=src, beta=beta, q=q, k=q, v=v)
    o_r, S_r = perm.forward(q, q, v, w, src, beta)
    assert np.array_equal(o, o_r) and np.array_equal(S, S_r)


def test_perm_workload_prefix_all_heads():
    x = generate_perm(PERM_WORKLOADS["stack"], T=256)
    check(run(x), perm.forward(x.q, x.k, x.v, x.w, x.src, x.beta), "perm workload 256 tokens")


def test_perm_workload_full_size_sampled_heads():
    """8 x 16 x 4096, d = 128, as timed; three heads through the oracle."""
    x = generate_perm(PERM_WORKLOADS["stack"])
    o, S = run(x)
    assert np.all(np.isfinite(o))
    heads = [(0, 0), (4, 7), (7, 15)]
    og, Sg, orf, Srf = [], [], [], []
    for b, h in heads:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        r = perm.forward(x.q[sl], x.k[sl], x.v[sl], x.w[sl], x.src[sl], x.beta[sl])
        og.append(o[b, :, h]); Sg.append(S[b, h]); orf.append(r[0][0, :, 0]); Srf.append(r[1][0, 0])
    check((np.stack(og), np.stack(Sg)), (np.stack(orf), np.stack(Srf)), "perm full size (3 heads)")


def test_perm_inplace_and_rerun():
    x = generate_perm(_wl(128, T=75, seed=540))
    S0 = random_state(2, 3, 128, 128, 3)
    o1, S1 = run(x, S0)
    o2, S2 = run(x, S0, inplace=True)
    o3, S3 = run(x, S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    assert np.array_equal(o1, o3) and np.array_equal(S1, S3)
