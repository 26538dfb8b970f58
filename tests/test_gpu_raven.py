"""Parity of the Raven slot-memory forward (gdr_raven_fwd) with the fp64 oracle
(oracle/raven.py, pinned in test_oracle_raven.py).

Both sides read the same bf16 q, k, v and router logits and the same fp32
decay rates.  Bars (max |x - ref| / max |ref| per tensor, as in
test_gpu_parity.py): the bf16 output o within 2e-2; the fp32 slot states within
1e-3 (their update coefficients enter the matrix cores as a bf16 pair, so they
keep nearly fp32 accuracy).

Cases: ragged lengths around the 32-token chunk, start states, both widths,
top-K of 1, 3 and 8; the workload's 128 heads on a prefix and its full size on
sampled heads; the page's two extremes -- one-hot routing with full
replacement (sliding-window attention) and strong decay, which take the
exact per-chunk path -- mixed with mild chunks; logits with many exact ties;
frozen slots (a = 0) bitwise; in-place states; a bitwise rerun.
"""
import numpy as np
import pytest

from _gpu import dev
from oracle import raven
from oracle.errors import max_rel_err
from synth.gen import RAVEN_WORKLOADS, RavenWorkload, bf16_round, generate_raven

pytestmark = pytest.mark.gpu

TOL_O, TOL_S = 2e-2, 1e-3


def _wl(d, B=2, H=3, T=100, topk=8, seed=400, a_scale=1.0):
    return RavenWorkload("raven-test", B, H, T, d, d, 64, topk, seed, a_scale)


def _start(x, seed):
    rng = np.random.default_rng(seed)
    B, H, M, d = x.wl.B, x.wl.H, x.wl.slots, x.wl.dk
    return ((rng.standard_normal((B, H, M, d)) / np.sqrt(d)).astype(np.float32),
            rng.standard_normal((B, H, M, d)).astype(np.float32))


def run(x, Sk0=None, Sv0=None, a=None, z=None, scale=None, inplace=False):
    import torch
    import recurrent_state_memory_amd as gdr
    bf = torch.bfloat16
    sk, sv = dev(Sk0), dev(Sv0)
    o, Sk, Sv = gdr.gdr_raven_fwd(
        dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.z if z is None else z, bf),
        dev(x.a if a is None else a), topk=x.wl.topk, scale=x.wl.scale if scale is None else scale,
        Sk0=sk, Sv0=sv, Sk_out=sk if inplace else None, Sv_out=sv if inplace else None)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), Sk.cpu().numpy(), Sv.cpu().numpy()


def oracle(x, Sk0=None, Sv0=None, a=None, z=None, scale=None, heads=None):
    a = x.a if a is None else a
    z = x.z if z is None else z
    scale = x.wl.scale if scale is None else scale
    if heads is None:
        return raven.forward(x.q, x.k, x.v, z, a, x.wl.topk, scale, Sk0, Sv0)
    out = {}
    for b, h in heads:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        r = raven.forward(x.q[sl], x.k[sl], x.v[sl], z[sl], a[sl], x.wl.topk, scale,
                          None if Sk0 is None else Sk0[b:b + 1, h:h + 1],
                          None if Sv0 is None else Sv0[b:b + 1, h:h + 1])
        out[(b, h)] = (r[0][0, :, 0], r[1][0, 0], r[2][0, 0])
    return out


def check(got, ref, what):
    eo, ek, ev = (max_rel_err(g, r) for g, r in zip(got, ref))
    print(f"{what}: err(o) = {eo:.2e} err(Sk) = {ek:.2e} err(Sv) = {ev:.2e}", flush=True)
    assert np.all(np.isfinite(got[0])), what
    assert eo <= TOL_O and ek <= TOL_S and ev <= TOL_S, (what, eo, ek, ev)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 100])
def test_raven_ragged(d, T):
    x = generate_raven(_wl(d, T=T, seed=400 + T + d))
    Sk0, Sv0 = _start(x, T)
    check(run(x, Sk0, Sv0), oracle(x, Sk0, Sv0), f"raven d{d} T={T}")


@pytest.mark.parametrize("topk", [1, 3])
def test_raven_topk(topk):
    x = generate_raven(_wl(128, T=70, topk=topk, seed=410 + topk))
    check(run(x), oracle(x), f"raven top-{topk} from zero slots")


def test_raven_workload_heads_prefix():
    """The workload's 8 x 16 heads (d = 128, 64 slots, top-8) on 256 tokens."""
    x = generate_raven(RAVEN_WORKLOADS["raven"], T=256)
    check(run(x), oracle(x), "raven workload 256-token prefix")


def test_raven_workload_full_size_sampled_heads():
    """8 x 16 x 4096, as timed; the oracle runs three heads on the full length."""
    x = generate_raven(RAVEN_WORKLOADS["raven"])
    o, Sk, Sv = run(x)
    assert np.all(np.isfinite(o))
    heads = [(0, 0), (3, 9), (7, 15)]
    ref = oracle(x, heads=heads)
    got = (np.stack([o[b, :, h] for b, h in heads]), np.stack([Sk[b, h] for b, h in heads]),
           np.stack([Sv[b, h] for b, h in heads]))
    want = tuple(np.stack([ref[k][i] for k in heads]) for i in range(3))
    check(got, want, "raven full size (3 heads)")


def test_raven_one_hot_full_replacement():
    """K = 1, slot t mod 64 on top, a = -1e30: the slots hold the last 64 tokens
    (sliding-window attention; every chunk has factors of 0, the exact path)."""
    x = generate_raven(_wl(128, T=200, topk=1, seed=420))
    B, T, H, M = x.z.shape
    z = np.full(x.z.shape, -4.0, np.float32)
    for t in range(T):
        z[:, t, :, t % M] = 4.0
    a = np.full(x.a.shape, -1e30, np.float32)
    check(run(x, z=z, a=a), oracle(x, z=z, a=a), "raven one-hot full replacement")


@pytest.mark.parametrize("pattern", ["strong", "mixed", "zeros"])
def test_raven_strong_decay(pattern):
    """strong: a ~ -U(20, 200) everywhere (products below e^-40: exact path);
    mixed: such rates only on tokens of every third chunk, so fast and exact
    chunks alternate; zeros: a = -1e30 on every 7th token."""
    x = generate_raven(_wl(128, T=160, seed=430))
    rng = np.random.default_rng(431)
    a = x.a.copy()
    if pattern == "strong":
        a = -rng.uniform(20, 200, a.shape).astype(np.float32)
    elif pattern == "mixed":
        for c0 in range(0, a.shape[1], 96):
            a[:, c0:c0 + 32] = -rng.uniform(20, 200, a[:, c0:c0 + 32].shape)
    else:
        a[:, ::7] = -1e30
    Sk0, Sv0 = _start(x, 5)
    check(run(x, Sk0, Sv0, a=a), oracle(x, Sk0, Sv0, a=a), f"raven strong decay {pattern}")


def test_raven_ties_in_router():
    """Logits on a coarse grid (many exact ties, including -0 and +0): the lower
    slot wins a tie on both sides."""
    x = generate_raven(_wl(64, T=90, topk=8, seed=440))
    rng = np.random.default_rng(441)
    z = (np.round(rng.standard_normal(x.z.shape) * 2) / 2).astype(np.float32)
    z[z == 0] = np.where(rng.uniform(size=np.count_nonzero(z == 0)) < 0.5, -0.0, 0.0)
    z = bf16_round(z)
    check(run(x, z=z), oracle(x, z=z), "raven router ties")


def test_raven_frozen_slots_bitwise():
    """a = 0: every factor is exactly 1, nothing is written; the states come back
    bitwise, and o is attention over the start slots."""
    x = generate_raven(_wl(128, T=50, seed=450))
    Sk0, Sv0 = _start(x, 6)
    a = np.zeros(x.a.shape, np.float32)
    o, Sk, Sv = run(x, Sk0, Sv0, a=a)
    assert np.array_equal(Sk, Sk0) and np.array_equal(Sv, Sv0)
    check((o, Sk, Sv), oracle(x, Sk0, Sv0, a=a), "raven frozen")


def test_raven_inplace_and_rerun():
    """States written over the start states; a second call is bitwise equal."""
    x = generate_raven(_wl(128, T=75, seed=460))
    Sk0, Sv0 = _start(x, 7)
    o1, k1, v1 = run(x, Sk0, Sv0)
    o2, k2, v2 = run(x, Sk0, Sv0, inplace=True)
    o3, k3, v3 = run(x, Sk0, Sv0)
    assert np.array_equal(o1, o2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert np.array_equal(o1, o3) and np.array_equal(k1, k3) and np.array_equal(v1, v3)
