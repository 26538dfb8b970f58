"""Pins of the partial-permutation oracle (oracle/perm.py), CPU only.

* a bounded stack (SFDA technical summary, finite-state expressivity: partial
  permutations realise a bounded stack) driven by random push / pop / no-op
  sequences reads back exactly what a Python list of capacity d_k holds;
* the column selection equals the product with the dense 0/1 matrix D;
* the identity map is the plain delta rule (oracle/seq.py with alpha = 1);
* with beta = 0 the state is S0 times the composed map, folded in integers.
"""
import numpy as np
import pytest

from oracle import perm, seq


def _shift_down(d):
    return np.array([-1] + list(range(d - 1)))          # cell j <- cell j-1


def _shift_up(d):
    return np.array(list(range(1, d)) + [-1])           # cell j <- cell j+1


@pytest.mark.parametrize("d", [4, 8])
def test_bounded_stack_reads_back_exactly(d):
    """Push x: shift down, then write x at channel 0 (k = e_0, beta = w = 1);
    pop: shift up, no write; the query e_0 reads the top (0 when empty).  Each
    value row holds its own stack of scalars."""
    rng = np.random.default_rng(d)
    T, dv = 200, 3
    e0 = np.eye(d)[0]
    q = np.tile(e0, (1, T, 1, 1))
    k = np.tile(e0, (1, T, 1, 1))
    v = np.zeros((1, T, 1, dv))
    beta = np.zeros((1, T, 1))
    src = np.zeros((1, T, 1, d), dtype=np.int64)
    stacks = [[] for _ in range(dv)]
    want = np.zeros((T, dv))
    for t in range(T):
        op = rng.choice(["push", "push", "pop", "noop"])
        if op == "push":
            x = rng.integers(1, 100, dv).astype(float)
            src[0, t, 0] = _shift_down(d)
            v[0, t, 0] = x
            beta[0, t, 0] = 1.0
            for i in range(dv):
                stacks[i].insert(0, x[i])
                del stacks[i][d:]                       # bounded: the deepest falls off
        elif op == "pop":
            src[0, t, 0] = _shift_up(d)
            for i in range(dv):
                if stacks[i]:
                    stacks[i].pop(0)
        else:
            src[0, t, 0] = np.arange(d)
        want[t] = [st[0] if st else 0.0 for st in stacks]
    o, S = perm.forward(q, k, v, np.ones((1, T, 1)), src, beta)
    assert np.array_equal(o[0, :, 0], want)
    for i in range(dv):                                  # the whole stack, cell by cell
        full = stacks[i] + [0.0] * (d - len(stacks[i]))
        assert np.array_equal(S[0, 0, i], full)


def test_column_selection_equals_dense_matrix_product():
    rng = np.random.default_rng(1)
    B, H, dv, dk = 2, 3, 4, 6
    S = rng.standard_normal((B, H, dv, dk))
    src = rng.integers(-2, dk + 2, (B, H, dk))           # includes out-of-range -> zero
    D = np.zeros((B, H, dk, dk))
    for b in range(B):
        for h in range(H):
            for j in range(dk):
                if 0 <= src[b, h, j] < dk:
                    D[b, h, src[b, h, j], j] = 1.0
    assert np.array_equal(perm.select_columns(S, src), S @ D)


def test_identity_map_is_the_plain_delta_rule():
    rng = np.random.default_rng(2)
    B, T, H, d = 2, 9, 2, 5
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    w, beta = rng.uniform(0.2, 1, (B, T, H)), rng.uniform(0.1, 0.9, (B, T, H))
    S0 = rng.standard_normal((B, H, d, d))
    src = np.broadcast_to(np.arange(d), (B, T, H, d))
    o1, S1 = perm.forward(q, k, v, w, src, beta, S0)
    o2, S2 = seq.forward(q, k, v, w, np.ones((B, T, H, d)), beta=beta, decay="diag", S0=S0)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(S1 - S2)) < 1e-12


def test_no_write_composes_the_maps():
    """beta = 0: column j of S_T is column (src_1 o ... o src_T)(j) of S0, folded
    as integer index maps (zero once any step drops it)."""
    rng = np.random.default_rng(3)
    B, T, H, dv, dk = 1, 12, 1, 3, 7
    S0 = rng.standard_normal((B, H, dv, dk))
    src = np.stack([rng.permutation(dk) for _ in range(T)])
    src[4, 2] = -1                                        # one channel dropped on the way
    z = np.zeros((B, T, H))
    q = rng.standard_normal((B, T, H, dk))
    _, S = perm.forward(q, q, np.zeros((B, T, H, dv)), z, src[None, :, None], z, S0)
    comp = np.arange(dk)                                  # S_T[:, j] = S0[:, comp[j]]
    for t in range(T - 1, -1, -1):
        comp = np.array([src[t][c] if c >= 0 else -1 for c in comp])
    want = np.where(comp >= 0, S0[0, 0][:, np.maximum(comp, 0)], 0.0)
    assert np.array_equal(S[0, 0], want)
