"""Backward parity under strong forgetting: heads with a 32-token block whose
decay product leaves the block form's range (below e^-40 in some key channel
or pair) are redone token by token; every gradient is compared with the fp64
reverse-mode oracle (``oracle.grad.backward_seq``), which has no range limit.

Decay patterns as in test_gpu_strong_decay.py (uniform strong decay, bursts in
some channels of alternate blocks, exact zeros and fp32 subnormals, one
stretch below e^-150), plus the SFDA page's register reset (finite-state
expressivity, with delta correction: decay 0, beta = w = 1) and a launch where
only some heads need the token path.
"""
import dataclasses

import numpy as np
import pytest

from _gpu import random_state
from synth.gen import generate
from test_gpu_bwd import _upstream, _wl, check
from test_gpu_strong_decay import strong_transition

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pattern", ["uniform", "bursts", "reset", "cum150"])
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_bwd_strong(decay, dk, pattern):
    """Ragged tail (T = 100), S0 and grad_S set."""
    x = generate(_wl(decay, dk, seed=141 + dk))
    x = dataclasses.replace(x, alpha=strong_transition(x.alpha, pattern, 32, seed=dk + 3))
    dO, dS = _upstream(x, 15)
    S0 = random_state(2, 2, dk, dk, 18)
    check(x, dO, S0, dS, f"bwd strong {pattern} {decay}/d{dk}")


@pytest.mark.parametrize("decay", ["diag", "rot2"])
def test_bwd_strong_some_heads(decay):
    """One launch with block-form and token-path heads side by side: strong decay
    on head 1 of batch row 0 and head 2 of batch row 1 only (three heads, d = 128,
    four value tiles each, T = 200)."""
    x = generate(_wl(decay, 128, H=3, T=200, seed=151))
    a = x.alpha.copy()
    a[0, :, 1] = strong_transition(a[0:1, :, 1:2], "uniform", 32, seed=4)[0, :, 0]
    a[1, :, 2] = strong_transition(a[1:2, :, 2:3], "reset", 32, seed=5)[0, :, 0]
    x = dataclasses.replace(x, alpha=a)
    dO, dS = _upstream(x, 16)
    S0 = random_state(2, 3, 128, 128, 19)
    check(x, dO, S0, dS, f"bwd strong some heads {decay}")


@pytest.mark.parametrize("decay", ["diag", "rot2"])
@pytest.mark.parametrize("dk", [64, 128])
def test_bwd_pure_reset(decay, dk):
    """Decay 0 everywhere and beta = w = 1: S_t = v_t k_t^T exactly."""
    x = generate(_wl(decay, dk, T=77, seed=161))
    ones = np.ones_like(x.w)
    x = dataclasses.replace(x, alpha=np.zeros_like(x.alpha), beta=ones, w=ones)
    dO, dS = _upstream(x, 17)
    S0 = random_state(2, 2, dk, dk, 20)
    check(x, dO, S0, dS, f"bwd pure reset {decay}/d{dk}")
