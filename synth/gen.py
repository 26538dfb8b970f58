"""Seeded synthetic inputs for the gated delta-rule forward and its decode step.

This module draws random numbers and shapes them into the input tensors that
both the fp64 oracle and the HIP path consume.  It holds none of the
recurrence's arithmetic: only the draws, the input transforms that fix the
distributions (L2-normalisation of q and k, sigmoid gates, softplus decays),
and round-to-nearest-even casting to bfloat16, so that both sides read
bit-identical values.

Workloads (the shapes of the five named configurations):

====  ==============================  =====  ===========  ====================
name  B, H, T, d_k = d_v              chunk  io dtype     transition
====  ==============================  =====  ===========  ====================
tiny  1, 1, 256, 32                   16     fp32         per-channel decay
small 4, 8, 2048, 64                  64     bf16         per-channel decay
layer 8, 16, 4096, 128                64     bf16         per-channel decay
long  1, 16, 32768, 128               128    bf16         decay + content erase
rot   4, 16, 8192, 128 (+ decode)     64     bf16         2x2 rotation blocks
====  ==============================  =====  ===========  ====================

The partial-permutation forward has ``PERM_WORKLOADS`` (the layer shape with a
random stack move per token and head) and ``generate_perm``.  The Raven
slot-memory forward has its own workload (``RAVEN_WORKLOADS``:
the layer shape B=8, H=16, T=4096, d=128 with 64 slots and top-8 routing) and
generator (``generate_raven``).

Draw order for one workload (all fp32 standard normal unless noted):
q, k, v, beta-logit (content-aware: b_x), w-logit, then either the decay
noise [B,T,H,d_k] or theta ~ U(-pi, pi) followed by the block-magnitude noise
[B,T,H,d_k/2]; content-aware workloads then draw the low-rank erase
projection B_h [H,r,d_v] and a_h [H,r], both scaled by 0.02.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# bfloat16 casting (round to nearest, ties to even), done on the fp32 bits
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Return the uint16 bfloat16 bit patterns of fp32 ``x`` (RNE rounding)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    out = r.astype(np.uint16)
    # NaN stays NaN (quiet); the generator never produces one.
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 ``x`` to the nearest bfloat16 and return it as fp32."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# input transforms (distributions only)
# --------------------------------------------------------------------------
def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    # stable form: max(x, 0) + log1p(exp(-|x|))
    return (np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    io: str            # "f32" | "bf16"
    decay: str         # "diag" | "rot2" | "dihedral" (rot2 with reflection blocks) | "perm"
    content: bool      # content-aware erase
    seed: int
    rank: int = 16     # low-rank width of the erase projection
    decay_scale: float = 0.1   # alpha = exp(-decay_scale * softplus(x))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 256, 32, 32, 16, "f32", "diag", False, 0),
    "small": Workload("small", 4, 8, 2048, 64, 64, 64, "bf16", "diag", False, 1),
    "layer": Workload("layer", 8, 16, 4096, 128, 128, 64, "bf16", "diag", False, 2),
    "long": Workload("long", 1, 16, 32768, 128, 128, 128, "bf16", "diag", True, 3),
    "rot": Workload("rot", 4, 16, 8192, 128, 128, 64, "bf16", "rot2", False, 4,
                    decay_scale=0.05),
    "dihedral": Workload("dihedral", 4, 16, 8192, 128, 128, 64, "bf16", "dihedral", False, 5,
                         decay_scale=0.05),
}

DECODE_N = 256


@dataclasses.dataclass
class Inputs:
    """fp32 host arrays; bf16-valued tensors hold exactly representable values."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: Optional[np.ndarray]        # [B,T,H] (None when content-aware)
    w: np.ndarray                     # [B,T,H]
    alpha: Optional[np.ndarray]       # diag: [B,T,H,dk]; rot2: block magnitude [B,T,H,dk/2]
    theta: Optional[np.ndarray]       # rot2: [B,T,H,dk/2]
    beta_logit: Optional[np.ndarray]  # content-aware b_x [B,T,H]
    ub_down: Optional[np.ndarray]     # content-aware B_h [H,r,dv]
    ub_up: Optional[np.ndarray]       # content-aware a_h [H,r]
    S0: Optional[np.ndarray] = None   # [B,H,dv,dk]


def _io_cast(x: np.ndarray, io: str) -> np.ndarray:
    return bf16_round(x) if io == "bf16" else np.ascontiguousarray(x, np.float32)


def generate(wl: Workload, T: Optional[int] = None, B: Optional[int] = None,
             ub_std: float = 0.02) -> Inputs:
    """Draw the inputs of ``wl`` (optionally overriding T or B, keeping the recipe).

    ``ub_std`` scales the low-rank erase projection of content-aware workloads
    (0.02 is the recipe; a larger value is a stress setting for tests).
    """
    if T is not None or B is not None:
        wl = wl.replace(T=T if T is not None else wl.T, B=B if B is not None else wl.B)
    rng = np.random.default_rng(wl.seed)
    Bn, Tn, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    q = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    k = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    v = rng.standard_normal((Bn, Tn, H, dv), dtype=np.float32)
    b_logit = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    w_logit = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    theta = None
    if wl.decay == "diag":
        a_noise = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    else:
        theta = rng.uniform(-math.pi, math.pi, (Bn, Tn, H, dk // 2)).astype(np.float32)
        a_noise = rng.standard_normal((Bn, Tn, H, dk // 2), dtype=np.float32)
    refl = None
    if wl.decay == "dihedral":   # each block a reflection with probability 1/2
        refl = rng.uniform(0.0, 1.0, (Bn, Tn, H, dk // 2)) < 0.5
    ub_down = ub_up = None
    if wl.content:
        ub_down = (rng.standard_normal((H, wl.rank, dv), dtype=np.float32)
                   * np.float32(ub_std)).astype(np.float32)
        ub_up = (rng.standard_normal((H, wl.rank), dtype=np.float32)
                 * np.float32(ub_std)).astype(np.float32)

    q = _io_cast(_l2_normalise(q), wl.io)
    k = _io_cast(_l2_normalise(k), wl.io)
    v = _io_cast(v, wl.io)
    alpha = np.exp(np.float32(-wl.decay_scale) * _softplus(a_noise)).astype(np.float32)
    if refl is not None:   # a reflection block carries its magnitude with the sign bit set
        alpha = np.where(refl, -alpha, alpha).astype(np.float32)
    w = _sigmoid(w_logit)
    if wl.content:
        beta, beta_logit = None, b_logit
    else:
        beta, beta_logit = _sigmoid(b_logit), None
    return Inputs(wl, q, k, v, beta, w, alpha, theta, beta_logit, ub_down, ub_up)


@dataclasses.dataclass
class DecodeInputs:
    """One token for N independent states of shape [H, dv, dk]."""
    N: int
    H: int
    dk: int
    dv: int
    io: str
    decay: str
    S: np.ndarray          # [N,H,dv,dk] fp32
    q: np.ndarray          # [N,H,dk]
    k: np.ndarray
    v: np.ndarray          # [N,H,dv]
    beta: np.ndarray       # [N,H]
    w: np.ndarray          # [N,H]
    alpha: np.ndarray      # diag: [N,H,dk]; rot2: [N,H,dk/2]
    theta: Optional[np.ndarray]


def generate_decode(wl: Workload = WORKLOADS["rot"], N: int = DECODE_N,
                    rng: Optional[np.random.Generator] = None) -> DecodeInputs:
    """Decode-step inputs drawn after the chunk inputs of ``wl`` (same stream).

    The state is N(0,1)/sqrt(d_k) so that the step does real work.  Pass an
    explicit ``rng`` to skip drawing the chunk inputs first (cheap tests).
    """
    H, dk, dv = wl.H, wl.dk, wl.dv
    if rng is None:
        rng = np.random.default_rng(wl.seed)
        # advance the stream past the chunk inputs, in draw order
        Bn, Tn = wl.B, wl.T
        rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
        rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
        rng.standard_normal((Bn, Tn, H, dv), dtype=np.float32)
        rng.standard_normal((Bn, Tn, H), dtype=np.float32)
        rng.standard_normal((Bn, Tn, H), dtype=np.float32)
        if wl.decay == "diag":
            rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
        else:
            rng.uniform(-math.pi, math.pi, (Bn, Tn, H, dk // 2))
            rng.standard_normal((Bn, Tn, H, dk // 2), dtype=np.float32)
            if wl.decay == "dihedral":
                rng.uniform(0.0, 1.0, (Bn, Tn, H, dk // 2))
    S = (rng.standard_normal((N, H, dv, dk), dtype=np.float32)
         / np.float32(math.sqrt(dk))).astype(np.float32)
    q = rng.standard_normal((N, H, dk), dtype=np.float32)
    k = rng.standard_normal((N, H, dk), dtype=np.float32)
    v = rng.standard_normal((N, H, dv), dtype=np.float32)
    b_logit = rng.standard_normal((N, H), dtype=np.float32)
    w_logit = rng.standard_normal((N, H), dtype=np.float32)
    theta = None
    refl = None
    if wl.decay == "diag":
        a_noise = rng.standard_normal((N, H, dk), dtype=np.float32)
    else:
        theta = rng.uniform(-math.pi, math.pi, (N, H, dk // 2)).astype(np.float32)
        a_noise = rng.standard_normal((N, H, dk // 2), dtype=np.float32)
        if wl.decay == "dihedral":
            refl = rng.uniform(0.0, 1.0, (N, H, dk // 2)) < 0.5
    io = wl.io
    alpha = np.exp(np.float32(-wl.decay_scale) * _softplus(a_noise)).astype(np.float32)
    if refl is not None:
        alpha = np.where(refl, -alpha, alpha).astype(np.float32)
    return DecodeInputs(
        N, H, dk, dv, io, wl.decay, S,
        _io_cast(_l2_normalise(q), io), _io_cast(_l2_normalise(k), io), _io_cast(v, io),
        _sigmoid(b_logit), _sigmoid(w_logit), alpha, theta)


@dataclasses.dataclass
class GatedInputs:
    """Inputs of the gated forward: raw (unnormalised) q and k, and the decay as
    its pre-activation x with a per-head scale a (decay = exp(-a softplus(x)))."""
    wl: Workload
    q: np.ndarray          # [B,T,H,dk] bf16-valued, not normalised
    k: np.ndarray
    v: np.ndarray          # [B,T,H,dv]
    beta: np.ndarray       # [B,T,H]
    w: np.ndarray          # [B,T,H]
    x: np.ndarray          # diag: [B,T,H,dk]; rot2: [B,T,H,dk/2], bf16-valued
    a: np.ndarray          # [H] fp32
    theta: Optional[np.ndarray]


def generate_gated(wl: Workload, T: Optional[int] = None) -> GatedInputs:
    """The recipe's draws in the recipe's order, passed on before the transforms
    that the gated forward applies itself: q, k and the decay noise are rounded
    to bf16 as drawn; a_h is the recipe's decay scale for every head."""
    if T is not None:
        wl = wl.replace(T=T)
    rng = np.random.default_rng(wl.seed)
    Bn, Tn, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    q = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    k = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    v = rng.standard_normal((Bn, Tn, H, dv), dtype=np.float32)
    b_logit = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    w_logit = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    theta = None
    if wl.decay == "diag":
        noise = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    else:
        theta = rng.uniform(-math.pi, math.pi, (Bn, Tn, H, dk // 2)).astype(np.float32)
        noise = rng.standard_normal((Bn, Tn, H, dk // 2), dtype=np.float32)
    return GatedInputs(wl, bf16_round(q), bf16_round(k), _io_cast(v, "bf16"), _sigmoid(b_logit),
                       _sigmoid(w_logit), bf16_round(noise),
                       np.full((H,), wl.decay_scale, dtype=np.float32), theta)


# --------------------------------------------------------------------------
# Raven routing slot memory (a second recurrence: M slots, top-K router)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class RavenWorkload:
    """Shapes of the slot-memory forward: M slots of d_k (keys) and d_v (values)
    per head, the top-K router, and the decay rate a = -a_scale * softplus(x)."""
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    slots: int
    topk: int
    seed: int
    a_scale: float = 1.0

    def replace(self, **kw) -> "RavenWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)


RAVEN_WORKLOADS = {
    # the layer shape (B=8, H=16, T=4096, d=128) with 64 slots, top-8 routing
    "raven": RavenWorkload("raven", 8, 16, 4096, 128, 128, 64, 8, 6),
}


@dataclasses.dataclass
class RavenInputs:
    """fp32 host arrays; q, k, v and the router logits z hold bf16 values."""
    wl: RavenWorkload
    q: np.ndarray      # [B,T,H,dk], L2-normalised per token
    k: np.ndarray      # [B,T,H,dk], L2-normalised per token
    v: np.ndarray      # [B,T,H,dv]
    z: np.ndarray      # [B,T,H,slots] router logits
    a: np.ndarray      # [B,T,H] decay rate, <= 0


def generate_raven(wl: RavenWorkload, T: Optional[int] = None,
                   B: Optional[int] = None) -> RavenInputs:
    """Draw order: q, k, v, router logits z, decay noise x (all fp32 standard
    normal); then q, k L2-normalised and rounded to bf16, v and z rounded to
    bf16, a = -a_scale * softplus(x) in fp32."""
    if T is not None or B is not None:
        wl = wl.replace(T=T if T is not None else wl.T, B=B if B is not None else wl.B)
    rng = np.random.default_rng(wl.seed)
    Bn, Tn, H = wl.B, wl.T, wl.H
    q = rng.standard_normal((Bn, Tn, H, wl.dk), dtype=np.float32)
    k = rng.standard_normal((Bn, Tn, H, wl.dk), dtype=np.float32)
    v = rng.standard_normal((Bn, Tn, H, wl.dv), dtype=np.float32)
    z = rng.standard_normal((Bn, Tn, H, wl.slots), dtype=np.float32)
    x = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    a = (np.float32(-wl.a_scale) * _softplus(x)).astype(np.float32)
    return RavenInputs(wl, bf16_round(_l2_normalise(q)), bf16_round(_l2_normalise(k)),
                       bf16_round(v), bf16_round(z), a)


# --------------------------------------------------------------------------
# partial-permutation transitions (bounded-stack moves)
# --------------------------------------------------------------------------
PERM_WORKLOADS = {
    # the layer shape with a stack move per (token, head): push (every channel one
    # deeper, channel 0 emptied), pop (one channel up) or stay, with probability 1/3 each
    "stack": Workload("stack", 8, 16, 4096, 128, 128, 64, "bf16", "perm", False, 7),
}


@dataclasses.dataclass
class PermInputs:
    """fp32 host arrays (q, k, v hold bf16 values) and int16 source maps."""
    wl: Workload
    q: np.ndarray      # [B,T,H,dk], L2-normalised per token
    k: np.ndarray      # [B,T,H,dk], L2-normalised per token
    v: np.ndarray      # [B,T,H,dv]
    beta: np.ndarray   # [B,T,H]
    w: np.ndarray      # [B,T,H]
    src: np.ndarray    # [B,T,H,dk] int16: column j of S D_t is column src[j] of S (-1: zero)


def stack_moves(op: np.ndarray, dk: int) -> np.ndarray:
    """Source maps of stack moves: op 0 = push (src[j] = j - 1, src[0] = -1),
    1 = pop (src[j] = j + 1, src[dk-1] = -1), 2 = stay (src[j] = j)."""
    j = np.arange(dk)
    push = np.where(j >= 1, j - 1, -1)
    pop = np.where(j + 1 < dk, j + 1, -1)
    stay = j
    table = np.stack([push, pop, stay]).astype(np.int16)
    return table[op]


def generate_perm(wl: Workload, T: Optional[int] = None, B: Optional[int] = None) -> PermInputs:
    """Draw order: q, k, v, beta-logit, w-logit (fp32 standard normal), then the
    move per (b, t, h) uniform over {push, pop, stay}.  q, k L2-normalised and
    rounded to bf16, v rounded to bf16, beta = w = sigmoid."""
    if T is not None or B is not None:
        wl = wl.replace(T=T if T is not None else wl.T, B=B if B is not None else wl.B)
    rng = np.random.default_rng(wl.seed)
    Bn, Tn, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    q = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    k = rng.standard_normal((Bn, Tn, H, dk), dtype=np.float32)
    v = rng.standard_normal((Bn, Tn, H, dv), dtype=np.float32)
    b_logit = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    w_logit = rng.standard_normal((Bn, Tn, H), dtype=np.float32)
    op = rng.integers(0, 3, (Bn, Tn, H))
    return PermInputs(wl, bf16_round(_l2_normalise(q)), bf16_round(_l2_normalise(k)),
                      bf16_round(v), _sigmoid(b_logit), _sigmoid(w_logit), stack_moves(op, dk))
