"""Throughput of the chunked gated delta-rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer]

A step is one gdr_chunk_fwd call over the whole workload (every stage of the
chunked method runs inside it), with inputs already resident in HBM.  The
default workload is the 1.3B-scale mixer layer: B=8, H=16, T=4096,
d_k = d_v = 128, chunk 64, bf16 q/k/v, fp32 gates and fp32 state, synthetic
seeded inputs.  A token is one (b, t) position covering all H heads.

The default warm-up (150 steps, about 30 ms of back-to-back work on the
layer workload) lets the GPU clock settle before the 200 timed steps.

Prints one JSON line with the throughput, a roofline object for the forward
kernel (algorithmic bytes per launch / measured launch time, against the HBM
peak) and a CPU baseline: the fp64 oracle timed on a bounded sample of the
same workload on this host.

Other workloads (``--workload small|rot|dihedral|long|decode|raven|stack|copy``) are for profiling
and are not the reported metric; ``copy`` is a plain device copy of known size
used to calibrate the HBM byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec gated-delta chunk fwd (H=16,d=128,T=4096) + % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 matrix peak
MFMA_F32_PEAK_TFS = 157.3
VALU_F32_PEAK_TFS = 157.3      # fp32 vector peak: 256 CUs x 128 FMA per cycle x 2 flops x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gdr_fwd_pipe_kernel_layer_traffic.txt")
TRAFFIC_FILE_GATED = os.path.join(ROOT, "profiles", "gdr_fwd_pipe_kernel_layer_gated_traffic.txt")
KERNEL_SRCS = [os.path.join(ROOT, "recurrent_state_memory_amd", "csrc", f)
               for f in ("gdr_fwd_pipe.hip", "gdr_mfma.h", "gdr_kernels.h", "gdr_token.h")]


def algorithmic_bytes(wl, s0: bool = False, gated: bool = False) -> int:
    """Bytes the forward must move at least once: q, k, v, transition, beta, w
    in; o out; S_out (and S0 when given).  Gated forward: the decay as a bf16
    pre-activation (2 bytes per channel, or per block beside the fp32 angle)."""
    s_in = 2 if wl.io == "bf16" else 4
    trans = 4 * wl.dk  # alpha [dk] fp32, or theta + gamma [dk/2] each
    if gated:
        trans = 2 * wl.dk if wl.decay == "diag" else (2 + 4) * (wl.dk // 2)
    per_th = (2 * wl.dk + wl.dv) * s_in + trans + 8 + wl.dv * s_in
    state = 4 * wl.dv * wl.dk * wl.B * wl.H
    return per_th * wl.B * wl.T * wl.H + state * (2 if s0 else 1)


def algorithmic_flops(wl, L: int) -> float:
    """Matrix-core-eligible flops of the chunked method per launch: the state
    GEMMs 6 d_k d_v, the intra-chunk products L (3 d_k + 2 d_v) and the
    triangular solve L^2/3 per token-head (triangles at half)."""
    per_th = 6 * wl.dk * wl.dv + L * (3 * wl.dk + 2 * wl.dv) + L * L / 3
    return per_th * wl.B * wl.T * wl.H


def bwd_flops(wl) -> float:
    """Matrix-core flops of the backward kernel per launch, each product counted
    once (the value-tile workgroups repeat the key-side ones): per 32-token
    block, eight d_k x d_v products with one L-sized side (16 L d_k d_v),
    six L x L x d_k (12 L^2 d_k) and five L x L x d_v (10 L^2 d_v)."""
    L = 32
    per_th = 16 * wl.dk * wl.dv + 12 * L * wl.dk + 10 * L * wl.dv
    return per_th * wl.B * wl.T * wl.H


def wy_block(wl) -> int:
    """Token block of the WY solve that actually runs for this workload: the
    pipelined bf16 kernel (d in {64, 128}) always uses 32-token blocks; the
    sequential-stage kernel uses min(chunk, 64), or 32 for fp32 at d = 128."""
    if wl.io == "bf16" and wl.dk in (64, 128) and (not wl.content or wl.chunk % 32 == 0):
        return 32
    return min(wl.chunk, 32 if (wl.io == "f32" and wl.dk == 128) else 64)


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _kernel_hash() -> str:
    """First 16 hex digits of the sha256 of the kernel sources' code (comments
    and whitespace removed): a comment edit keeps the recorded counters valid,
    any code change invalidates them."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _traffic(path=TRAFFIC_FILE):
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    counter reads for a copy of known size) from the committed rocprofv3
    summary, if it was taken on the current kernel source (else None)."""
    try:
        vals = {}
        for ln in open(path):
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
        if vals.get("kernel_source_sha256_16") != _kernel_hash():
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _to_dev(x, dtype=None):
    import numpy as np
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t if dtype is None else t.to(dtype)


def _fwd_closure(wl):
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import generate
    x = generate(wl)
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    q, k, v = _to_dev(x.q, io), _to_dev(x.k, io), _to_dev(x.v, io)
    alpha, theta, beta, w = map(_to_dev, (x.alpha, x.theta, x.beta, x.w))
    bl, ud, uu = map(_to_dev, (x.beta_logit, x.ub_down, x.ub_up))
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=io, device="cuda")
    S = torch.empty((wl.B, wl.H, wl.dv, wl.dk), dtype=torch.float32, device="cuda")

    def step():
        gdr.gdr_chunk_fwd(q, k, v, alpha, w, beta, theta=theta, chunk=wl.chunk, o=o,
                          S_out=S, beta_logit=bl, ub_down=ud, ub_up=uu,
                          reflections=wl.decay == "dihedral")
    return step, x


def _gated_closure(wl):
    """The gated forward on the workload's raw draws: decay from its bf16
    pre-activation, q and k normalised in the kernel."""
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import generate_gated
    x = generate_gated(wl)
    bf = torch.bfloat16
    q, k, v, xx = (_to_dev(t, bf) for t in (x.q, x.k, x.v, x.x))
    a, theta, beta, w = map(_to_dev, (x.a, x.theta, x.beta, x.w))
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=bf, device="cuda")
    S = torch.empty((wl.B, wl.H, wl.dv, wl.dk), dtype=torch.float32, device="cuda")

    def step():
        gdr.gdr_chunk_fwd_gated(q, k, v, xx, a, w, beta, theta=theta, qk_l2norm=True,
                                chunk=wl.chunk, o=o, S_out=S)
    return step, x


def _bwd_closure(wl):
    """gdr_chunk_bwd on the workload's inputs with a seeded bf16 grad_o and an
    fp32 grad_S; the workspace is allocated once, outside the timed region."""
    import numpy as np
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import bf16_round, generate
    x = generate(wl)
    bf = torch.bfloat16
    q, k, v = (_to_dev(t, bf) for t in (x.q, x.k, x.v))
    alpha, theta, beta, w = map(_to_dev, (x.alpha, x.theta, x.beta, x.w))
    rng = np.random.default_rng(wl.seed + 1)
    dO = _to_dev(bf16_round(rng.standard_normal(x.v.shape, dtype=np.float32)), bf)
    dS = _to_dev((rng.standard_normal((wl.B, wl.H, wl.dv, wl.dk)) / 8).astype(np.float32))
    ws = {}

    def step():
        g = gdr.gdr_chunk_bwd(q, k, v, alpha, w, beta, dO, theta=theta, grad_S=dS,
                              workspace=ws.get("w"))
        return g
    # size the workspace with one call, then reuse it
    import ctypes
    a = gdr.BwdArgs()
    a.B, a.T, a.H, a.dk, a.dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    a.decay = gdr.GDR_DECAY_ROT2 if theta is not None else gdr.GDR_DECAY_DIAG
    for f in ("q", "k", "v", "alpha", "beta", "w", "grad_o", "grad_q", "grad_k", "grad_v",
              "grad_alpha", "grad_beta", "grad_w"):
        setattr(a, f, 1 << 20)
    if theta is not None:
        a.theta = a.grad_theta = 1 << 20
    need = gdr.load_library().gdr_chunk_bwd_workspace(ctypes.byref(a))
    ws["w"] = torch.empty(need, dtype=torch.uint8, device="cuda")
    return step, x


def _bwd_gated_closure(wl):
    """gdr_chunk_bwd_gated on the gated forward's raw draws (bf16 decay
    pre-activation, raw q and k normalised per token) with a seeded bf16 grad_o
    and an fp32 grad_S; the workspace is allocated once, outside the timed
    region."""
    import ctypes
    import numpy as np
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import bf16_round, generate_gated
    x = generate_gated(wl)
    bf = torch.bfloat16
    q, k, v, xx = (_to_dev(t, bf) for t in (x.q, x.k, x.v, x.x))
    a_h, theta, beta, w = map(_to_dev, (x.a, x.theta, x.beta, x.w))
    rng = np.random.default_rng(wl.seed + 1)
    dO = _to_dev(bf16_round(rng.standard_normal(x.v.shape, dtype=np.float32)), bf)
    dS = _to_dev((rng.standard_normal((wl.B, wl.H, wl.dv, wl.dk)) / 8).astype(np.float32))
    a = gdr.BwdArgs()
    a.B, a.T, a.H, a.dk, a.dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    a.decay = gdr.GDR_DECAY_ROT2 if theta is not None else gdr.GDR_DECAY_DIAG
    for f in ("q", "k", "v", "beta", "w", "grad_o", "grad_q", "grad_k", "grad_v",
              "grad_beta", "grad_w"):
        setattr(a, f, 1 << 20)
    if theta is not None:
        a.theta = a.grad_theta = 1 << 20
    g = gdr.GateArgs()
    g.decay_x, g.decay_a, g.qk_l2norm, g.reserved = 1 << 20, 1 << 20, 1, 0
    need = gdr.load_library().gdr_chunk_bwd_gated_workspace(ctypes.byref(a), ctypes.byref(g))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        return gdr.gdr_chunk_bwd_gated(q, k, v, xx, a_h, w, beta, dO, theta=theta,
                                       qk_l2norm=True, grad_S=dS, workspace=ws)
    return step, x


def raven_bytes(wl) -> int:
    """Bytes the Raven slot-memory forward must move at least once: q, k, v and
    the router logits (bf16), the decay rate (fp32) in; o (bf16) out; the final
    key and value slots (fp32) out."""
    per_th = (2 * wl.dk + wl.dv + wl.slots) * 2 + 4 + wl.dv * 2
    return per_th * wl.B * wl.T * wl.H + 4 * wl.slots * (wl.dk + wl.dv) * wl.B * wl.H


def raven_flops(wl, L: int = 32) -> float:
    """Matrix flops of the chunk form per launch, each product counted once:
    per token q.Sk (M d), the value read-out (M d), both slot updates (2 M d),
    and the in-chunk token-pair terms at half (L d / 2 twice, L M / 2 twice)."""
    d, M = wl.dk, wl.slots
    return 2.0 * (4 * M * d + L * d + L * M) * wl.B * wl.T * wl.H


def _raven_closure(wl):
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import generate_raven
    x = generate_raven(wl)
    bf = torch.bfloat16
    q, k, v, z = (_to_dev(t, bf) for t in (x.q, x.k, x.v, x.z))
    a = _to_dev(x.a)
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=bf, device="cuda")
    Sk = torch.empty((wl.B, wl.H, wl.slots, wl.dk), dtype=torch.float32, device="cuda")
    Sv = torch.empty((wl.B, wl.H, wl.slots, wl.dv), dtype=torch.float32, device="cuda")

    def step():
        gdr.gdr_raven_fwd(q, k, v, z, a, topk=wl.topk, scale=wl.scale, o=o, Sk_out=Sk, Sv_out=Sv)
    return step, x


def cpu_baseline_raven(wl, x, budget_s: float = 15.0):
    """The Raven oracle on this host's cores, as ``cpu_baseline``: one worker
    thread per batch row, all heads, a prefix sized to about ``budget_s``."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import raven

    workers = max(1, min(16, len(os.sched_getaffinity(0)), wl.B))

    def run(b, T_s):
        sl = (slice(b, b + 1), slice(0, T_s))
        return raven.forward(x.q[sl], x.k[sl], x.v[sl], x.z[sl], x.a[sl], wl.topk, wl.scale)[0]

    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        probe = 16
        t0 = time.perf_counter()
        list(ex.map(lambda b: run(b, probe), range(wl.B)))
        per_tok = (time.perf_counter() - t0) / probe
        T_s = int(max(32, min(wl.T, budget_s / max(per_tok, 1e-9))))
        t0 = time.perf_counter()
        outs = list(ex.map(lambda b: run(b, T_s), range(wl.B)))
        secs = time.perf_counter() - t0
    assert all(np.all(np.isfinite(o)) for o in outs)
    return {"value": round(wl.B * T_s / secs, 2), "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": (f"fp64 numpy token-by-token Raven oracle, {workers} worker threads "
                       f"(BLAS single-threaded) on {_cpu_model()}, all {wl.B}x{wl.H} heads, "
                       f"first {T_s} of {wl.T} tokens, {secs:.1f} s")}


def perm_bytes(wl) -> int:
    """Bytes the partial-permutation forward must move at least once: q, k, v
    (bf16), the int16 source maps, beta and w (fp32) in; o (bf16) and the final
    state (fp32) out."""
    per_th = (2 * wl.dk + wl.dv) * 2 + 2 * wl.dk + 8 + 2 * wl.dv
    return per_th * wl.B * wl.T * wl.H + 4 * wl.dv * wl.dk * wl.B * wl.H


def perm_flops(wl) -> float:
    """fp32 vector flops per launch: X k, the rank-1 update and S q, 2 d_v d_k
    each per token-head (the column selection moves data only)."""
    return 6.0 * wl.dv * wl.dk * wl.B * wl.T * wl.H


def _perm_closure(wl):
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import generate_perm
    x = generate_perm(wl)
    bf = torch.bfloat16
    q, k, v = (_to_dev(t, bf) for t in (x.q, x.k, x.v))
    w, beta = _to_dev(x.w), _to_dev(x.beta)
    src = torch.from_numpy(x.src).to("cuda")
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=bf, device="cuda")
    S = torch.empty((wl.B, wl.H, wl.dv, wl.dk), dtype=torch.float32, device="cuda")

    def step():
        gdr.gdr_perm_fwd(q, k, v, w, src, beta, o=o, S_out=S)
    return step, x


def cpu_baseline_perm(wl, x, budget_s: float = 15.0):
    """The partial-permutation oracle on this host's cores (as ``cpu_baseline``)."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import perm

    workers = max(1, min(16, len(os.sched_getaffinity(0)), wl.B))

    def run(b, T_s):
        sl = (slice(b, b + 1), slice(0, T_s))
        return perm.forward(x.q[sl], x.k[sl], x.v[sl], x.w[sl], x.src[sl], x.beta[sl])[0]

    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        probe = 16
        t0 = time.perf_counter()
        list(ex.map(lambda b: run(b, probe), range(wl.B)))
        per_tok = (time.perf_counter() - t0) / probe
        T_s = int(max(32, min(wl.T, budget_s / max(per_tok, 1e-9))))
        t0 = time.perf_counter()
        outs = list(ex.map(lambda b: run(b, T_s), range(wl.B)))
        secs = time.perf_counter() - t0
    assert all(np.all(np.isfinite(o)) for o in outs)
    return {"value": round(wl.B * T_s / secs, 2), "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": (f"fp64 numpy token-by-token partial-permutation oracle, {workers} worker "
                       f"threads (BLAS single-threaded) on {_cpu_model()}, all {wl.B}x{wl.H} heads, "
                       f"first {T_s} of {wl.T} tokens, {secs:.1f} s")}


def _decode_closure():
    import torch
    import recurrent_state_memory_amd as gdr
    from synth.gen import generate_decode
    d = generate_decode()
    io = torch.bfloat16
    S = _to_dev(d.S)
    args = [_to_dev(d.q, io), _to_dev(d.k, io), _to_dev(d.v, io), _to_dev(d.alpha),
            _to_dev(d.beta), _to_dev(d.w)]
    th = _to_dev(d.theta)
    o = torch.empty((d.N, d.H, d.dv), dtype=io, device="cuda")

    def step():
        gdr.gdr_step_decode(S, *args, theta=th, o=o)
    return step, d


MALL_BYTES = 256 << 20   # MI355X Infinity Cache


def _time(step, steps, warmup, flush=False):
    """Seconds for ``steps`` launches after ``warmup`` untimed ones, with HIP
    events on the stream the launches use.  With ``flush`` every launch is timed
    on its own and a 512 MB buffer is written between launches, so inputs that
    would fit in the 256 MB Infinity Cache are read from HBM each time."""
    import torch
    scratch = torch.empty(2 * MALL_BYTES // 4, dtype=torch.float32, device="cuda") if flush else None
    for _ in range(warmup):
        step()
        if flush:
            scratch.fill_(1.0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    if not flush:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3, time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        scratch.fill_(1.0)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / 1e3, time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, budget_s: float = 15.0, gated: bool = False):
    """Time the fp64 oracle on this host's cores: one worker thread per group of
    batch rows (numpy releases the interpreter lock inside its array operations),
    BLAS single-threaded in each, all B*H heads over a prefix of the sequence
    sized to roughly ``budget_s`` seconds; tokens/s = B * T_sample / s."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import seq

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    workers = min(cores, wl.B * wl.H)
    # (b, h-range) slices: one per worker, heads split when B is small
    per_b = max(1, -(-workers // wl.B))
    hs = -(-wl.H // per_b)
    parts = [(b, h0, min(wl.H, h0 + hs)) for b in range(wl.B) for h0 in range(0, wl.H, hs)]
    workers = min(workers, len(parts))

    def run(part, T_s):
        b, h0, h1 = part
        sl = (slice(b, b + 1), slice(0, T_s), slice(h0, h1))
        th = None if x.theta is None else x.theta[sl]
        if gated:
            return seq.forward_gated(x.q[sl], x.k[sl], x.v[sl], x.w[sl], x.x[sl], x.a[h0:h1],
                                     x.beta[sl], theta=th, decay=wl.decay)[0]
        return seq.forward(x.q[sl], x.k[sl], x.v[sl], x.w[sl], x.alpha[sl],
                           beta=x.beta[sl], decay=wl.decay, theta=th)[0]

    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        # probe the per-token cost on a short prefix, then size the sample
        probe = 32
        t0 = time.perf_counter()
        list(ex.map(lambda pt: run(pt, probe), parts))
        per_tok = (time.perf_counter() - t0) / probe
        T_s = int(max(64, min(wl.T, budget_s / max(per_tok, 1e-9))))
        t0 = time.perf_counter()
        outs = list(ex.map(lambda pt: run(pt, T_s), parts))
        secs = time.perf_counter() - t0
    assert all(np.all(np.isfinite(o)) for o in outs)
    return {"value": round(wl.B * T_s / secs, 2), "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": (f"fp64 numpy token-by-token oracle, {workers} worker threads "
                       f"(BLAS single-threaded) on {_cpu_model()}, all {wl.B}x{wl.H} heads, "
                       f"first {T_s} of {wl.T} tokens, {secs:.1f} s")}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--workload", default="layer",
                    choices=["layer", "small", "rot", "dihedral", "long", "tiny", "decode", "copy",
                             "raven", "stack"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd", action="store_true",
                    help="gdr_chunk_bwd: the backward (forward recompute + reverse blocks + reduction)")
    ap.add_argument("--gated", action="store_true",
                    help="gdr_chunk_fwd_gated: bf16 decay pre-activation, q/k normalised in the "
                         "kernel (with --bwd: gdr_chunk_bwd_gated)")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward runs independent (b, h) units "
              "per GPU and this build has no multi-GPU path; run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from synth.gen import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if a.workload == "copy":
        n = 1 << 28   # 1 GiB of fp32
        src = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        secs, _ = _time(lambda: dst.copy_(src), a.steps, a.warmup)
        gbs = 2 * 4 * n * a.steps / secs / 1e9
        print(json.dumps({"workload": "copy", "bytes_per_launch": 8 * n, "GB/s": round(gbs, 1)}))
        return 0

    if a.workload == "decode":
        step, d = _decode_closure()
        secs, wall = _time(step, a.steps, a.warmup)
        per = secs / a.steps
        nbytes = d.N * d.H * (8 * d.dv * d.dk + 2 * (2 * d.dk + d.dv) + 4 * d.dk + 8 + 2 * d.dv)
        print(json.dumps({
            "metric": "decode steps gdr_step_decode", "value": round(d.N * d.H / per, 1),
            "unit": "state-heads/s", "ms_per_step": round(per * 1e3, 4),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / per / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4)},
            "config": {"workload": f"decode N={d.N} H={d.H} d={d.dk} rot2 bf16, fp32 state"}}))
        return 0

    if a.workload == "raven":
        from synth.gen import RAVEN_WORKLOADS
        wl = RAVEN_WORKLOADS["raven"]
        step, x = _raven_closure(wl)
        secs, wall = _time(step, a.steps, a.warmup)
        per = secs / a.steps
        nbytes = raven_bytes(wl)
        fl = raven_flops(wl)
        out = {
            "metric": "tokens/sec Raven routing slot-memory fwd",
            "value": round(wl.B * wl.T / per, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(per * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; q,k L2-normalised, N(0,1) router logits, a = -softplus(x))",
            "config": {"workload": (f"raven: B={wl.B} H={wl.H} T={wl.T} d_k=d_v={wl.dk} "
                                    f"slots={wl.slots} top-{wl.topk}, bf16 q/k/v/logits, fp32 "
                                    "decay rate and slot states, 32-token chunks"),
                       "global_batch": wl.B, "seq_len": wl.T, "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": round(nbytes / per / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4), "traffic": None},
            "roofline_mfma": {"achieved": round(fl / per / 1e12, 2), "peak": MFMA_BF16_PEAK_TFS,
                              "unit": "TFLOP/s",
                              "frac": round(fl / per / 1e12 / MFMA_BF16_PEAK_TFS, 4)},
            "wall_s_timed_region": round(wall, 4),
        }
        if not a.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_raven(wl, x)
        print(json.dumps(out))
        return 0

    if a.workload == "stack":
        from synth.gen import PERM_WORKLOADS
        wl = PERM_WORKLOADS["stack"]
        step, x = _perm_closure(wl)
        secs, wall = _time(step, a.steps, a.warmup)
        per = secs / a.steps
        nbytes = perm_bytes(wl)
        fl = perm_flops(wl)
        out = {
            "metric": "tokens/sec delta rule with partial-permutation transitions fwd",
            "value": round(wl.B * wl.T / per, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(per * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded; q,k L2-normalised, sigmoid gates, random stack moves)",
            "config": {"workload": (f"stack: B={wl.B} H={wl.H} T={wl.T} d_k=d_v={wl.dk}, bf16 "
                                    "q/k/v, int16 source maps (push/pop/stay), fp32 state and "
                                    "arithmetic, token by token"),
                       "global_batch": wl.B, "seq_len": wl.T, "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": round(fl / per / 1e12, 2),
                         "peak": VALU_F32_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(fl / per / 1e12 / VALU_F32_PEAK_TFS, 4), "traffic": None},
            "roofline_hbm": {"achieved": round(nbytes / per / 1e9, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4)},
            "wall_s_timed_region": round(wall, 4),
        }
        if not a.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_perm(wl, x)
        print(json.dumps(out))
        return 0

    wl = WORKLOADS[a.workload]
    if a.bwd:
        if wl.content or wl.io != "bf16" or wl.dk not in (64, 128) or wl.decay == "dihedral":
            print("--bwd runs the bf16 plain-erase workloads with d in {64, 128} "
                  "(no reflection blocks)", file=sys.stderr)
            return 2
        step, x = _bwd_gated_closure(wl) if a.gated else _bwd_closure(wl)
        secs, wall = _time(step, a.steps, a.warmup)
        per = secs / a.steps
        fl = bwd_flops(wl)
        out = {
            "metric": ("tokens/sec gated-delta chunk bwd, gated (activation and q/k normalisation "
                       "+ recompute + backward + reduction + chain rule)" if a.gated else
                       "tokens/sec gated-delta chunk bwd (recompute + backward + reduction)"),
            "value": round(wl.B * wl.T / per, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(per * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": ("synthetic (seeded; the gated forward's raw draws, bf16 grad_o, fp32 grad_S)"
                     if a.gated else
                     "synthetic (seeded; the forward's inputs, bf16 grad_o, fp32 grad_S)"),
            "config": {"workload": (f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} d_k=d_v={wl.dk}, "
                                    f"{'2x2 rotation-decay' if wl.decay == 'rot2' else 'per-channel decay'}, "
                                    "gradients of q,k,v,decay,beta,w,S0 in fp32"),
                       "global_batch": wl.B, "seq_len": wl.T, "parallelism": "single GPU"},
            "roofline_scope": ("whole gdr_chunk_bwd_gated call (7 kernels); flops of the backward "
                               "kernel only" if a.gated else
                               "whole gdr_chunk_bwd call (4 kernels); per-kernel times in profiles/"),
            "roofline": {"bound": "mfma", "achieved": round(fl / per / 1e12, 2),
                         "peak": MFMA_F32_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(fl / per / 1e12 / MFMA_F32_PEAK_TFS, 4), "traffic": None},
            "wall_s_timed_region": round(wall, 4),
        }
        print(json.dumps(out))
        return 0
    gated = a.gated
    if gated and (wl.content or wl.io != "bf16" or wl.dk not in (64, 128)
                  or wl.decay == "dihedral"):
        print("--gated runs the bf16 plain-erase workloads with d in {64, 128}", file=sys.stderr)
        return 2
    step, x = _gated_closure(wl) if gated else _fwd_closure(wl)
    flush = algorithmic_bytes(wl, gated=gated) < MALL_BYTES
    secs, wall = _time(step, a.steps, a.warmup, flush=flush)
    per = secs / a.steps
    tokens = wl.B * wl.T
    value = tokens / per
    from recurrent_state_memory_amd.build import ARCH  # noqa: F401  (built for gfx950)
    nbytes = algorithmic_bytes(wl, gated=gated)
    L_eff = wy_block(wl)
    flops = algorithmic_flops(wl, L_eff)
    achieved = nbytes / per / 1e9
    mfma_peak = MFMA_BF16_PEAK_TFS if wl.io == "bf16" else MFMA_F32_PEAK_TFS
    traffic = None
    if a.workload == "layer":
        traffic = _traffic(TRAFFIC_FILE_GATED if gated else TRAFFIC_FILE)
    # the headline metric names the layer workload; variants name their own
    if a.workload == "layer" and not gated:
        metric = METRIC
    else:
        metric = (f"tokens/sec gated-delta chunk fwd{' (gated)' if gated else ''} "
                  f"({wl.name}: B={wl.B},H={wl.H},d={wl.dk},T={wl.T}) + % MFMA/HBM roofline")
    out = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(per * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.io,
        "data": ("synthetic (seeded; q,k L2-normalised, gates from the stated distributions)"
                 if not gated else
                 "synthetic (seeded; raw q,k and decay pre-activations from the stated distributions)"),
        "config": {
            "workload": (f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} d_k=d_v={wl.dk} chunk={wl.chunk} "
                         f"({L_eff}-token WY blocks{', MALL flushed between launches' if flush else ''}) "
                         + (f"{wl.io} q/k/v, fp32 gates and state, " if not gated else
                            "gated: bf16 raw q/k (L2-normalised in the kernel), bf16 v, bf16 decay "
                            "pre-activation exp(-a softplus(x)), fp32 beta/w/state, ")
                         + {"rot2": "2x2 rotation-decay", "diag": "per-channel decay",
                            "dihedral": "2x2 rotation/reflection blocks (dihedral)"}[wl.decay]
                         + (", content-aware erase" if wl.content else "")),
            "global_batch": wl.B, "seq_len": wl.T, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "roofline_mfma": {
            "achieved": round(flops / per / 1e12, 2), "peak": mfma_peak, "unit": "TFLOP/s",
            "frac": round(flops / per / 1e12 / mfma_peak, 4),
        },
        "wall_s_timed_region": round(wall, 4),
    }
    if not a.no_cpu_baseline and a.workload in ("layer", "small", "rot", "dihedral", "tiny"):
        out["cpu_baseline"] = cpu_baseline(wl, x, gated=gated)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
