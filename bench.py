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

Other workloads (``--workload small|rot|long|decode|copy``) are for profiling
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gdr_fwd_pipe_kernel_layer_traffic.txt")
KERNEL_SRCS = [os.path.join(ROOT, "recurrent_state_memory_amd", "csrc", f)
               for f in ("gdr_fwd_pipe.hip", "gdr_mfma.h", "gdr_kernels.h")]


def algorithmic_bytes(wl, s0: bool = False) -> int:
    """Bytes the forward must move at least once: q, k, v, transition, beta, w
    in; o out; S_out (and S0 when given)."""
    s_in = 2 if wl.io == "bf16" else 4
    trans = 4 * wl.dk  # alpha [dk] fp32, or theta + gamma [dk/2] each
    per_th = (2 * wl.dk + wl.dv) * s_in + trans + 8 + wl.dv * s_in
    state = 4 * wl.dv * wl.dk * wl.B * wl.H
    return per_th * wl.B * wl.T * wl.H + state * (2 if s0 else 1)


def algorithmic_flops(wl, L: int) -> float:
    """Matrix-core-eligible flops of the chunked method per launch: the state
    GEMMs 6 d_k d_v, the intra-chunk products L (3 d_k + 2 d_v) and the
    triangular solve L^2/3 per token-head (triangles at half)."""
    per_th = 6 * wl.dk * wl.dv + L * (3 * wl.dk + 2 * wl.dv) + L * L / 3
    return per_th * wl.B * wl.T * wl.H


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


def _traffic():
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    counter reads for a copy of known size) from the committed rocprofv3
    summary, if it was taken on the current kernel source (else None)."""
    try:
        vals = {}
        for ln in open(TRAFFIC_FILE):
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
                          S_out=S, beta_logit=bl, ub_down=ud, ub_up=uu)
    return step, x


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


def _time(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def cpu_baseline(wl, x, budget_s: float = 15.0):
    """Time the fp64 oracle (single thread) on all B*H heads over a prefix of
    the sequence sized to roughly ``budget_s`` seconds; tokens/s = B * T_sample / s."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import seq
    with threadpool_limits(limits=1):
        # probe the per-token cost on a short prefix, then size the sample
        probe = 32
        sl = slice(0, probe)
        t0 = time.perf_counter()
        seq.forward(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.w[:, sl], x.alpha[:, sl],
                    beta=x.beta[:, sl], decay=wl.decay,
                    theta=None if x.theta is None else x.theta[:, sl])
        per_tok = (time.perf_counter() - t0) / probe
        T_s = int(max(64, min(wl.T, budget_s / max(per_tok, 1e-9))))
        sl = slice(0, T_s)
        t0 = time.perf_counter()
        o, _ = seq.forward(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.w[:, sl], x.alpha[:, sl],
                           beta=x.beta[:, sl], decay=wl.decay,
                           theta=None if x.theta is None else x.theta[:, sl])
        secs = time.perf_counter() - t0
    assert np.all(np.isfinite(o))
    return {"value": round(wl.B * T_s / secs, 2), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"fp64 numpy token-by-token oracle, single thread, all {wl.B}x{wl.H} "
                       f"heads, first {T_s} of {wl.T} tokens, {secs:.1f} s")}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--workload", default="layer",
                    choices=["layer", "small", "rot", "long", "tiny", "decode", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    wl = WORKLOADS[a.workload]
    step, x = _fwd_closure(wl)
    secs, wall = _time(step, a.steps, a.warmup)
    per = secs / a.steps
    tokens = wl.B * wl.T
    value = tokens / per
    from recurrent_state_memory_amd.build import ARCH  # noqa: F401  (built for gfx950)
    nbytes = algorithmic_bytes(wl)
    L_eff = min(wl.chunk, 64)
    flops = algorithmic_flops(wl, L_eff)
    achieved = nbytes / per / 1e9
    mfma_peak = MFMA_BF16_PEAK_TFS if wl.io == "bf16" else MFMA_F32_PEAK_TFS
    traffic = _traffic() if a.workload == "layer" else None
    out = {
        "metric": METRIC,
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
        "data": "synthetic (seeded; q,k L2-normalised, gates from the stated distributions)",
        "config": {
            "workload": (f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} d_k=d_v={wl.dk} chunk={wl.chunk} "
                         f"{wl.io} q/k/v, fp32 gates and state, "
                         f"{'2x2 rotation-decay' if wl.decay == 'rot2' else 'per-channel decay'}"
                         f"{', content-aware erase' if wl.content else ''}"),
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
    if not a.no_cpu_baseline and a.workload in ("layer", "small", "rot", "tiny"):
        out["cpu_baseline"] = cpu_baseline(wl, x)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
