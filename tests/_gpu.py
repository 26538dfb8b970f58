"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
call the HIP path through the C ABI, and run the fp64 oracle on chosen heads."""
from __future__ import annotations

import numpy as np

from oracle import seq
from oracle.errors import max_rel_err

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max |x - ref| / max |ref| per output tensor


def dev(x, dtype=None):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t if dtype is None else t.to(dtype)


def io_dtype(io: str):
    import torch
    return torch.bfloat16 if io == "bf16" else torch.float32


def run_gpu(x, chunk=None, S0=None, m_carry=None, alias=False, return_m=False):
    """Run gdr_chunk_fwd on host inputs ``x`` (synth.gen.Inputs)."""
    import torch
    import recurrent_state_memory_amd as gdr
    io = io_dtype(x.wl.io)
    q, k, v = dev(x.q, io), dev(x.k, io), dev(x.v, io)
    S0d = dev(S0)
    mc = dev(m_carry) if m_carry is not None else None
    if x.wl.content and return_m and mc is None:
        mc = torch.zeros((x.wl.B, x.wl.H, x.wl.dv), dtype=torch.float32, device="cuda")
    o, S = gdr.gdr_chunk_fwd(
        q, k, v, dev(x.alpha), dev(x.w), dev(x.beta), theta=dev(x.theta), S0=S0d,
        chunk=chunk or x.wl.chunk, S_out=S0d if alias else None,
        beta_logit=dev(x.beta_logit), ub_down=dev(x.ub_down), ub_up=dev(x.ub_up),
        m_carry=mc)
    torch.cuda.synchronize()
    res = (o.float().cpu().numpy(), S.cpu().numpy())
    if return_m:
        res = res + (mc.cpu().numpy(),)
    return res


def oracle_heads(x, heads=None, S0=None, m_carry=None, return_m=False):
    """fp64 oracle on the (b, h) pairs in ``heads``, or on every head at once with
    one call vectorised over (B, H) when ``heads`` is None.

    Returns dict (b, h) -> (o [T, dv], S [dv, dk] (, m [dv])).
    """
    wl = x.wl
    if heads is None:
        kw = {}
        if wl.content:
            kw = dict(beta_logit=x.beta_logit, ub_down=x.ub_down, ub_up=x.ub_up,
                      chunk=wl.chunk, m_carry=m_carry, return_m=return_m)
        r = seq.forward(x.q, x.k, x.v, x.w, x.alpha, beta=x.beta, theta=x.theta,
                        decay=wl.decay, S0=S0, **kw)
        out = {}
        for b in range(wl.B):
            for h in range(wl.H):
                item = (r[0][b, :, h], r[1][b, h])
                if return_m and wl.content:
                    item = item + (r[2][b, h],)
                out[(b, h)] = item
        return out
    out = {}
    for b, h in heads:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        kw = {}
        if wl.content:
            kw = dict(beta_logit=x.beta_logit[sl], ub_down=x.ub_down[h:h + 1],
                      ub_up=x.ub_up[h:h + 1], chunk=wl.chunk,
                      m_carry=None if m_carry is None else m_carry[b:b + 1, h:h + 1],
                      return_m=return_m)
        r = seq.forward(x.q[sl], x.k[sl], x.v[sl], x.w[sl], x.alpha[sl],
                        beta=None if x.beta is None else x.beta[sl],
                        theta=None if x.theta is None else x.theta[sl], decay=wl.decay,
                        S0=None if S0 is None else S0[b:b + 1, h:h + 1], **kw)
        item = (r[0][0, :, 0], r[1][0, 0])
        if return_m and wl.content:
            item = item + (r[2][0, 0],)
        out[(b, h)] = item
    return out


def compare_heads(o, S, ref, tol, what=""):
    """Max-normalised errors over the sampled heads; asserts both within tol."""
    o_g = np.stack([o[b, :, h] for (b, h) in ref])
    o_r = np.stack([ref[k][0] for k in ref])
    S_g = np.stack([S[b, h] for (b, h) in ref])
    S_r = np.stack([ref[k][1] for k in ref])
    eo, es = max_rel_err(o_g, o_r), max_rel_err(S_g, S_r)
    print(f"{what}: err(o) = {eo:.3e}  err(S) = {es:.3e}  (tol {tol:g})", flush=True)
    assert eo <= tol, f"{what}: o error {eo:.3e} > {tol}"
    assert es <= tol, f"{what}: S error {es:.3e} > {tol}"
    return eo, es


def random_state(B, H, dv, dk, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, dv, dk)) / np.sqrt(dk)).astype(np.float32)
