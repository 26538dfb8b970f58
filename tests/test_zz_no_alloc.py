"""The static-scratch backward (gdr_chunk_bwd_noalloc) against gdr_chunk_bwd on
the same inputs, through the C ABI: two calls in a row, the second smaller, so
that the second runs on the scratch the first left behind.  Same kernels on the
same inputs: the outputs must agree exactly."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _case(B, T, H, d, decay, seed):
    import torch
    from synth.gen import Workload, bf16_round, generate
    wl = Workload("noalloc", B, H, T, d, d, 64, "bf16", decay, False, seed,
                  decay_scale=0.1 if decay == "diag" else 0.05)
    x = generate(wl)
    rng = np.random.default_rng(seed + 1)
    dO = bf16_round(rng.standard_normal(x.v.shape).astype(np.float32))
    dS = (rng.standard_normal((B, H, d, d)) / 8).astype(np.float32)

    def t(a, dt=torch.float32):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    bf = torch.bfloat16
    ins = dict(q=t(x.q, bf), k=t(x.k, bf), v=t(x.v, bf), alpha=t(x.alpha), theta=t(x.theta),
               beta=t(x.beta), w=t(x.w), grad_o=t(dO, bf), grad_S=t(dS))
    return ins


def _args(ins, B, T, H, d, rot):
    import torch
    import recurrent_state_memory_amd as gdr
    a = gdr.BwdArgs()
    a.B, a.T, a.H, a.dk, a.dv = B, T, H, d, d
    a.decay = gdr.GDR_DECAY_ROT2 if rot else gdr.GDR_DECAY_DIAG
    for f in ("q", "k", "v", "alpha", "theta", "beta", "w", "grad_o", "grad_S"):
        setattr(a, f, None if ins[f] is None else ins[f].data_ptr())
    C = d // 2 if rot else d
    out = dict(grad_q=torch.empty(B, T, H, d, device="cuda"), grad_k=torch.empty(B, T, H, d, device="cuda"),
               grad_v=torch.empty(B, T, H, d, device="cuda"), grad_alpha=torch.empty(B, T, H, C, device="cuda"),
               grad_beta=torch.empty(B, T, H, device="cuda"), grad_w=torch.empty(B, T, H, device="cuda"),
               grad_S0=torch.empty(B, H, d, d, device="cuda"))
    if rot:
        out["grad_theta"] = torch.empty(B, T, H, C, device="cuda")
    for f, tns in out.items():
        setattr(a, f, tns.data_ptr())
    return a, out


@pytest.mark.parametrize("shapes", [((2, 300, 3, 128, "diag"), (1, 45, 2, 128, "diag")),
                                    ((2, 160, 2, 64, "rot2"), (1, 33, 1, 64, "rot2"))])
def test_noalloc_matches_workspace_backward(shapes):
    import torch
    import recurrent_state_memory_amd as gdr
    lib = gdr.load_library()
    for (B, T, H, d, decay) in shapes:
        rot = decay == "rot2"
        print(f"noalloc case B={B} T={T} H={H} d={d} {decay}", flush=True)
        ins = _case(B, T, H, d, decay, seed=B * 1000 + T)
        a_ref, ref = _args(ins, B, T, H, d, rot)
        need = lib.gdr_chunk_bwd_workspace(ctypes.byref(a_ref))
        assert 0 < need <= 256 << 20
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        a_ref.workspace, a_ref.workspace_bytes = ws.data_ptr(), need
        assert gdr.call_chunk_bwd(a_ref, torch.cuda.current_stream()) == gdr.GDR_OK
        a_na, got = _args(ins, B, T, H, d, rot)
        assert gdr.call_chunk_bwd_noalloc(a_na, torch.cuda.current_stream()) == gdr.GDR_OK
        torch.cuda.synchronize()
        for name in ref:
            r, g = ref[name].cpu().numpy(), got[name].cpu().numpy()
            assert np.all(np.isfinite(g)), name
            assert np.array_equal(r, g), (name, float(np.max(np.abs(r - g))))
