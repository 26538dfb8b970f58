"""Guard bands: every kernel writes exactly its outputs and nothing around them.

o, S_out and m_carry are views into larger buffers whose head and tail are
filled with a sentinel bit pattern; after ragged-length launches of every
kernel path the sentinels must be bit-identical."""
import numpy as np
import pytest

from _gpu import dev, io_dtype, random_state
from synth.gen import Workload, generate, generate_decode

pytestmark = pytest.mark.gpu

GUARD = 4096   # elements on each side (a multiple of 16 bytes for every dtype)


def guarded(shape, dtype, sentinel_bits):
    """A contiguous tensor of ``shape`` inside a buffer with sentinel guard bands."""
    import torch
    n = int(np.prod(shape))
    itemsize = torch.empty((), dtype=dtype).element_size()
    ity = {2: torch.int16, 4: torch.int32}[itemsize]
    buf = torch.empty(GUARD + n + GUARD, dtype=dtype, device="cuda")
    buf.view(ity).fill_(sentinel_bits)
    return buf, buf[GUARD:GUARD + n].view(shape)


def check_guards(buf, sentinel_bits, what):
    import torch
    itemsize = buf.element_size()
    ity = {2: torch.int16, 4: torch.int32}[itemsize]
    bits = buf.view(ity).cpu().numpy()
    head, tail = bits[:GUARD], bits[-GUARD:]
    assert np.all(head == sentinel_bits) and np.all(tail == sentinel_bits), f"{what}: guard band written"


@pytest.mark.parametrize("io,decay,dk,chunk,content", [
    ("bf16", "diag", 128, 64, False),     # pipelined, 64-channel tiles path
    ("bf16", "rot2", 64, 64, False),      # pipelined d = 64
    ("bf16", "diag", 128, 128, True),     # pipelined content-aware (value tiles + projection)
    ("bf16", "diag", 128, 16, True),      # sequential-stage content-aware (16-token window)
    ("f32", "rot2", 128, 32, False),      # sequential-stage fp32
    ("bf16", "diag", 32, 16, False),      # sequential-stage d = 32
])
def test_outputs_stay_inside_their_buffers(io, decay, dk, chunk, content):
    import torch
    import recurrent_state_memory_amd as gdr
    B, H, T = 2, 3, 3 * chunk + 5 if not content else 4 * chunk
    wl = Workload("guard", B, H, T, dk, dk, chunk, io, decay, content, 77)
    x = generate(wl, ub_std=1.0)
    iot = io_dtype(io)
    SENT16, SENT32 = 0x7FA5, 0x7FC0A5A5       # NaN patterns no kernel produces
    obuf, o = guarded((B, T, H, dk), iot, SENT16 if io == "bf16" else SENT32)
    sbuf, S = guarded((B, H, dk, dk), torch.float32, SENT32)
    mbuf, m = guarded((B, H, dk), torch.float32, SENT32)
    m.zero_()
    S0 = dev(random_state(B, H, dk, dk, 5))
    # a strong-decay burst so that both passes of the pipelined kernel run
    a = x.alpha.copy()
    a[:, 3:9] = 1e-6
    kw = dict(beta_logit=dev(x.beta_logit), ub_down=dev(x.ub_down), ub_up=dev(x.ub_up),
              m_carry=m) if content else dict(beta=dev(x.beta))
    for alpha in (x.alpha, a):
        gdr.gdr_chunk_fwd(dev(x.q, iot), dev(x.k, iot), dev(x.v, iot), dev(alpha), dev(x.w),
                          theta=dev(x.theta), S0=S0, chunk=chunk, o=o, S_out=S, **kw)
        torch.cuda.synchronize()
        check_guards(obuf, SENT16 if io == "bf16" else SENT32, "o")
        check_guards(sbuf, SENT32, "S_out")
        check_guards(mbuf, SENT32, "m_carry")
        assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_decode_stays_inside_its_buffers():
    import torch
    import recurrent_state_memory_amd as gdr
    wl = Workload("guard", 1, 16, 1, 128, 128, 64, "bf16", "rot2", False, 3, decay_scale=0.05)
    d = generate_decode(wl, N=9, rng=np.random.default_rng(8))
    SENT16, SENT32 = 0x7FA5, 0x7FC0A5A5
    sbuf, S = guarded((d.N, d.H, 128, 128), torch.float32, SENT32)
    S.copy_(dev(d.S))
    obuf, o = guarded((d.N, d.H, 128), torch.bfloat16, SENT16)
    bf = torch.bfloat16
    gdr.gdr_step_decode(S, dev(d.q, bf), dev(d.k, bf), dev(d.v, bf), dev(d.alpha), dev(d.beta),
                        dev(d.w), theta=dev(d.theta), o=o)
    torch.cuda.synchronize()
    check_guards(sbuf, SENT32, "S")
    check_guards(obuf, SENT16, "o")
