"""C-ABI tests that need no GPU: the library loads, exports what the header
declares, and rejects every invalid argument before touching HIP."""
import ctypes
import os
import re
import subprocess

import pytest

import recurrent_state_memory_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")
RAVEN_HEADER = os.path.join(ROOT, "include", "gdr_raven.h")
PERM_HEADER = os.path.join(ROOT, "include", "gdr_perm.h")

FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MISALIGNED = 0x10004


def _declared():
    """Functions declared by every header under include/."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, f)).read(), flags=re.S)
            names |= set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_library_loads_and_exports_header_symbols():
    lib = gdr.load_library()
    names = _declared()
    assert {"gdr_chunk_fwd", "gdr_chunk_fwd_gated", "gdr_chunk_bwd", "gdr_chunk_bwd_workspace",
            "gdr_step_decode", "gdr_chunk_fwd_workspace", "gdr_status_str",
            "gdr_abi_version", "gdr_chunk_bwd_noalloc", "gdr_raven_fwd",
            "gdr_perm_fwd", "gdr_chunk_bwd_gated", "gdr_chunk_bwd_gated_workspace"} <= set(names)
    for nm in names:
        assert hasattr(lib, nm), nm
    out = subprocess.run(["nm", "-D", "--defined-only", gdr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdr_\w+)", out))
    assert set(names) <= exported


def test_abi_version_and_status_strings():
    lib = gdr.load_library()
    assert lib.gdr_abi_version() == 1
    for s in range(9):
        assert gdr.status_str(s)
    assert gdr.status_str(12345) == "unknown status"


def _good_fwd(**kw):
    a = gdr.FwdArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.chunk = 2, 100, 4, 64, 64, 64
    a.io_dtype, a.decay = gdr.GDR_BF16, gdr.GDR_DECAY_DIAG
    for f in ("q", "k", "v", "alpha", "beta", "w", "o"):
        setattr(a, f, FAKE)
    for f, val in kw.items():
        setattr(a, f, val)
    return a


FWD_CASES = [
    (dict(q=None), gdr.GDR_ERR_NULL),
    (dict(w=None), gdr.GDR_ERR_NULL),
    (dict(o=None), gdr.GDR_ERR_NULL),
    (dict(beta=None), gdr.GDR_ERR_NULL),
    (dict(B=0), gdr.GDR_ERR_SHAPE),
    (dict(T=0), gdr.GDR_ERR_SHAPE),
    (dict(H=-1), gdr.GDR_ERR_SHAPE),
    (dict(chunk=0), gdr.GDR_ERR_SHAPE),
    (dict(dk=48, dv=48), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dk=64, dv=128), gdr.GDR_ERR_UNSUPPORTED),
    (dict(chunk=24), gdr.GDR_ERR_UNSUPPORTED),
    (dict(chunk=256), gdr.GDR_ERR_UNSUPPORTED),
    (dict(io_dtype=7), gdr.GDR_ERR_DTYPE),
    (dict(decay=3), gdr.GDR_ERR_DTYPE),
    (dict(q=MISALIGNED), gdr.GDR_ERR_ALIGN),
    (dict(S0=MISALIGNED), gdr.GDR_ERR_ALIGN),
    (dict(theta=FAKE), gdr.GDR_ERR_ARG),                       # diag with theta
    (dict(decay=gdr.GDR_DECAY_ROT2), gdr.GDR_ERR_NULL),        # rot2 without theta
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL), gdr.GDR_ERR_NULL),    # reflections without theta
    # reflection blocks: the pipelined kernel's plain launch only
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL, theta=FAKE, io_dtype=gdr.GDR_F32),
     gdr.GDR_ERR_UNSUPPORTED),
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL, theta=FAKE, dk=32, dv=32), gdr.GDR_ERR_UNSUPPORTED),
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL, theta=FAKE, beta=None, beta_logit=FAKE, ub_down=FAKE,
          ub_up=FAKE, ub_rank=16), gdr.GDR_ERR_UNSUPPORTED),
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL, theta=FAKE, T=1 << 23, H=1), gdr.GDR_ERR_UNSUPPORTED),
    (dict(m_carry=FAKE), gdr.GDR_ERR_ARG),                     # carry without content
    (dict(ub_down=FAKE), gdr.GDR_ERR_ARG),
    (dict(beta_logit=FAKE, ub_down=FAKE, ub_up=FAKE, ub_rank=16), gdr.GDR_ERR_ARG),  # beta too
    (dict(beta=None, beta_logit=FAKE, ub_up=FAKE, ub_rank=16), gdr.GDR_ERR_NULL),
    (dict(beta=None, beta_logit=FAKE, ub_down=FAKE, ub_up=FAKE, ub_rank=0),
     gdr.GDR_ERR_UNSUPPORTED),
    (dict(beta=None, beta_logit=FAKE, ub_down=FAKE, ub_up=FAKE, ub_rank=16, m_carry=FAKE),
     gdr.GDR_ERR_SHAPE),                                       # T % chunk != 0 with carry
    (dict(S0=FAKE, S_out=FAKE + 64), gdr.GDR_ERR_ARG),         # partial overlap
    (dict(workspace_bytes=16), gdr.GDR_ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,status", FWD_CASES)
def test_fwd_rejects_before_any_hip_call(kw, status):
    assert gdr.call_chunk_fwd(_good_fwd(**kw)) == status


def _good_gate(**kw):
    g = gdr.GateArgs()
    g.decay_x, g.decay_a, g.qk_l2norm, g.reserved = FAKE, FAKE, 1, 0
    for f, val in kw.items():
        setattr(g, f, val)
    return g


GATE_CASES = [
    (dict(), dict(reserved=1), gdr.GDR_ERR_ARG),
    (dict(), dict(decay_x=None), gdr.GDR_ERR_NULL),
    (dict(), dict(decay_a=None), gdr.GDR_ERR_NULL),
    (dict(), dict(decay_x=FAKE + 2), gdr.GDR_ERR_ALIGN),
    (dict(), dict(decay_a=FAKE + 2), gdr.GDR_ERR_ALIGN),
    (dict(alpha=FAKE), dict(), gdr.GDR_ERR_ARG),              # decay comes from decay_x
    (dict(io_dtype=gdr.GDR_F32), dict(), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dk=32, dv=32), dict(), gdr.GDR_ERR_UNSUPPORTED),
    (dict(beta=None, beta_logit=FAKE, ub_down=FAKE, ub_up=FAKE, ub_rank=16), dict(),
     gdr.GDR_ERR_UNSUPPORTED),
    (dict(T=1 << 23, H=1), dict(), gdr.GDR_ERR_UNSUPPORTED),  # T * H * dk >= 2^29
    (dict(beta=None), dict(), gdr.GDR_ERR_NULL),
    (dict(decay=gdr.GDR_DECAY_ROT2), dict(), gdr.GDR_ERR_NULL),  # rot2 without theta
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL, theta=FAKE), dict(), gdr.GDR_ERR_UNSUPPORTED),
    (dict(B=0), dict(), gdr.GDR_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,gkw,status", GATE_CASES)
def test_gated_fwd_rejects_before_any_hip_call(kw, gkw, status):
    a = _good_fwd(alpha=None, **{k: v for k, v in kw.items() if k != "alpha"})
    if "alpha" in kw:
        a.alpha = kw["alpha"]
    assert gdr.call_chunk_fwd_gated(a, _good_gate(**gkw)) == status


def test_gated_fwd_null_structs():
    lib = gdr.load_library()
    g = _good_gate()
    assert lib.gdr_chunk_fwd_gated(None, ctypes.byref(g), None) == gdr.GDR_ERR_NULL
    assert lib.gdr_chunk_fwd_gated(ctypes.byref(_good_fwd(alpha=None)), None, None) == gdr.GDR_ERR_NULL


def _good_bwd(**kw):
    a = gdr.BwdArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.decay = 2, 100, 4, 64, 64, gdr.GDR_DECAY_DIAG
    for f in ("q", "k", "v", "alpha", "beta", "w", "grad_o", "grad_q", "grad_k", "grad_v",
              "grad_alpha", "grad_beta", "grad_w"):
        setattr(a, f, FAKE)
    for f, val in kw.items():
        setattr(a, f, val)
    return a


BWD_CASES = [
    (dict(q=None), gdr.GDR_ERR_NULL),
    (dict(grad_o=None), gdr.GDR_ERR_NULL),
    (dict(grad_w=None), gdr.GDR_ERR_NULL),
    (dict(dk=32, dv=32), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dk=64, dv=128), gdr.GDR_ERR_UNSUPPORTED),
    (dict(decay=5), gdr.GDR_ERR_DTYPE),
    (dict(H=0), gdr.GDR_ERR_SHAPE),
    (dict(T=1 << 23, H=1), gdr.GDR_ERR_UNSUPPORTED),
    (dict(theta=FAKE), gdr.GDR_ERR_ARG),
    (dict(decay=gdr.GDR_DECAY_ROT2, theta=FAKE), gdr.GDR_ERR_NULL),   # no grad_theta
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL, theta=FAKE, grad_theta=FAKE), gdr.GDR_ERR_UNSUPPORTED),
    (dict(grad_S0=MISALIGNED), gdr.GDR_ERR_ALIGN),
    (dict(), gdr.GDR_ERR_WORKSPACE),                                  # no workspace
    (dict(workspace=FAKE, workspace_bytes=1024), gdr.GDR_ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,status", BWD_CASES)
def test_bwd_rejects_before_any_hip_call(kw, status):
    assert gdr.call_chunk_bwd(_good_bwd(**kw)) == status


def test_bwd_noalloc_rejects_before_any_hip_call():
    """The static-scratch backward: no caller workspace, at most 256 MiB of it,
    and the backward's own argument checks."""
    lib = gdr.load_library()
    assert lib.gdr_chunk_bwd_noalloc(None, None) == gdr.GDR_ERR_NULL
    assert gdr.call_chunk_bwd_noalloc(_good_bwd(workspace=FAKE, workspace_bytes=1 << 30)) == \
        gdr.GDR_ERR_ARG
    assert gdr.call_chunk_bwd_noalloc(_good_bwd(dk=32, dv=32)) == gdr.GDR_ERR_UNSUPPORTED
    assert gdr.call_chunk_bwd_noalloc(_good_bwd(grad_q=None)) == gdr.GDR_ERR_NULL
    big = _good_bwd(B=8, T=4096, H=16, dk=128, dv=128)      # ~2.9 GB of workspace
    assert lib.gdr_chunk_bwd_workspace(ctypes.byref(big)) > 256 << 20
    assert gdr.call_chunk_bwd_noalloc(big) == gdr.GDR_ERR_WORKSPACE


def test_bwd_workspace_size():
    """Checkpoints of every 32-token block, the recompute's o, the partials and
    one range flag per (b, h, 32-channel value tile)."""
    lib = gdr.load_library()
    a = _good_bwd()
    nc = (100 + 31) // 32
    parts = (2 * 4 * nc * 64 * 64 * 4, 2 * 100 * 4 * 64 * 2, 2 * (2 * 100 * 4) * (3 * 64 + 2) * 4,
             2 * 4 * 2 * 4)
    want = sum(parts)
    rounded = sum(-(-x // 256) * 256 for x in parts)
    assert lib.gdr_chunk_bwd_workspace(ctypes.byref(a)) == rounded >= want
    assert lib.gdr_chunk_bwd_workspace(ctypes.byref(_good_bwd(dk=48, dv=48))) == 0


def test_fwd_null_args():
    lib = gdr.load_library()
    assert lib.gdr_chunk_fwd(None, None) == gdr.GDR_ERR_NULL
    assert lib.gdr_step_decode(None, None) == gdr.GDR_ERR_NULL
    assert lib.gdr_chunk_fwd_workspace(ctypes.byref(_good_fwd())) == 0


def _good_step(**kw):
    a = gdr.StepArgs()
    a.N, a.H, a.dk, a.dv = 4, 2, 128, 128
    a.io_dtype, a.decay = gdr.GDR_BF16, gdr.GDR_DECAY_DIAG
    for f in ("q", "k", "v", "alpha", "beta", "w", "S", "o"):
        setattr(a, f, FAKE)
    for f, val in kw.items():
        setattr(a, f, val)
    return a


STEP_CASES = [
    (dict(S=None), gdr.GDR_ERR_NULL),
    (dict(beta=None), gdr.GDR_ERR_NULL),
    (dict(N=0), gdr.GDR_ERR_SHAPE),
    (dict(dk=96, dv=96), gdr.GDR_ERR_UNSUPPORTED),
    (dict(io_dtype=2), gdr.GDR_ERR_DTYPE),
    (dict(S=MISALIGNED), gdr.GDR_ERR_ALIGN),
    (dict(decay=gdr.GDR_DECAY_ROT2), gdr.GDR_ERR_NULL),
    (dict(decay=gdr.GDR_DECAY_DIHEDRAL), gdr.GDR_ERR_NULL),
    (dict(theta=FAKE), gdr.GDR_ERR_ARG),
]


@pytest.mark.parametrize("kw,status", STEP_CASES)
def test_step_rejects_before_any_hip_call(kw, status):
    assert gdr.call_step_decode(_good_step(**kw)) == status


def test_struct_layout_matches_header(tmp_path):
    """Field offsets of the ctypes mirrors equal the C compiler's offsetof()."""
    fields = {"gdr_fwd_args": gdr.FwdArgs, "gdr_step_args": gdr.StepArgs,
              "gdr_gate_args": gdr.GateArgs, "gdr_bwd_args": gdr.BwdArgs,
              "gdr_raven_args": gdr.RavenArgs, "gdr_perm_args": gdr.PermArgs}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"',
             f'#include "{RAVEN_HEADER}"', f'#include "{PERM_HEADER}"',
             "int main(void) {"]
    for cname, cls in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for ln in out.splitlines():
        cname, f, val = ln.split()
        got[(cname, f)] = int(val)
    for cname, cls in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls)
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and has no CPU path."""
    pkg = os.path.join(ROOT, "recurrent_state_memory_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.replace("no oracle", ""), f
                assert "import numpy" not in txt, f


# ------------------------------------------------------------ binding checks
def _cpu_fwd_args(B=2, T=5, H=3, dk=8, dv=8, rot=False, content=False):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    g = dk // 2 if rot else dk
    a = dict(q=torch.zeros(B, T, H, dk, dtype=bf), k=torch.zeros(B, T, H, dk, dtype=bf),
             v=torch.zeros(B, T, H, dv, dtype=bf), alpha=torch.ones(B, T, H, g, dtype=f32),
             w=torch.zeros(B, T, H, dtype=f32))
    if rot:
        a["theta"] = torch.zeros(B, T, H, g, dtype=f32)
    if content:
        a.update(beta_logit=torch.zeros(B, T, H, dtype=f32), ub_down=torch.zeros(H, 4, dv),
                 ub_up=torch.zeros(H, 4))
    else:
        a["beta"] = torch.zeros(B, T, H, dtype=f32)
    return a


def test_binding_accepts_good_shapes_then_needs_gpu():
    """Correct shapes pass every check; the first thing rejected is the CPU device."""
    for kw in (dict(), dict(rot=True), dict(content=True)):
        with pytest.raises(ValueError, match="GPU"):
            gdr.gdr_chunk_fwd(**_cpu_fwd_args(**kw))


@pytest.mark.parametrize("name,bad", [
    ("alpha", lambda a: a["alpha"][..., :4].contiguous()),       # scalar-ish gate, short
    ("alpha", lambda a: a["alpha"].to(__import__("torch").bfloat16)),
    ("w", lambda a: a["w"][:, :, :2].contiguous()),
    ("beta", lambda a: a["beta"][:1].contiguous()),
    ("k", lambda a: a["k"][:, :4].contiguous()),
    ("v", lambda a: a["v"].float()),
    ("S0", lambda a: __import__("torch").zeros(2, 3, 8, 4)),
    ("S_out", lambda a: __import__("torch").zeros(2, 3, 8, 8, dtype=__import__("torch").bfloat16)),
    ("o", lambda a: __import__("torch").zeros(2, 5, 3, 4, dtype=__import__("torch").bfloat16)),
    ("alpha", lambda a: a["alpha"].transpose(1, 2).contiguous().transpose(1, 2)),  # not contiguous
])
def test_binding_rejects_bad_argument(name, bad):
    a = _cpu_fwd_args()
    a[name] = bad(a)
    with pytest.raises(ValueError, match=name):
        gdr.gdr_chunk_fwd(**a)


def test_binding_rejects_bad_content_and_rotation_arguments():
    import torch
    a = _cpu_fwd_args(rot=True)
    a["theta"] = torch.zeros(2, 5, 3, 8)                       # per channel, not per pair
    with pytest.raises(ValueError, match="theta"):
        gdr.gdr_chunk_fwd(**a)
    a = _cpu_fwd_args(content=True)
    a["ub_down"] = torch.zeros(3, 4, 4)
    with pytest.raises(ValueError, match="ub_down"):
        gdr.gdr_chunk_fwd(**a)
    a = _cpu_fwd_args(content=True)
    a["m_carry"] = torch.zeros(2, 3, 4)
    with pytest.raises(ValueError, match="m_carry"):
        gdr.gdr_chunk_fwd(**a)
    a = _cpu_fwd_args()
    a["m_carry"] = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="content-aware"):
        gdr.gdr_chunk_fwd(**a)
    a = _cpu_fwd_args()
    with pytest.raises(ValueError, match="reflection"):
        gdr.gdr_chunk_fwd(**a, reflections=True)               # no theta


def _cpu_gated_args(B=2, T=5, H=3, d=8, rot=False):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    g = d // 2 if rot else d
    a = dict(q=torch.zeros(B, T, H, d, dtype=bf), k=torch.zeros(B, T, H, d, dtype=bf),
             v=torch.zeros(B, T, H, d, dtype=bf), decay_x=torch.zeros(B, T, H, g, dtype=bf),
             decay_a=torch.ones(H, dtype=f32), w=torch.zeros(B, T, H, dtype=f32),
             beta=torch.zeros(B, T, H, dtype=f32))
    if rot:
        a["theta"] = torch.zeros(B, T, H, g, dtype=f32)
    return a


def test_gated_binding_checks():
    """Good shapes pass every check (then the CPU device is refused); each bad
    argument is named."""
    import torch
    for rot in (False, True):
        with pytest.raises(ValueError, match="GPU"):
            gdr.gdr_chunk_fwd_gated(**_cpu_gated_args(rot=rot))
    bad = [("decay_x", torch.zeros(2, 5, 3, 8)),                     # fp32, not bf16
           ("decay_x", torch.zeros(2, 5, 3, 4, dtype=torch.bfloat16)),
           ("decay_a", torch.ones(2)), ("decay_a", torch.ones(3, dtype=torch.bfloat16)),
           ("q", torch.zeros(2, 5, 3, 8)), ("v", torch.zeros(2, 5, 3, 8)),
           ("beta", torch.zeros(2, 5)), ("w", torch.zeros(2, 5, 3, dtype=torch.bfloat16))]
    for name, val in bad:
        a = _cpu_gated_args()
        a[name] = val
        with pytest.raises(ValueError, match=name):
            gdr.gdr_chunk_fwd_gated(**a)
    a = _cpu_gated_args(rot=True)
    a["theta"] = torch.zeros(2, 5, 3, 8)
    with pytest.raises(ValueError, match="theta"):
        gdr.gdr_chunk_fwd_gated(**a)


def test_bwd_binding_checks():
    """Good shapes pass every check (then the CPU device is refused); each bad
    argument is named."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    B, T, H, d = 2, 5, 3, 8
    good = dict(q=torch.zeros(B, T, H, d, dtype=bf), k=torch.zeros(B, T, H, d, dtype=bf),
                v=torch.zeros(B, T, H, d, dtype=bf), alpha=torch.ones(B, T, H, d),
                w=torch.zeros(B, T, H), beta=torch.zeros(B, T, H),
                grad_o=torch.zeros(B, T, H, d, dtype=bf))
    with pytest.raises(ValueError, match="GPU"):
        gdr.gdr_chunk_bwd(**good)
    for name, val in (("grad_o", torch.zeros(B, T, H, d)), ("alpha", torch.ones(B, T, H, 4)),
                      ("q", torch.zeros(B, T, H, d)), ("beta", torch.zeros(B, T)),
                      ("grad_S", torch.zeros(B, H, d, 4)), ("S0", torch.zeros(B, H, d, d, dtype=bf))):
        a = dict(good)
        a[name] = val
        with pytest.raises(ValueError, match=name):
            gdr.gdr_chunk_bwd(**a)


def test_bwd_gated_binding_checks():
    """gdr_chunk_bwd_gated: good shapes pass every check (then the CPU device is
    refused); each bad argument is named, the rotation form included."""
    import torch
    bf = torch.bfloat16
    B, T, H, d = 2, 5, 3, 8
    good = dict(q=torch.zeros(B, T, H, d, dtype=bf), k=torch.zeros(B, T, H, d, dtype=bf),
                v=torch.zeros(B, T, H, d, dtype=bf), decay_x=torch.zeros(B, T, H, d, dtype=bf),
                decay_a=torch.ones(H), w=torch.zeros(B, T, H), beta=torch.zeros(B, T, H),
                grad_o=torch.zeros(B, T, H, d, dtype=bf))
    with pytest.raises(ValueError, match="GPU"):
        gdr.gdr_chunk_bwd_gated(**good)
    for name, val in (("decay_x", torch.zeros(B, T, H, d)), ("decay_a", torch.ones(H + 1)),
                      ("grad_o", torch.zeros(B, T, H, d)), ("k", torch.zeros(B, T, H, d)),
                      ("w", torch.zeros(B, T)), ("grad_S", torch.zeros(B, H, d, 4)),
                      ("S0", torch.zeros(B, H, d, d, dtype=bf))):
        a = dict(good)
        a[name] = val
        with pytest.raises(ValueError, match=name):
            gdr.gdr_chunk_bwd_gated(**a)
    a = dict(good, decay_x=torch.zeros(B, T, H, d // 2, dtype=bf),
             theta=torch.zeros(B, T, H, d))   # theta must match the pair-wise decay
    with pytest.raises(ValueError, match="theta"):
        gdr.gdr_chunk_bwd_gated(**a)


def test_decode_binding_checks():
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    N, H, d = 3, 2, 8
    good = dict(S=torch.zeros(N, H, d, d), q=torch.zeros(N, H, d, dtype=bf),
                k=torch.zeros(N, H, d, dtype=bf), v=torch.zeros(N, H, d, dtype=bf),
                alpha=torch.ones(N, H, d), beta=torch.zeros(N, H), w=torch.zeros(N, H))
    with pytest.raises(ValueError, match="GPU"):
        gdr.gdr_step_decode(**good)
    for name, val in (("S", torch.zeros(N, H, d, d, dtype=bf)), ("alpha", torch.ones(N, H)),
                      ("beta", torch.zeros(N, H, dtype=bf)), ("k", torch.zeros(N, H, d)),
                      ("v", torch.zeros(N, H, 4, dtype=bf)), ("w", torch.zeros(N, 1))):
        a = dict(good)
        a[name] = val
        with pytest.raises(ValueError, match=name):
            gdr.gdr_step_decode(**a)
    with pytest.raises(ValueError, match="reflection"):
        gdr.gdr_step_decode(**good, reflections=True)


def test_host_half_under_sanitizers(tmp_path):
    """gdr_api.cpp (argument checks, parameter marshalling) built for the host with
    AddressSanitizer and UndefinedBehaviorSanitizer, kernel launchers replaced by
    recorders (tests/abi_host_harness.cpp): every valid call reaches the launcher
    with its fields intact, every invalid one is rejected, and no check overflows."""
    import shutil
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "abi_harness"
    cmd = [gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "recurrent_state_memory_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g",
           os.path.join(ROOT, "tests", "abi_host_harness.cpp"),
           os.path.join(ROOT, "recurrent_state_memory_amd", "csrc", "gdr_api.cpp"),
           os.path.join(ROOT, "recurrent_state_memory_amd", "csrc", "raven_api.cpp"),
           os.path.join(ROOT, "recurrent_state_memory_amd", "csrc", "perm_api.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    # the environment is passed through unchanged; ASan is told not to insist on
    # coming first in the library list
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0")
    out = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert out.returncode == 0 and "ABI_HARNESS_OK" in out.stdout, out.stderr


# ------------------------------------------------------------ Raven slot memory
def _good_raven(**kw):
    r = gdr.RavenArgs()
    r.B, r.T, r.H, r.dk, r.dv, r.slots, r.topk, r.scale = 2, 70, 3, 128, 128, 64, 8, 0.088
    for f in ("q", "k", "v", "z", "a", "o"):
        setattr(r, f, FAKE)
    for f, val in kw.items():
        setattr(r, f, val)
    return r


RAVEN_CASES = [
    (dict(q=None), gdr.GDR_ERR_NULL),
    (dict(z=None), gdr.GDR_ERR_NULL),
    (dict(a=None), gdr.GDR_ERR_NULL),
    (dict(o=None), gdr.GDR_ERR_NULL),
    (dict(T=0), gdr.GDR_ERR_SHAPE),
    (dict(topk=0), gdr.GDR_ERR_SHAPE),
    (dict(topk=9), gdr.GDR_ERR_UNSUPPORTED),
    (dict(slots=128), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dk=32, dv=32), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dk=128, dv=64), gdr.GDR_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), gdr.GDR_ERR_UNSUPPORTED),
    (dict(z=MISALIGNED), gdr.GDR_ERR_ALIGN),
    (dict(Sk0=FAKE, Sk_out=FAKE + 64), gdr.GDR_ERR_ARG),      # partial overlap
    (dict(Sk_out=FAKE, Sv_out=FAKE), gdr.GDR_ERR_ARG),        # the two states in one buffer
]


@pytest.mark.parametrize("kw,status", RAVEN_CASES)
def test_raven_rejects_before_any_hip_call(kw, status):
    assert gdr.call_raven_fwd(_good_raven(**kw)) == status


def test_raven_binding_checks():
    """Good shapes pass every check (then the CPU device is refused); each bad
    shape or dtype is named."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    B, T, H, d, M = 2, 5, 3, 64, 64
    good = dict(q=torch.zeros(B, T, H, d, dtype=bf), k=torch.zeros(B, T, H, d, dtype=bf),
                v=torch.zeros(B, T, H, d, dtype=bf), z=torch.zeros(B, T, H, M, dtype=bf),
                a=torch.zeros(B, T, H, dtype=f32))
    with pytest.raises(ValueError, match="GPU"):
        gdr.gdr_raven_fwd(**good, topk=8)
    for name, val in (("k", torch.zeros(B, T, H, d)), ("z", torch.zeros(B, T, H + 1, M, dtype=bf)),
                      ("a", torch.zeros(B, T, H, dtype=bf)), ("v", torch.zeros(B, T, 2, d, dtype=bf)),
                      ("Sk0", torch.zeros(B, H, M, d - 1)), ("Sv0", torch.zeros(B, H, M, d, dtype=bf))):
        a = dict(good)
        a[name] = val
        with pytest.raises(ValueError, match=name):
            gdr.gdr_raven_fwd(**a, topk=8)


# ------------------------------------------------------------ partial permutations
def _good_perm(**kw):
    a = gdr.PermArgs()
    a.B, a.T, a.H, a.dk, a.dv = 2, 70, 3, 128, 128
    for f in ("q", "k", "v", "src", "beta", "w", "o"):
        setattr(a, f, FAKE)
    for f, val in kw.items():
        setattr(a, f, val)
    return a


PERM_CASES = [
    (dict(src=None), gdr.GDR_ERR_NULL),
    (dict(beta=None), gdr.GDR_ERR_NULL),
    (dict(o=None), gdr.GDR_ERR_NULL),
    (dict(T=0), gdr.GDR_ERR_SHAPE),
    (dict(dk=32), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dv=24), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dv=48), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dv=288), gdr.GDR_ERR_UNSUPPORTED),
    (dict(src=MISALIGNED), gdr.GDR_ERR_ALIGN),
    (dict(S0=FAKE, S_out=FAKE + 64), gdr.GDR_ERR_ARG),
    (dict(B=1 << 20, T=1 << 12, H=1 << 8), gdr.GDR_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,status", PERM_CASES)
def test_perm_rejects_before_any_hip_call(kw, status):
    assert gdr.call_perm_fwd(_good_perm(**kw)) == status


def test_perm_binding_checks():
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    B, T, H, d = 2, 5, 3, 64
    good = dict(q=torch.zeros(B, T, H, d, dtype=bf), k=torch.zeros(B, T, H, d, dtype=bf),
                v=torch.zeros(B, T, H, d, dtype=bf), w=torch.zeros(B, T, H, dtype=f32),
                src=torch.zeros(B, T, H, d, dtype=torch.int16), beta=torch.zeros(B, T, H, dtype=f32))
    with pytest.raises(ValueError, match="GPU"):
        gdr.gdr_perm_fwd(**good)
    for name, val in (("src", torch.zeros(B, T, H, d, dtype=torch.int32)),
                      ("src", torch.zeros(B, T, H, d - 1, dtype=torch.int16)),
                      ("beta", torch.zeros(B, T, H, dtype=bf)), ("w", torch.zeros(B, T, 1)),
                      ("S0", torch.zeros(B, H, d, d, dtype=bf))):
        a = dict(good)
        a[name] = val
        with pytest.raises(ValueError, match=name):
            gdr.gdr_perm_fwd(**a)
