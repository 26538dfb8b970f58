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

FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MISALIGNED = 0x10004


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_header_symbols():
    lib = gdr.load_library()
    names = _declared()
    assert {"gdr_chunk_fwd", "gdr_step_decode", "gdr_chunk_fwd_workspace",
            "gdr_status_str", "gdr_abi_version"} <= set(names)
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
    (dict(theta=FAKE), gdr.GDR_ERR_ARG),
]


@pytest.mark.parametrize("kw,status", STEP_CASES)
def test_step_rejects_before_any_hip_call(kw, status):
    assert gdr.call_step_decode(_good_step(**kw)) == status


def test_struct_layout_matches_header(tmp_path):
    """Field offsets of the ctypes mirrors equal the C compiler's offsetof()."""
    fields = {"gdr_fwd_args": gdr.FwdArgs, "gdr_step_args": gdr.StepArgs}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"',
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
