"""MI355X (gfx950) gated delta-rule library: Python binding over libgdr.so.

The binding only marshals arguments: it reads device pointers and the
current HIP stream from torch tensors, fills the C structs declared in
``include/gdr.h`` and calls the exported functions.  Every step of the
computation runs in the HIP kernels of ``libgdr.so``; there is no fallback.
If the library has not been built, every call raises ``RuntimeError``.

Entry points (same names as the C ABI):

* ``gdr_chunk_fwd``   -- chunked forward over a sequence, returns (o, S_out)
* ``gdr_step_decode`` -- one token on a batch of states, in place, returns o
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_ERR_NULL, GDR_ERR_SHAPE, GDR_ERR_DTYPE, GDR_ERR_UNSUPPORTED, \
    GDR_ERR_ALIGN, GDR_ERR_WORKSPACE, GDR_ERR_HIP, GDR_ERR_ARG = range(9)
GDR_F32, GDR_BF16 = 0, 1
GDR_DECAY_DIAG, GDR_DECAY_ROT2 = 0, 1
ABI_VERSION = 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class FwdArgs(ctypes.Structure):
    """Mirror of ``gdr_fwd_args``."""
    _fields_ = [
        ("B", _i32), ("T", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32),
        ("chunk", _i32), ("io_dtype", _i32), ("decay", _i32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("alpha", _vp), ("theta", _vp),
        ("beta", _vp), ("w", _vp), ("beta_logit", _vp), ("ub_down", _vp),
        ("ub_up", _vp), ("ub_rank", _i32), ("reserved0", _i32), ("m_carry", _vp),
        ("S0", _vp), ("o", _vp), ("S_out", _vp), ("workspace", _vp),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class StepArgs(ctypes.Structure):
    """Mirror of ``gdr_step_args``."""
    _fields_ = [
        ("N", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32),
        ("io_dtype", _i32), ("decay", _i32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("alpha", _vp), ("theta", _vp),
        ("beta", _vp), ("w", _vp), ("S", _vp), ("o", _vp),
    ]


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gdr status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libgdr.so (built by ``python -m recurrent_state_memory_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m recurrent_state_memory_amd.build`")
    lib = ctypes.CDLL(p)
    lib.gdr_chunk_fwd.argtypes = [ctypes.POINTER(FwdArgs), _vp]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_fwd_workspace.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.gdr_chunk_fwd_workspace.restype = ctypes.c_size_t
    lib.gdr_step_decode.argtypes = [ctypes.POINTER(StepArgs), _vp]
    lib.gdr_step_decode.restype = ctypes.c_int
    lib.gdr_status_str.argtypes = [ctypes.c_int]
    lib.gdr_status_str.restype = ctypes.c_char_p
    lib.gdr_abi_version.argtypes = []
    lib.gdr_abi_version.restype = ctypes.c_int
    if lib.gdr_abi_version() != ABI_VERSION:
        raise RuntimeError("libgdr ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().gdr_status_str(status).decode()


def _check(status: int):
    if status != GDR_OK:
        raise GdrError(status, status_str(status))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("gdr: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("gdr: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _io(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise ValueError(f"gdr: q/k/v must be bfloat16 or float32, got {t.dtype}")


def call_chunk_fwd(args: FwdArgs, stream=None) -> int:
    """Raw call with a filled ``FwdArgs``; returns the status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_chunk_fwd(ctypes.byref(args), s)


def call_step_decode(args: StepArgs, stream=None) -> int:
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_step_decode(ctypes.byref(args), s)


def gdr_chunk_fwd(q, k, v, alpha, w, beta=None, *, theta=None, S0=None, chunk=64,
                  o=None, S_out=None, return_state=True, beta_logit=None,
                  ub_down=None, ub_up=None, m_carry=None, stream=None):
    """Chunked gated delta-rule forward (see ``gdr_chunk_fwd`` in include/gdr.h).

    q, k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32, same dtype); alpha fp32
    [B,T,H,dk] (per-channel decay) or [B,T,H,dk/2] with ``theta`` (2x2
    rotation-decay blocks); beta, w fp32 [B,T,H].  Content-aware erase: pass
    ``beta_logit``, ``ub_down`` [H,r,dv], ``ub_up`` [H,r] instead of ``beta``.
    Returns (o [B,T,H,dv], S_out [B,H,dv,dk] fp32 or None).
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if S_out is None and return_state:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    a = FwdArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.chunk = B, T, H, dk, dv, chunk
    a.io_dtype = _io(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("gdr: q, k, v and o must share one dtype")
    a.decay = GDR_DECAY_ROT2 if theta is not None else GDR_DECAY_DIAG
    a.q, a.k, a.v, a.alpha, a.theta = map(_ptr, (q, k, v, alpha, theta))
    a.beta, a.w, a.beta_logit = map(_ptr, (beta, w, beta_logit))
    a.ub_down, a.ub_up, a.m_carry = map(_ptr, (ub_down, ub_up, m_carry))
    a.ub_rank = 0 if ub_up is None else int(ub_up.shape[-1])
    a.S0, a.o, a.S_out = _ptr(S0), _ptr(o), _ptr(S_out)
    a.workspace, a.workspace_bytes = None, 0
    for t in (alpha, theta, beta, w, beta_logit, ub_down, ub_up, m_carry, S0, S_out):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("gdr: gates, projections and states must be float32")
    _check(call_chunk_fwd(a, _stream(stream)))
    return o, S_out


def gdr_step_decode(S, q, k, v, alpha, beta, w, *, theta=None, o=None, stream=None):
    """One token on N states in place (see ``gdr_step_decode`` in include/gdr.h).

    S [N,H,dv,dk] fp32 (overwritten), q,k [N,H,dk], v [N,H,dv], alpha [N,H,dk]
    or gamma [N,H,dk/2] with theta, beta, w [N,H].  Returns o [N,H,dv].
    """
    import torch
    N, H, dv, dk = S.shape
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    a = StepArgs()
    a.N, a.H, a.dk, a.dv = N, H, dk, dv
    a.io_dtype = _io(q)
    a.decay = GDR_DECAY_ROT2 if theta is not None else GDR_DECAY_DIAG
    a.q, a.k, a.v, a.alpha, a.theta = map(_ptr, (q, k, v, alpha, theta))
    a.beta, a.w, a.S, a.o = map(_ptr, (beta, w, S, o))
    _check(call_step_decode(a, _stream(stream)))
    return o
