"""MI355X (gfx950) gated delta-rule library: Python binding over libgdr.so.

The binding only marshals arguments: it reads device pointers and the
current HIP stream from torch tensors, fills the C structs declared in
``include/gdr.h`` and calls the exported functions.  Every step of the
computation runs in the HIP kernels of ``libgdr.so``; there is no fallback.
If the library has not been built, every call raises ``RuntimeError``.

Entry points (same names as the C ABI):

* ``gdr_chunk_fwd``   -- chunked forward over a sequence, returns (o, S_out)
* ``gdr_chunk_fwd_gated`` -- the same with the decay activation (and optionally
  the q/k L2 normalisation) computed in the kernel from raw inputs
* ``gdr_chunk_bwd``   -- gradients of the plain-erase forward (recomputes it)
* ``gdr_step_decode`` -- one token on a batch of states, in place, returns o
* ``gdr_raven_fwd``   -- the Raven routing slot memory (include/gdr_raven.h),
  returns (o, Sk_out, Sv_out)
* ``gdr_perm_fwd``    -- the delta rule with partial-permutation transitions
  (include/gdr_perm.h), returns (o, S_out)
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
GDR_DECAY_DIAG, GDR_DECAY_ROT2, GDR_DECAY_DIHEDRAL = 0, 1, 2
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


class GateArgs(ctypes.Structure):
    """Mirror of ``gdr_gate_args``."""
    _fields_ = [("decay_x", _vp), ("decay_a", _vp), ("qk_l2norm", _i32), ("reserved", _i32)]


class GateGrads(ctypes.Structure):
    """Mirror of ``gdr_gate_grads``."""
    _fields_ = [("grad_decay_x", _vp), ("grad_decay_a", _vp)]


class BwdArgs(ctypes.Structure):
    """Mirror of ``gdr_bwd_args``."""
    _fields_ = [
        ("B", _i32), ("T", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32), ("decay", _i32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("alpha", _vp), ("theta", _vp),
        ("beta", _vp), ("w", _vp), ("S0", _vp), ("grad_o", _vp), ("grad_S", _vp),
        ("grad_q", _vp), ("grad_k", _vp), ("grad_v", _vp), ("grad_alpha", _vp),
        ("grad_theta", _vp), ("grad_beta", _vp), ("grad_w", _vp), ("grad_S0", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


class StepArgs(ctypes.Structure):
    """Mirror of ``gdr_step_args``."""
    _fields_ = [
        ("N", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32),
        ("io_dtype", _i32), ("decay", _i32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("alpha", _vp), ("theta", _vp),
        ("beta", _vp), ("w", _vp), ("S", _vp), ("o", _vp),
    ]


class RavenArgs(ctypes.Structure):
    """Mirror of ``gdr_raven_args`` (include/gdr_raven.h)."""
    _fields_ = [
        ("B", _i32), ("T", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32),
        ("slots", _i32), ("topk", _i32), ("scale", ctypes.c_float),
        ("q", _vp), ("k", _vp), ("v", _vp), ("z", _vp), ("a", _vp),
        ("Sk0", _vp), ("Sv0", _vp), ("o", _vp), ("Sk_out", _vp), ("Sv_out", _vp),
    ]


class PermArgs(ctypes.Structure):
    """Mirror of ``gdr_perm_args`` (include/gdr_perm.h)."""
    _fields_ = [
        ("B", _i32), ("T", _i32), ("H", _i32), ("dk", _i32), ("dv", _i32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("src", _vp), ("beta", _vp), ("w", _vp),
        ("S0", _vp), ("o", _vp), ("S_out", _vp),
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
    lib.gdr_chunk_fwd_gated.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(GateArgs), _vp]
    lib.gdr_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdr_chunk_bwd.argtypes = [ctypes.POINTER(BwdArgs), _vp]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_chunk_bwd_noalloc.argtypes = [ctypes.POINTER(BwdArgs), _vp]
    lib.gdr_chunk_bwd_noalloc.restype = ctypes.c_int
    lib.gdr_chunk_bwd_gated.argtypes = [ctypes.POINTER(BwdArgs), ctypes.POINTER(GateArgs),
                                        ctypes.POINTER(GateGrads), _vp]
    lib.gdr_chunk_bwd_gated.restype = ctypes.c_int
    lib.gdr_chunk_bwd_gated_workspace.argtypes = [ctypes.POINTER(BwdArgs), ctypes.POINTER(GateArgs)]
    lib.gdr_chunk_bwd_gated_workspace.restype = ctypes.c_size_t
    lib.gdr_chunk_bwd_workspace.argtypes = [ctypes.POINTER(BwdArgs)]
    lib.gdr_chunk_bwd_workspace.restype = ctypes.c_size_t
    lib.gdr_chunk_fwd_workspace.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.gdr_chunk_fwd_workspace.restype = ctypes.c_size_t
    lib.gdr_step_decode.argtypes = [ctypes.POINTER(StepArgs), _vp]
    lib.gdr_step_decode.restype = ctypes.c_int
    lib.gdr_raven_fwd.argtypes = [ctypes.POINTER(RavenArgs), _vp]
    lib.gdr_raven_fwd.restype = ctypes.c_int
    lib.gdr_perm_fwd.argtypes = [ctypes.POINTER(PermArgs), _vp]
    lib.gdr_perm_fwd.restype = ctypes.c_int
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


def _expect(t, name: str, shape, dtype, required: bool = True):
    """Check one argument's presence, shape and dtype (before any pointer is taken,
    so that a wrong shape can never make a kernel read past an allocation)."""
    if t is None:
        if required:
            raise ValueError(f"gdr: {name} is required")
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"gdr: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"gdr: {name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"gdr: {name} must be contiguous")


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


def call_chunk_fwd_gated(args: FwdArgs, gate: GateArgs, stream=None) -> int:
    """Raw call with filled ``FwdArgs`` and ``GateArgs``; returns the status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_chunk_fwd_gated(ctypes.byref(args), ctypes.byref(gate), s)


def call_chunk_bwd(args: BwdArgs, stream=None) -> int:
    """Raw call with a filled ``BwdArgs``; returns the status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_chunk_bwd(ctypes.byref(args), s)


def call_chunk_bwd_gated(args: BwdArgs, gate: GateArgs, grads: GateGrads, stream=None) -> int:
    """Raw call with filled ``BwdArgs``, ``GateArgs`` and ``GateGrads``; returns the
    status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_chunk_bwd_gated(ctypes.byref(args), ctypes.byref(gate), ctypes.byref(grads), s)


def call_chunk_bwd_noalloc(args: BwdArgs, stream=None) -> int:
    """Raw call of the static-scratch backward (``args.workspace`` must be
    NULL); returns the status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_chunk_bwd_noalloc(ctypes.byref(args), s)


def call_raven_fwd(args: RavenArgs, stream=None) -> int:
    """Raw call with a filled ``RavenArgs``; returns the status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_raven_fwd(ctypes.byref(args), s)


def call_perm_fwd(args: PermArgs, stream=None) -> int:
    """Raw call with a filled ``PermArgs``; returns the status code."""
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_perm_fwd(ctypes.byref(args), s)


def call_step_decode(args: StepArgs, stream=None) -> int:
    lib = load_library()
    s = stream if isinstance(stream, ctypes.c_void_p) else (
        ctypes.c_void_p(0) if stream is None else _stream(stream))
    return lib.gdr_step_decode(ctypes.byref(args), s)


def _decay_kind(rot, reflections):
    if reflections and not rot:
        raise ValueError("gdr: reflection blocks need theta (2x2 blocks)")
    if reflections:
        return GDR_DECAY_DIHEDRAL
    return GDR_DECAY_ROT2 if rot else GDR_DECAY_DIAG


def gdr_chunk_fwd(q, k, v, alpha, w, beta=None, *, theta=None, S0=None, chunk=64,
                  o=None, S_out=None, return_state=True, beta_logit=None,
                  ub_down=None, ub_up=None, m_carry=None, reflections=False, stream=None):
    """Chunked gated delta-rule forward (see ``gdr_chunk_fwd`` in include/gdr.h).

    q, k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32, same dtype); alpha fp32
    [B,T,H,dk] (per-channel decay) or [B,T,H,dk/2] with ``theta`` (2x2
    rotation-decay blocks); beta, w fp32 [B,T,H].  ``reflections=True`` (with
    ``theta``) makes a block whose alpha is negative (sign bit set) the
    reflection of magnitude |alpha| (GDR_DECAY_DIHEDRAL).  Content-aware erase: pass
    ``beta_logit``, ``ub_down`` [H,r,dv], ``ub_up`` [H,r] instead of ``beta``.
    Returns (o [B,T,H,dv], S_out [B,H,dv,dk] fp32 or None).

    Every tensor's shape, dtype and contiguity is checked against (B, T, H,
    dk, dv) before anything reaches the library.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("gdr: q, k and v must be [B,T,H,d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    f32 = torch.float32
    _io(q)
    _expect(k, "k", (B, T, H, dk), io)
    _expect(v, "v", (B, T, H, dv), io)
    rot = theta is not None
    content = beta_logit is not None
    gshape = (B, T, H, dk // 2) if rot else (B, T, H, dk)
    if rot and dk % 2:
        raise ValueError("gdr: rotation-decay blocks need an even d_k")
    _expect(alpha, "alpha", gshape, f32)
    _expect(theta, "theta", gshape, f32, required=False)
    _expect(w, "w", (B, T, H), f32)
    if content:
        if beta is not None:
            raise ValueError("gdr: pass either beta or beta_logit, not both")
        if ub_down is None or ub_up is None or ub_up.dim() != 2:
            raise ValueError("gdr: the content-aware erase needs ub_down [H,r,dv] and ub_up [H,r]")
        r = ub_up.shape[-1]
        _expect(beta_logit, "beta_logit", (B, T, H), f32)
        _expect(ub_down, "ub_down", (H, r, dv), f32)
        _expect(ub_up, "ub_up", (H, r), f32)
        _expect(m_carry, "m_carry", (B, H, dv), f32, required=False)
    else:
        if ub_down is not None or ub_up is not None or m_carry is not None:
            raise ValueError("gdr: ub_down, ub_up and m_carry belong to the content-aware erase")
        _expect(beta, "beta", (B, T, H), f32)
    _expect(S0, "S0", (B, H, dv, dk), f32, required=False)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=io, device=q.device)
    _expect(o, "o", (B, T, H, dv), io)
    if S_out is None and return_state:
        S_out = torch.empty((B, H, dv, dk), dtype=f32, device=q.device)
    _expect(S_out, "S_out", (B, H, dv, dk), f32, required=False)
    a = FwdArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.chunk = B, T, H, dk, dv, chunk
    a.io_dtype = _io(q)
    a.decay = _decay_kind(rot, reflections)
    a.q, a.k, a.v, a.alpha, a.theta = map(_ptr, (q, k, v, alpha, theta))
    a.beta, a.w, a.beta_logit = map(_ptr, (beta, w, beta_logit))
    a.ub_down, a.ub_up, a.m_carry = map(_ptr, (ub_down, ub_up, m_carry))
    a.ub_rank = 0 if ub_up is None else int(ub_up.shape[-1])
    a.S0, a.o, a.S_out = _ptr(S0), _ptr(o), _ptr(S_out)
    a.workspace, a.workspace_bytes = None, 0
    _check(call_chunk_fwd(a, _stream(stream)))
    return o, S_out


def gdr_chunk_fwd_gated(q, k, v, decay_x, decay_a, w, beta, *, theta=None, qk_l2norm=True,
                        S0=None, chunk=64, o=None, S_out=None, return_state=True, stream=None):
    """Forward with the decay activation in the kernel (``gdr_chunk_fwd_gated`` in
    include/gdr.h): decay = exp(-decay_a[h] * softplus(decay_x)).

    q, k [B,T,H,dk], v [B,T,H,dv] bf16 (raw q, k when ``qk_l2norm``); decay_x
    bf16 [B,T,H,dk] (per-channel decay) or [B,T,H,dk/2] with ``theta`` fp32 of
    the same shape (2x2 rotation-decay blocks); decay_a fp32 [H]; beta, w fp32
    [B,T,H].  Returns (o [B,T,H,dv] bf16, S_out [B,H,dv,dk] fp32 or None).
    Shapes, dtypes and contiguity are checked first.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("gdr: q, k and v must be [B,T,H,d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bf, f32 = torch.bfloat16, torch.float32
    _expect(q, "q", (B, T, H, dk), bf)
    _expect(k, "k", (B, T, H, dk), bf)
    _expect(v, "v", (B, T, H, dv), bf)
    rot = theta is not None
    if rot and dk % 2:
        raise ValueError("gdr: rotation-decay blocks need an even d_k")
    gshape = (B, T, H, dk // 2) if rot else (B, T, H, dk)
    _expect(decay_x, "decay_x", gshape, bf)
    _expect(theta, "theta", gshape, f32, required=False)
    _expect(decay_a, "decay_a", (H,), f32)
    _expect(w, "w", (B, T, H), f32)
    _expect(beta, "beta", (B, T, H), f32)
    _expect(S0, "S0", (B, H, dv, dk), f32, required=False)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=bf, device=q.device)
    _expect(o, "o", (B, T, H, dv), bf)
    if S_out is None and return_state:
        S_out = torch.empty((B, H, dv, dk), dtype=f32, device=q.device)
    _expect(S_out, "S_out", (B, H, dv, dk), f32, required=False)
    a = FwdArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.chunk = B, T, H, dk, dv, chunk
    a.io_dtype = GDR_BF16
    a.decay = GDR_DECAY_ROT2 if rot else GDR_DECAY_DIAG
    a.q, a.k, a.v, a.theta = map(_ptr, (q, k, v, theta))
    a.alpha = None
    a.beta, a.w = _ptr(beta), _ptr(w)
    a.beta_logit = a.ub_down = a.ub_up = a.m_carry = None
    a.ub_rank = 0
    a.S0, a.o, a.S_out = _ptr(S0), _ptr(o), _ptr(S_out)
    a.workspace, a.workspace_bytes = None, 0
    g = GateArgs()
    g.decay_x, g.decay_a = _ptr(decay_x), _ptr(decay_a)
    g.qk_l2norm, g.reserved = int(bool(qk_l2norm)), 0
    _check(call_chunk_fwd_gated(a, g, _stream(stream)))
    return o, S_out


def gdr_chunk_bwd(q, k, v, alpha, w, beta, grad_o, *, theta=None, S0=None, grad_S=None,
                  need_grad_S0=True, workspace=None, stream=None):
    """Gradients of the plain-erase forward (``gdr_chunk_bwd`` in include/gdr.h).

    Inputs as ``gdr_chunk_fwd`` (bf16 q, k, v; fp32 alpha [and theta], beta,
    w; optional S0) plus grad_o [B,T,H,dv] bf16 and optional grad_S
    [B,H,dv,dk] fp32.  Returns a dict of fp32 tensors: q, k, v, alpha, beta,
    w, theta (rotation decay only) and S0 (when ``need_grad_S0``).  The
    workspace (``gdr_chunk_bwd_workspace`` bytes) is allocated here unless a
    large enough uint8 CUDA tensor is passed.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("gdr: q, k and v must be [B,T,H,d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bf, f32 = torch.bfloat16, torch.float32
    _expect(q, "q", (B, T, H, dk), bf)
    _expect(k, "k", (B, T, H, dk), bf)
    _expect(v, "v", (B, T, H, dv), bf)
    rot = theta is not None
    if rot and dk % 2:
        raise ValueError("gdr: rotation-decay blocks need an even d_k")
    gshape = (B, T, H, dk // 2) if rot else (B, T, H, dk)
    _expect(alpha, "alpha", gshape, f32)
    _expect(theta, "theta", gshape, f32, required=False)
    _expect(w, "w", (B, T, H), f32)
    _expect(beta, "beta", (B, T, H), f32)
    _expect(S0, "S0", (B, H, dv, dk), f32, required=False)
    _expect(grad_o, "grad_o", (B, T, H, dv), bf)
    _expect(grad_S, "grad_S", (B, H, dv, dk), f32, required=False)
    dev = q.device
    g = {"q": torch.empty((B, T, H, dk), dtype=f32, device=dev),
         "k": torch.empty((B, T, H, dk), dtype=f32, device=dev),
         "v": torch.empty((B, T, H, dv), dtype=f32, device=dev),
         "alpha": torch.empty(gshape, dtype=f32, device=dev),
         "beta": torch.empty((B, T, H), dtype=f32, device=dev),
         "w": torch.empty((B, T, H), dtype=f32, device=dev)}
    if rot:
        g["theta"] = torch.empty(gshape, dtype=f32, device=dev)
    if need_grad_S0:
        g["S0"] = torch.empty((B, H, dv, dk), dtype=f32, device=dev)
    a = BwdArgs()
    a.B, a.T, a.H, a.dk, a.dv = B, T, H, dk, dv
    a.decay = GDR_DECAY_ROT2 if rot else GDR_DECAY_DIAG
    a.q, a.k, a.v, a.alpha, a.theta = map(_ptr, (q, k, v, alpha, theta))
    a.beta, a.w, a.S0, a.grad_o, a.grad_S = map(_ptr, (beta, w, S0, grad_o, grad_S))
    a.grad_q, a.grad_k, a.grad_v = _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"])
    a.grad_alpha, a.grad_theta = _ptr(g["alpha"]), _ptr(g.get("theta"))
    a.grad_beta, a.grad_w, a.grad_S0 = _ptr(g["beta"]), _ptr(g["w"]), _ptr(g.get("S0"))
    need = load_library().gdr_chunk_bwd_workspace(ctypes.byref(a))
    if need == 0:
        _check(call_chunk_bwd(a, _stream(stream)))   # reports why the arguments are invalid
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"gdr: workspace must be a uint8 tensor of at least {need} bytes")
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(call_chunk_bwd(a, _stream(stream)))
    return g


def gdr_chunk_bwd_gated(q, k, v, decay_x, decay_a, w, beta, grad_o, *, theta=None,
                        qk_l2norm=True, S0=None, grad_S=None, need_grad_S0=True,
                        workspace=None, stream=None):
    """Gradients of the gated forward (``gdr_chunk_bwd_gated`` in include/gdr.h).

    Inputs as ``gdr_chunk_fwd_gated`` (bf16 q, k, v, raw q and k when
    ``qk_l2norm``; bf16 decay_x [B,T,H,dk] or [B,T,H,dk/2] with ``theta``; fp32
    decay_a [H], beta, w) plus grad_o [B,T,H,dv] bf16 and optional grad_S
    [B,H,dv,dk] fp32.  Returns a dict of fp32 tensors: q, k (of the raw
    inputs), v, x (decay_x), a (decay_a), beta, w, theta (rotation decay only)
    and S0 (when ``need_grad_S0``).  The workspace
    (``gdr_chunk_bwd_gated_workspace`` bytes) is allocated here unless a large
    enough uint8 CUDA tensor is passed.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("gdr: q, k and v must be [B,T,H,d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bf, f32 = torch.bfloat16, torch.float32
    _expect(q, "q", (B, T, H, dk), bf)
    _expect(k, "k", (B, T, H, dk), bf)
    _expect(v, "v", (B, T, H, dv), bf)
    rot = theta is not None
    if rot and dk % 2:
        raise ValueError("gdr: rotation-decay blocks need an even d_k")
    gshape = (B, T, H, dk // 2) if rot else (B, T, H, dk)
    _expect(decay_x, "decay_x", gshape, bf)
    _expect(theta, "theta", gshape, f32, required=False)
    _expect(decay_a, "decay_a", (H,), f32)
    _expect(w, "w", (B, T, H), f32)
    _expect(beta, "beta", (B, T, H), f32)
    _expect(S0, "S0", (B, H, dv, dk), f32, required=False)
    _expect(grad_o, "grad_o", (B, T, H, dv), bf)
    _expect(grad_S, "grad_S", (B, H, dv, dk), f32, required=False)
    dev = q.device
    g = {"q": torch.empty((B, T, H, dk), dtype=f32, device=dev),
         "k": torch.empty((B, T, H, dk), dtype=f32, device=dev),
         "v": torch.empty((B, T, H, dv), dtype=f32, device=dev),
         "x": torch.empty(gshape, dtype=f32, device=dev),
         "a": torch.empty((H,), dtype=f32, device=dev),
         "beta": torch.empty((B, T, H), dtype=f32, device=dev),
         "w": torch.empty((B, T, H), dtype=f32, device=dev)}
    if rot:
        g["theta"] = torch.empty(gshape, dtype=f32, device=dev)
    if need_grad_S0:
        g["S0"] = torch.empty((B, H, dv, dk), dtype=f32, device=dev)
    a = BwdArgs()
    a.B, a.T, a.H, a.dk, a.dv = B, T, H, dk, dv
    a.decay = GDR_DECAY_ROT2 if rot else GDR_DECAY_DIAG
    a.q, a.k, a.v, a.theta = map(_ptr, (q, k, v, theta))
    a.alpha, a.grad_alpha = None, None
    a.beta, a.w, a.S0, a.grad_o, a.grad_S = map(_ptr, (beta, w, S0, grad_o, grad_S))
    a.grad_q, a.grad_k, a.grad_v = _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"])
    a.grad_theta = _ptr(g.get("theta"))
    a.grad_beta, a.grad_w, a.grad_S0 = _ptr(g["beta"]), _ptr(g["w"]), _ptr(g.get("S0"))
    ga = GateArgs()
    ga.decay_x, ga.decay_a = _ptr(decay_x), _ptr(decay_a)
    ga.qk_l2norm, ga.reserved = int(bool(qk_l2norm)), 0
    gg = GateGrads()
    gg.grad_decay_x, gg.grad_decay_a = _ptr(g["x"]), _ptr(g["a"])
    need = load_library().gdr_chunk_bwd_gated_workspace(ctypes.byref(a), ctypes.byref(ga))
    if need == 0:
        _check(call_chunk_bwd_gated(a, ga, gg, _stream(stream)))   # reports why the arguments are invalid
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"gdr: workspace must be a uint8 tensor of at least {need} bytes")
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(call_chunk_bwd_gated(a, ga, gg, _stream(stream)))
    return g


def gdr_step_decode(S, q, k, v, alpha, beta, w, *, theta=None, o=None, reflections=False,
                    stream=None):
    """One token on N states in place (see ``gdr_step_decode`` in include/gdr.h).

    S [N,H,dv,dk] fp32 (overwritten), q,k [N,H,dk], v [N,H,dv], alpha [N,H,dk]
    or gamma [N,H,dk/2] with theta, beta, w [N,H]; ``reflections`` as in
    ``gdr_chunk_fwd``.  Returns o [N,H,dv].
    Every tensor's shape, dtype and contiguity is checked first.
    """
    import torch
    if S.dim() != 4:
        raise ValueError("gdr: S must be [N,H,dv,dk]")
    N, H, dv, dk = S.shape
    f32 = torch.float32
    io = q.dtype
    _io(q)
    _expect(S, "S", (N, H, dv, dk), f32)
    _expect(q, "q", (N, H, dk), io)
    _expect(k, "k", (N, H, dk), io)
    _expect(v, "v", (N, H, dv), io)
    rot = theta is not None
    gshape = (N, H, dk // 2) if rot else (N, H, dk)
    _expect(alpha, "alpha", gshape, f32)
    _expect(theta, "theta", gshape, f32, required=False)
    _expect(beta, "beta", (N, H), f32)
    _expect(w, "w", (N, H), f32)
    if o is None:
        o = torch.empty((N, H, dv), dtype=io, device=q.device)
    _expect(o, "o", (N, H, dv), io)
    a = StepArgs()
    a.N, a.H, a.dk, a.dv = N, H, dk, dv
    a.io_dtype = _io(q)
    a.decay = _decay_kind(rot, reflections)
    a.q, a.k, a.v, a.alpha, a.theta = map(_ptr, (q, k, v, alpha, theta))
    a.beta, a.w, a.S, a.o = map(_ptr, (beta, w, S, o))
    _check(call_step_decode(a, _stream(stream)))
    return o


def gdr_raven_fwd(q, k, v, z, a, *, topk, scale=None, Sk0=None, Sv0=None, o=None,
                  Sk_out=None, Sv_out=None, return_state=True, stream=None):
    """Raven routing slot-memory forward (see ``gdr_raven_fwd`` in
    include/gdr_raven.h).

    q, k [B,T,H,dk], v [B,T,H,dv], router logits z [B,T,H,slots], all bf16;
    decay rate a fp32 [B,T,H] (finite, <= 0); ``topk`` slots written per token;
    ``scale`` of the read-out logits (default 1/sqrt(dk)); start slots Sk0
    [B,H,slots,dk], Sv0 [B,H,slots,dv] fp32 or None (zero).  Returns
    (o [B,T,H,dv] bf16, Sk_out, Sv_out) -- the states None unless
    ``return_state`` or given.
    """
    import math
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or z.dim() != 4:
        raise ValueError("gdr: q, k, v and z must be [B,T,H,*]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    M = z.shape[-1]
    bf, f32 = torch.bfloat16, torch.float32
    _expect(q, "q", (B, T, H, dk), bf)
    _expect(k, "k", (B, T, H, dk), bf)
    _expect(v, "v", (B, T, H, dv), bf)
    _expect(z, "z", (B, T, H, M), bf)
    _expect(a, "a", (B, T, H), f32)
    _expect(Sk0, "Sk0", (B, H, M, dk), f32, required=False)
    _expect(Sv0, "Sv0", (B, H, M, dv), f32, required=False)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=bf, device=q.device)
    _expect(o, "o", (B, T, H, dv), bf)
    if return_state:
        if Sk_out is None:
            Sk_out = torch.empty((B, H, M, dk), dtype=f32, device=q.device)
        if Sv_out is None:
            Sv_out = torch.empty((B, H, M, dv), dtype=f32, device=q.device)
    _expect(Sk_out, "Sk_out", (B, H, M, dk), f32, required=False)
    _expect(Sv_out, "Sv_out", (B, H, M, dv), f32, required=False)
    r = RavenArgs()
    r.B, r.T, r.H, r.dk, r.dv, r.slots, r.topk = B, T, H, dk, dv, M, int(topk)
    r.scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    r.q, r.k, r.v, r.z, r.a = map(_ptr, (q, k, v, z, a))
    r.Sk0, r.Sv0, r.o, r.Sk_out, r.Sv_out = map(_ptr, (Sk0, Sv0, o, Sk_out, Sv_out))
    _check(call_raven_fwd(r, _stream(stream)))
    return o, Sk_out, Sv_out


def gdr_perm_fwd(q, k, v, w, src, beta, *, S0=None, o=None, S_out=None, return_state=True,
                 stream=None):
    """Delta rule with partial-permutation transitions (see ``gdr_perm_fwd`` in
    include/gdr_perm.h): column j of S D_t is column src[j] of S (zero for a
    value outside [0, dk)).

    q, k [B,T,H,dk], v [B,T,H,dv] bf16; w, beta fp32 [B,T,H]; src int16
    [B,T,H,dk]; S0 fp32 [B,H,dv,dk] or None.  Returns (o [B,T,H,dv] bf16, S_out).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("gdr: q, k and v must be [B,T,H,d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bf, f32 = torch.bfloat16, torch.float32
    _expect(q, "q", (B, T, H, dk), bf)
    _expect(k, "k", (B, T, H, dk), bf)
    _expect(v, "v", (B, T, H, dv), bf)
    _expect(src, "src", (B, T, H, dk), torch.int16)
    _expect(w, "w", (B, T, H), f32)
    _expect(beta, "beta", (B, T, H), f32)
    _expect(S0, "S0", (B, H, dv, dk), f32, required=False)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=bf, device=q.device)
    _expect(o, "o", (B, T, H, dv), bf)
    if S_out is None and return_state:
        S_out = torch.empty((B, H, dv, dk), dtype=f32, device=q.device)
    _expect(S_out, "S_out", (B, H, dv, dk), f32, required=False)
    a = PermArgs()
    a.B, a.T, a.H, a.dk, a.dv = B, T, H, dk, dv
    a.q, a.k, a.v, a.src, a.beta, a.w = map(_ptr, (q, k, v, src, beta, w))
    a.S0, a.o, a.S_out = _ptr(S0), _ptr(o), _ptr(S_out)
    _check(call_perm_fwd(a, _stream(stream)))
    return o, S_out
