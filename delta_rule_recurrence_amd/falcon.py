"""Thin Python binding of libfalcon (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/falcon.h``.  Tensors must be
contiguous device tensors; outputs are allocated with torch when not given.
There is no CPU fallback: without the built library, or without a GPU,
these functions raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfalcon.so")

VARIANTS = {"falcon1": 1, "falcon1a": 2, "falcon2": 3, "falcon2a": 4}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}

FALCON_OK = 0


class FalconProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("eps", ctypes.c_float), ("eps_gamma", ctypes.c_float)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "falcon_abi_version": (ctypes.c_int32, []),
    "falcon_set_wait_limit": (ctypes.c_int32, [ctypes.c_int32]),
    "falcon_set_f1_launch_form": (ctypes.c_int32, [ctypes.c_int32]),
    "falcon_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "falcon_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FalconProblem), ctypes.c_int32]),
    "falcon_fwd_recurrent": (ctypes.c_int32, [ctypes.POINTER(FalconProblem), _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, _P]),
    "falcon_fwd_chunked": (ctypes.c_int32, [ctypes.POINTER(FalconProblem), _P, _P, _P, _P, _P, _P,
                                            _P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "falcon_fwd_chunked_noalloc": (ctypes.c_int32, [ctypes.POINTER(FalconProblem), _P, _P, _P, _P, _P,
                                                    _P, _P, _P, _P, ctypes.c_int32, _P]),
    "falcon_decode_step": (ctypes.c_int32, [ctypes.POINTER(FalconProblem), _P, _P, _P, _P, _P,
                                            _P, _P, _P, _P]),
    "falcon_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FalconProblem)]),
    "falcon_bwd_chunked": (ctypes.c_int32, [ctypes.POINTER(FalconProblem)] + [_P] * 17
                           + [ctypes.c_size_t, _P]),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfalcon.so (built by ``delta_rule_recurrence_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m delta_rule_recurrence_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class FalconError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(falcon_status_string(status))


def falcon_status_string(status: int) -> str:
    return load_library().falcon_status_string(int(status)).decode()


def falcon_abi_version() -> int:
    return int(load_library().falcon_abi_version())


def falcon_set_wait_limit(polls: int) -> int:
    """Polls a bounded wait between waves makes before giving up; returns the
    previous limit (see ``falcon_set_wait_limit`` in falcon.h)."""
    prev = int(load_library().falcon_set_wait_limit(int(polls)))
    if prev < 0:
        raise ValueError("the wait limit must be >= 0")
    return prev


F1_ONE_LAUNCH = 0
F1_TWO_LAUNCH = 1


def falcon_set_f1_launch_form(form: int) -> int:
    """How the Falcon-1 bf16 chunked fast path runs: F1_ONE_LAUNCH (default)
    or F1_TWO_LAUNCH; returns the previous form (see
    ``falcon_set_f1_launch_form`` in falcon.h)."""
    prev = int(load_library().falcon_set_f1_launch_form(int(form)))
    if prev < 0:
        raise ValueError("form must be F1_ONE_LAUNCH or F1_TWO_LAUNCH")
    return prev


def make_problem(B, H, T, dk, dv, *, variant="falcon1", io_dtype=torch.bfloat16, eps=1e-6,
                 eps_gamma=1e-6) -> FalconProblem:
    return FalconProblem(B, H, T, dk, dv, VARIANTS[variant], DTYPES[io_dtype], eps, eps_gamma)


def falcon_workspace_bytes(problem: FalconProblem, C: int) -> int:
    return int(load_library().falcon_workspace_bytes(ctypes.byref(problem), int(C)))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _io_dtype(t: torch.Tensor, name: str) -> torch.dtype:
    if t.dtype not in DTYPES:
        raise ValueError(f"{name}: io dtype must be float32 or bfloat16, got {t.dtype}")
    return t.dtype


def _expect(t, name, shape, dtypes, device, *, optional=False):
    """Shape, dtype, device and layout check of one argument, done before any
    pointer crosses the C ABI (which cannot see shapes)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        names = " or ".join(str(d) for d in dtypes)
        raise ValueError(f"{name}: expected dtype {names}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def _expect_bytes(t, name, need, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    have = t.numel() * t.element_size()
    if have < need:
        raise ValueError(f"{name}: {have} bytes, at least {need} needed")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int):
    if status != FALCON_OK:
        raise FalconError(status)


def _forward_setup(phi_k, phi_q, v, beta, lam, variant, S0, k_prev, o, S_T, return_state):
    """Checks every forward argument against the problem that phi_k and v
    define, and allocates the outputs that were not given."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if not isinstance(phi_k, torch.Tensor) or phi_k.dim() != 4:
        raise ValueError("phi_k: expected a [B, H, T, dk] tensor")
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v: expected a [B, H, T, dv] tensor")
    B, H, T, dk = phi_k.shape
    dv = v.shape[-1]
    io = _io_dtype(v, "v")
    dev = v.device
    f32 = (torch.float32,)
    per_col = variant in ("falcon2", "falcon2a")
    _expect(phi_k, "phi_k", (B, H, T, dk), (io,), dev)
    _expect(phi_q, "phi_q", (B, H, T, dk), (io,), dev)
    _expect(v, "v", (B, H, T, dv), (io,), dev)
    _expect(beta, "beta", (B, H, T, dv) if per_col else (B, H, T), f32, dev)
    _expect(lam, "lam", (B, H, T), f32, dev)
    _expect(S0, "S0", (B, H, dk, dv), f32, dev, optional=True)
    _expect(k_prev, "k_prev", (B, H, dk), (io,), dev, optional=True)
    _expect(o, "o", (B, H, T, dv), (io,), dev, optional=True)
    _expect(S_T, "S_T", (B, H, dk, dv), f32, dev, optional=True)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=io, device=dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    return B, H, T, dk, dv, o, S_T


def falcon_fwd_recurrent(phi_k, phi_q, v, beta, lam, *, variant="falcon1", S0=None, k_prev=None,
                         eps=1e-6, eps_gamma=1e-6, o=None, S_T=None, return_state=True,
                         stream=None):
    """Recurrent form; returns ``(o, S_T)``."""
    B, H, T, dk, dv, o, S_T = _forward_setup(phi_k, phi_q, v, beta, lam, variant, S0, k_prev, o,
                                             S_T, return_state)
    p = make_problem(B, H, T, dk, dv, variant=variant, io_dtype=v.dtype, eps=eps, eps_gamma=eps_gamma)
    _check(load_library().falcon_fwd_recurrent(
        ctypes.byref(p), _ptr(phi_k), _ptr(phi_q), _ptr(v), _ptr(beta), _ptr(lam), _ptr(S0),
        _ptr(k_prev), _ptr(o), _ptr(S_T), _stream(stream)))
    return o, S_T


def falcon_fwd_chunked(phi_k, phi_q, v, beta, lam, *, variant="falcon1", C=64, S0=None,
                       k_prev=None, eps=1e-6, eps_gamma=1e-6, o=None, S_T=None, workspace=None,
                       return_state=True, stream=None):
    """Chunk-parallel form; returns ``(o, S_T)``."""
    B, H, T, dk, dv, o, S_T = _forward_setup(phi_k, phi_q, v, beta, lam, variant, S0, k_prev, o,
                                             S_T, return_state)
    p = make_problem(B, H, T, dk, dv, variant=variant, io_dtype=v.dtype, eps=eps, eps_gamma=eps_gamma)
    need = falcon_workspace_bytes(p, C)
    if need == ctypes.c_size_t(-1).value:
        raise FalconError(-2 if C in (16, 32, 64) else -4)
    _expect_bytes(workspace, "workspace", need, v.device)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().falcon_fwd_chunked(
        ctypes.byref(p), _ptr(phi_k), _ptr(phi_q), _ptr(v), _ptr(beta), _ptr(lam), _ptr(S0),
        _ptr(k_prev), _ptr(o), _ptr(S_T), int(C), _ptr(workspace), wbytes, _stream(stream)))
    return o, S_T


def falcon_fwd_chunked_noalloc(phi_k, phi_q, v, beta, lam, o, *, variant="falcon1", C=64, S0=None,
                               k_prev=None, eps=1e-6, eps_gamma=1e-6, S_T=None, stream=None):
    """Chunk-parallel form without any allocation: the caller passes ``o``
    (and ``S_T``, or None to skip the final state); scratch comes from the
    library's static device buffer.  Returns ``(o, S_T)``."""
    if o is None:
        raise ValueError("o is required: this entry point allocates nothing")
    B, H, T, dk, dv, o, S_T = _forward_setup(phi_k, phi_q, v, beta, lam, variant, S0, k_prev, o,
                                             S_T, False)
    p = make_problem(B, H, T, dk, dv, variant=variant, io_dtype=v.dtype, eps=eps, eps_gamma=eps_gamma)
    _check(load_library().falcon_fwd_chunked_noalloc(
        ctypes.byref(p), _ptr(phi_k), _ptr(phi_q), _ptr(v), _ptr(beta), _ptr(lam), _ptr(S0),
        _ptr(k_prev), _ptr(o), _ptr(S_T), int(C), _stream(stream)))
    return o, S_T


def falcon_decode_step(phi_k_prev, phi_q, v, beta, lam, S, *, variant="falcon1", is_first=None,
                       eps=1e-6, eps_gamma=1e-6, o=None, stream=None):
    """One decode token; updates ``S`` in place and returns ``o``."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if not isinstance(phi_k_prev, torch.Tensor) or phi_k_prev.dim() != 3:
        raise ValueError("phi_k_prev: expected a [B, H, dk] tensor")
    if not isinstance(v, torch.Tensor) or v.dim() != 3:
        raise ValueError("v: expected a [B, H, dv] tensor")
    B, H, dk = phi_k_prev.shape
    dv = v.shape[-1]
    io = _io_dtype(v, "v")
    dev = v.device
    f32 = (torch.float32,)
    per_col = variant in ("falcon2", "falcon2a")
    _expect(phi_k_prev, "phi_k_prev", (B, H, dk), (io,), dev)
    _expect(phi_q, "phi_q", (B, H, dk), (io,), dev)
    _expect(v, "v", (B, H, dv), (io,), dev)
    _expect(beta, "beta", (B, H, dv) if per_col else (B, H), f32, dev)
    _expect(lam, "lam", (B, H), f32, dev)
    _expect(S, "S", (B, H, dk, dv), f32, dev)
    _expect(is_first, "is_first", (B,), (torch.uint8, torch.bool), dev, optional=True)
    _expect(o, "o", (B, H, dv), (io,), dev, optional=True)
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    p = make_problem(B, H, 1, dk, dv, variant=variant, io_dtype=v.dtype, eps=eps, eps_gamma=eps_gamma)
    _check(load_library().falcon_decode_step(
        ctypes.byref(p), _ptr(phi_k_prev), _ptr(phi_q), _ptr(v), _ptr(beta), _ptr(lam), _ptr(S),
        _ptr(is_first), _ptr(o), _stream(stream)))
    return o


def falcon_bwd_workspace_bytes(problem: FalconProblem) -> int:
    return int(load_library().falcon_bwd_workspace_bytes(ctypes.byref(problem)))


def falcon_bwd_chunked(phi_k, phi_q, v, beta, lam, dO, *, S0=None, k_prev=None, dS_T=None,
                       eps=1e-6, eps_gamma=1e-6, grads=None, workspace=None, stream=None):
    """Gradients of ``<dO, o> + <dS_T, S_T>`` for the Falcon-1 forward.

    Returns a dict with float32 tensors dphi_k, dphi_q, dv, dbeta, dlam, dS0
    and dk_prev (None when ``k_prev`` is None).  ``grads`` may hold
    preallocated outputs under the same names.
    """
    B, H, T, dk, dv_, _, _ = _forward_setup(phi_k, phi_q, v, beta, lam, "falcon1", S0, k_prev,
                                            None, None, False)
    dev = v.device
    f32 = torch.float32
    _expect(dO, "dO", (B, H, T, dv_), (v.dtype,), dev)
    _expect(dS_T, "dS_T", (B, H, dk, dv_), (f32,), dev, optional=True)
    shapes = {"dphi_k": (B, H, T, dk), "dphi_q": (B, H, T, dk), "dv": (B, H, T, dv_),
              "dbeta": (B, H, T), "dlam": (B, H, T), "dS0": (B, H, dk, dv_), "dk_prev": (B, H, dk)}
    g = dict(grads or {})
    unknown = set(g) - set(shapes)
    if unknown:
        raise ValueError(f"grads: unknown names {sorted(unknown)}")
    for name, shape in shapes.items():
        _expect(g.get(name), f"grads[{name!r}]", shape, (f32,), dev, optional=True)
        if g.get(name) is None and (name != "dk_prev" or k_prev is not None):
            g[name] = torch.empty(shape, dtype=f32, device=dev)
    if k_prev is None:
        g["dk_prev"] = None
    p = make_problem(B, H, T, dk, dv_, variant="falcon1", io_dtype=v.dtype, eps=eps,
                     eps_gamma=eps_gamma)
    need = falcon_bwd_workspace_bytes(p)
    if need == ctypes.c_size_t(-1).value:
        raise FalconError(-2)
    _expect_bytes(workspace, "workspace", need, dev)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().falcon_bwd_chunked(
        ctypes.byref(p), _ptr(phi_k), _ptr(phi_q), _ptr(v), _ptr(beta), _ptr(lam), _ptr(S0),
        _ptr(k_prev), _ptr(dO), _ptr(dS_T), _ptr(g["dphi_k"]), _ptr(g["dphi_q"]), _ptr(g["dv"]),
        _ptr(g["dbeta"]), _ptr(g["dlam"]), _ptr(g["dS0"]), _ptr(g["dk_prev"]), _ptr(workspace),
        wbytes, _stream(stream)))
    return g
