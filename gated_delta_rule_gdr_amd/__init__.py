"""gated_delta_rule_gdr_amd -- Gated Delta Rule-2 layer on MI355X (gfx950).

Thin Python binding over the C ABI of ``libgdr2.so`` (see ``include/gdr2.h``).  It only marshals
arguments: every step of the computation runs in the library's HIP kernels.  PyTorch provides
device memory and the current HIP stream.  There is no fallback: if the library is missing or
fails to load, every call raises.

Entry points (same names as the C ABI):
  gdr2_fwd_chunked(q, k, v, log_alpha, b, w, S0=None, want_final_state=True) -> (o, S_T, fwd_ws)
  gdr2_bwd_chunked(q, k, v, log_alpha, b, w, dO, fwd_ws, dS_T=None, want_dS0=True) -> grads
  gdr2_fwd_infer(q, k, v, log_alpha, b, w, S0=None, want_final_state=True) -> (o, S_T)
  gdr2_bwd_chunked_recompute(q, k, v, log_alpha, b, w, dO, S0=None, dS_T=None) -> grads
  gdr2_decode_step(q, k, v, log_alpha, b, w, S_in=None, S_out=None)
  gdr2_out_gate_fwd(o, g, weight, eps) / gdr2_out_gate_bwd(o, g, weight, dy, eps)
Each of b, w and log_alpha may be channel-wise ([..., d]) or a scalar per head (the token shape of
q without its channel axis); the gate-shape bits passed to the *_ex entry points follow from the
shapes, and the gradients come back in the shape of their gate.  ``prologue=Prologue(c, eps)``
(forward, backward and decode) makes q, k, log_alpha, b and w pre-activations: the kernels apply
the L2 normalisation of q and k, the sigmoid gates and log alpha = -c * softplus(a) themselves,
and the backward returns gradients with respect to the pre-activations.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["gdr2_fwd_chunked", "gdr2_bwd_chunked", "gdr2_decode_step", "gdr2_fwd_factors",
           "gdr2_fwd_infer", "gdr2_bwd_chunked_recompute", "fwd_infer_workspace_bytes",
           "gdr2_fwd_infer_noalloc", "fwd_infer_noalloc_max_bytes",
           "bwd_recompute_workspace_bytes",
           "gdr2_fwd_carry", "gdr2_bwd_state", "gdr2_bwd_grads", "fwd_workspace_bytes",
           "bwd_workspace_bytes", "library_path", "load_library", "Gdr2Error", "CHUNK", "gate_bits",
           "ERASE_SCALAR", "WRITE_SCALAR", "DECAY_SCALAR", "gdr2_out_gate_fwd", "gdr2_out_gate_bwd",
           "Prologue"]

CHUNK = 64
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgdr2.so")
_lib = None

_STATUS = {0: "ok", 1: "GDR2_E_NULL", 2: "GDR2_E_SHAPE", 3: "GDR2_E_DTYPE",
           4: "GDR2_E_UNSUPPORTED", 5: "GDR2_E_ALIGN", 6: "GDR2_E_ALIAS", 7: "GDR2_E_WORKSPACE",
           8: "GDR2_E_HIP", 9: "GDR2_E_VALUE", 10: "GDR2_E_TOO_LARGE"}
_DT = {torch.float32: 0, torch.bfloat16: 1}


class Prologue(ctypes.Structure):
    """gdr2_prologue: decay_scale c (log alpha = -c * softplus(a)) and norm_eps (q, k are divided
    by sqrt(sum of squares + norm_eps))."""
    _fields_ = [("decay_scale", ctypes.c_float), ("norm_eps", ctypes.c_float)]

    def __init__(self, decay_scale=1.0, norm_eps=1e-6):
        super().__init__(float(decay_scale), float(norm_eps))


def _pro(prologue):
    if prologue is None:
        return None
    if not isinstance(prologue, Prologue):
        raise TypeError("prologue must be a Prologue or None")
    return ctypes.byref(prologue)


class Gdr2Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdr2.so (built in-tree by ``gated_delta_rule_gdr_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                           "(run python gated_delta_rule_gdr_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    I64, P, SZ = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.gdr2_fwd_chunked.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 10 + [SZ, P]
    lib.gdr2_fwd_chunked.restype = ctypes.c_int
    lib.gdr2_bwd_chunked.argtypes = ([I64] * 5 + [ctypes.c_int] + [P] * 7 + [SZ] + [P] * 10
                                     + [SZ, P])
    lib.gdr2_bwd_chunked.restype = ctypes.c_int
    lib.gdr2_fwd_factors.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 7 + [SZ, P]
    lib.gdr2_fwd_factors.restype = ctypes.c_int
    lib.gdr2_fwd_carry.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 4 + [SZ, P]
    lib.gdr2_fwd_carry.restype = ctypes.c_int
    lib.gdr2_bwd_state.argtypes = [I64] * 5 + [ctypes.c_int, P, SZ, P, P, P, P, SZ, P]
    lib.gdr2_bwd_state.restype = ctypes.c_int
    lib.gdr2_bwd_grads.argtypes = ([I64] * 5 + [ctypes.c_int] + [P] * 7 + [SZ] + [P] * 8
                                   + [SZ, P])
    lib.gdr2_bwd_grads.restype = ctypes.c_int
    lib.gdr2_fwd_infer_ex.argtypes = [I64] * 5 + [ctypes.c_int, ctypes.c_uint, P] + [P] * 10 + [SZ, P]
    lib.gdr2_fwd_infer_ex.restype = ctypes.c_int
    lib.gdr2_fwd_infer.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 10 + [SZ, P]
    lib.gdr2_fwd_infer.restype = ctypes.c_int
    lib.gdr2_bwd_chunked_recompute.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 17 + [SZ, P]
    lib.gdr2_bwd_chunked_recompute.restype = ctypes.c_int
    lib.gdr2_fwd_infer_noalloc_ex.argtypes = [I64] * 5 + [ctypes.c_int, ctypes.c_uint, P] + [P] * 10
    lib.gdr2_fwd_infer_noalloc_ex.restype = ctypes.c_int
    lib.gdr2_fwd_infer_noalloc_max_bytes.argtypes = []
    lib.gdr2_fwd_infer_noalloc_max_bytes.restype = SZ
    lib.gdr2_fwd_infer_workspace_bytes.argtypes = [I64] * 5 + [ctypes.c_int]
    lib.gdr2_fwd_infer_workspace_bytes.restype = SZ
    lib.gdr2_bwd_chunked_recompute_ex.argtypes = ([I64] * 5 + [ctypes.c_int, ctypes.c_uint, P]
                                                  + [P] * 17 + [SZ, P])
    lib.gdr2_bwd_chunked_recompute_ex.restype = ctypes.c_int
    lib.gdr2_bwd_recompute_workspace_bytes.argtypes = [I64] * 5 + [ctypes.c_int]
    lib.gdr2_bwd_recompute_workspace_bytes.restype = SZ
    lib.gdr2_decode_step.argtypes = [I64] * 4 + [ctypes.c_int] + [P] * 10
    lib.gdr2_decode_step.restype = ctypes.c_int
    U = ctypes.c_uint
    lib.gdr2_fwd_chunked_ex.argtypes = [I64] * 5 + [ctypes.c_int, U, P] + [P] * 10 + [SZ, P]
    lib.gdr2_fwd_chunked_ex.restype = ctypes.c_int
    lib.gdr2_bwd_chunked_ex.argtypes = ([I64] * 5 + [ctypes.c_int, U, P] + [P] * 7 + [SZ] + [P] * 10
                                        + [SZ, P])
    lib.gdr2_bwd_chunked_ex.restype = ctypes.c_int
    lib.gdr2_fwd_factors_ex.argtypes = [I64] * 5 + [ctypes.c_int, U, P] + [P] * 7 + [SZ, P]
    lib.gdr2_fwd_factors_ex.restype = ctypes.c_int
    lib.gdr2_bwd_grads_ex.argtypes = ([I64] * 5 + [ctypes.c_int, U, P] + [P] * 7 + [SZ] + [P] * 8
                                      + [SZ, P])
    lib.gdr2_bwd_grads_ex.restype = ctypes.c_int
    lib.gdr2_decode_step_ex.argtypes = [I64] * 4 + [ctypes.c_int, U, P] + [P] * 10
    lib.gdr2_decode_step_ex.restype = ctypes.c_int
    F = ctypes.c_float
    lib.gdr2_out_gate_fwd.argtypes = [I64, I64, ctypes.c_int, P, P, P, F, P, P]
    lib.gdr2_out_gate_fwd.restype = ctypes.c_int
    lib.gdr2_out_gate_bwd.argtypes = [I64, I64, ctypes.c_int, P, P, P, F, P, P, P, P, P, SZ, P]
    lib.gdr2_out_gate_bwd.restype = ctypes.c_int
    lib.gdr2_out_gate_bwd_workspace_bytes.argtypes = [I64, I64]
    lib.gdr2_out_gate_bwd_workspace_bytes.restype = SZ
    lib.gdr2_fwd_workspace_bytes.argtypes = [I64] * 5 + [ctypes.c_int]
    lib.gdr2_fwd_workspace_bytes.restype = SZ
    lib.gdr2_bwd_workspace_bytes.argtypes = [I64] * 5 + [ctypes.c_int]
    lib.gdr2_bwd_workspace_bytes.restype = SZ
    lib.gdr2_num_chunks.argtypes = [I64]
    lib.gdr2_num_chunks.restype = I64
    lib.gdr2_status_string.argtypes = [ctypes.c_int]
    lib.gdr2_status_string.restype = ctypes.c_char_p
    lib.gdr2_abi_version.argtypes = []
    lib.gdr2_abi_version.restype = ctypes.c_int
    lib.gdr2_dtype_size.argtypes = [ctypes.c_int]
    lib.gdr2_dtype_size.restype = SZ
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _run(fn_name, dev, fn, *args):
    """Call a C entry point with dev current and its current stream appended; raise on error."""
    with torch.cuda.device(dev):
        st = fn(*args, _stream(dev))
    _check(fn_name, st)


def _check(fn, st):
    if st != 0:
        raise Gdr2Error(fn, st)


def _shapes(q, v):
    B, T, H, dk = q.shape
    return B, T, H, dk, v.shape[-1]


def _dtype(q):
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return _DT[q.dtype]


# gate-shape bits (gdr2_gates in include/gdr2.h)
ERASE_SCALAR, WRITE_SCALAR, DECAY_SCALAR = 1, 2, 4


def gate_bits(q, log_alpha, b, w):
    """Gate shapes from the tensor shapes: a gate with the token shape of q without its channel
    axis ([B, T, H], or [N, H] for decode) is a scalar per head; otherwise it must have the full
    channel shape."""
    bits = 0
    for t, bit, name in ((b, ERASE_SCALAR, "b"), (w, WRITE_SCALAR, "w"), (log_alpha, DECAY_SCALAR, "log_alpha")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if tuple(t.shape) == tuple(q.shape[:-1]):
            bits |= bit
        elif t.dim() != q.dim() or tuple(t.shape[:-1]) != tuple(q.shape[:-1]):
            raise ValueError(f"{name} has shape {tuple(t.shape)}; expected the token shape "
                             f"{tuple(q.shape[:-1])} (scalar per head) or that plus a channel axis")
    return bits


# Tensor checks.  The C ABI receives raw pointers and cannot see shapes or dtypes, so a tensor of
# the wrong shape or dtype would be read out of bounds: every tensor is checked against the layout
# include/gdr2.h gives before any call.  Shape and dtype come first and the device last, so that a
# consistent set of host tensors fails only on the device check.
def _need(name, t, shape, dtype, dev, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}; expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}; expected {dev}")


def _on_gpu(dev):
    if dev.type != "cuda":
        raise ValueError(f"tensors must be GPU tensors; got device {dev}")


def _ws(name, t, dev):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 1:
        raise TypeError(f"{name} must be a 1-D uint8 tensor")
    _need(name, t, t.shape, torch.uint8, dev)


def _inputs(q, k, v, log_alpha, b, w, ndim):
    """Checks the layer inputs ([B, T, H, d], or [N, H, d] for decode, ndim = 4 or 3) against q
    and returns (device, gate bits)."""
    for name, t in (("q", q), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != ndim:
            raise ValueError(f"{name} must be a {ndim}-D tensor")
    dt, dev = q.dtype, q.device
    _dtype(q)
    tok, dk, dv = tuple(q.shape[:-1]), q.shape[-1], v.shape[-1]
    bits = gate_bits(q, log_alpha, b, w)
    _need("q", q, q.shape, dt, dev)
    _need("k", k, q.shape, dt, dev)
    _need("v", v, tok + (dv,), dt, dev)
    _need("log_alpha", log_alpha, tok if bits & DECAY_SCALAR else tok + (dk,), torch.float32, dev)
    _need("b", b, tok if bits & ERASE_SCALAR else tok + (dk,), dt, dev)
    _need("w", w, tok if bits & WRITE_SCALAR else tok + (dv,), dt, dev)
    return dev, bits


def gdr2_fwd_chunked(q, k, v, log_alpha, b, w, S0=None, want_final_state=True, workspace=None,
                     prologue=None):
    """Chunked forward.  Returns (o, S_T or None, fwd_ws); fwd_ws holds the per-chunk factors and
    chunk-entry states that gdr2_bwd_chunked needs.  ``workspace`` may pass a preallocated uint8
    device tensor of at least the required size."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    dt = _dtype(q)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev, optional=True)
    if workspace is not None:
        _ws("workspace", workspace, dev)
    _on_gpu(dev)
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_final_state else None
    need = lib.gdr2_fwd_workspace_bytes(B, T, H, dk, dv, dt)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8,
                                                             device=dev)
    _run("gdr2_fwd_chunked", dev, lib.gdr2_fwd_chunked_ex, B, T, H, dk, dv, dt, bits,
         _pro(prologue), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0),
         _ptr(o), _ptr(ST), _ptr(ws), ws.numel())
    return o, ST, ws


def gdr2_bwd_chunked(q, k, v, log_alpha, b, w, dO, fwd_ws, dS_T=None, want_dS0=True,
                     workspace=None, prologue=None):
    """Gate-aware backward.  ``fwd_ws`` is the third result of gdr2_fwd_chunked on the same inputs.
    Returns a dict dq, dk, dv, dlog_alpha, db, dw, dS0 (None if not wanted).  ``prologue`` must
    be the one the forward ran with."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    dt = _dtype(q)
    _need("dO", dO, (B, T, H, dv), q.dtype, dev)
    _need("dS_T", dS_T, (B, H, dk, dv), torch.float32, dev, optional=True)
    _ws("fwd_ws", fwd_ws, dev)
    if workspace is not None:
        _ws("workspace", workspace, dev)
    _on_gpu(dev)
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
             dlog_alpha=torch.empty_like(log_alpha), db=torch.empty_like(b),
             dw=torch.empty_like(w),
             dS0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None)
    need = lib.gdr2_bwd_workspace_bytes(B, T, H, dk, dv, dt)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8,
                                                             device=dev)
    _run("gdr2_bwd_chunked", dev, lib.gdr2_bwd_chunked_ex, B, T, H, dk, dv, dt, bits,
         _pro(prologue), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
         _ptr(fwd_ws), fwd_ws.numel(), _ptr(dO), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]),
         _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]),
         _ptr(ws), ws.numel())
    return g


def gdr2_fwd_infer(q, k, v, log_alpha, b, w, S0=None, want_final_state=True, workspace=None,
                   prologue=None):
    """Forward-only chunked forward (no backward follows): o and S_T bit for bit as
    gdr2_fwd_chunked, without the chunk-entry states the backward would read.  Returns
    (o, S_T or None).  ``workspace`` may pass a preallocated uint8 device tensor of at least
    fwd_infer_workspace_bytes(...) bytes."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    dt = _dtype(q)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev, optional=True)
    if workspace is not None:
        _ws("workspace", workspace, dev)
    _on_gpu(dev)
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_final_state else None
    need = lib.gdr2_fwd_infer_workspace_bytes(B, T, H, dk, dv, dt)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8,
                                                             device=dev)
    _run("gdr2_fwd_infer", dev, lib.gdr2_fwd_infer_ex, B, T, H, dk, dv, dt, bits, _pro(prologue),
         _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(ST),
         _ptr(ws), ws.numel())
    return o, ST


def gdr2_fwd_infer_noalloc(q, k, v, log_alpha, b, w, S0=None, want_final_state=True, o=None,
                           S_T=None, prologue=None):
    """gdr2_fwd_infer through the no-allocation entry point: the library keeps the per-chunk
    factors in its static device scratch (at most fwd_infer_noalloc_max_bytes() bytes of them).
    ``o`` / ``S_T`` may pass preallocated outputs so that the call itself allocates nothing.
    Returns (o, S_T or None)."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    dt = _dtype(q)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev, optional=True)
    _need("o", o, (B, T, H, dv), q.dtype, dev, optional=True)
    _need("S_T", S_T, (B, H, dk, dv), torch.float32, dev, optional=True)
    _on_gpu(dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if S_T is None and want_final_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _run("gdr2_fwd_infer_noalloc", dev, lib.gdr2_fwd_infer_noalloc_ex, B, T, H, dk, dv, dt, bits,
         _pro(prologue), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0),
         _ptr(o), _ptr(S_T))
    return o, S_T


def fwd_infer_noalloc_max_bytes():
    return load_library().gdr2_fwd_infer_noalloc_max_bytes()


def gdr2_bwd_chunked_recompute(q, k, v, log_alpha, b, w, dO, S0=None, dS_T=None, want_dS0=True,
                               workspace=None, prologue=None):
    """Gate-aware backward without a forward workspace: the factors and chunk-entry states are
    recomputed from the inputs and S0.  Returns the dict of gdr2_bwd_chunked (bitwise equal)."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    dt = _dtype(q)
    _need("dO", dO, (B, T, H, dv), q.dtype, dev)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev, optional=True)
    _need("dS_T", dS_T, (B, H, dk, dv), torch.float32, dev, optional=True)
    if workspace is not None:
        _ws("workspace", workspace, dev)
    _on_gpu(dev)
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
             dlog_alpha=torch.empty_like(log_alpha), db=torch.empty_like(b),
             dw=torch.empty_like(w),
             dS0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None)
    need = lib.gdr2_bwd_recompute_workspace_bytes(B, T, H, dk, dv, dt)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8,
                                                             device=dev)
    _run("gdr2_bwd_chunked_recompute", dev, lib.gdr2_bwd_chunked_recompute_ex, B, T, H, dk, dv, dt,
         bits, _pro(prologue), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
         _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
         _ptr(g["dlog_alpha"]), _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]), _ptr(ws), ws.numel())
    return g


def _dt_code(dtype):
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}")
    return _DT[dtype]


def fwd_workspace_bytes(B, T, H, dk, dv, dtype):
    return load_library().gdr2_fwd_workspace_bytes(B, T, H, dk, dv, _dt_code(dtype))


def bwd_workspace_bytes(B, T, H, dk, dv, dtype):
    return load_library().gdr2_bwd_workspace_bytes(B, T, H, dk, dv, _dt_code(dtype))


def fwd_infer_workspace_bytes(B, T, H, dk, dv, dtype):
    return load_library().gdr2_fwd_infer_workspace_bytes(B, T, H, dk, dv, _dt_code(dtype))


def bwd_recompute_workspace_bytes(B, T, H, dk, dv, dtype):
    return load_library().gdr2_bwd_recompute_workspace_bytes(B, T, H, dk, dv, _dt_code(dtype))


def gdr2_fwd_factors(q, k, v, log_alpha, b, w, ws, prologue=None):
    """Stage 1 of the forward: per-chunk WY factors into ``ws`` (uint8 device tensor)."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    _ws("ws", ws, dev)
    _on_gpu(dev)
    _run("gdr2_fwd_factors", dev, lib.gdr2_fwd_factors_ex, B, T, H, dk, dv, _dtype(q), bits,
         _pro(prologue), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(ws),
         ws.numel())


def gdr2_fwd_carry(B, T, H, dk, dv, dtype, ws, o, S0=None, S_T=None):
    """Stage 2 of the forward: o (and S_T) from the factors in ``ws``."""
    lib = load_library()
    dt = _dt_code(dtype)
    if not isinstance(o, torch.Tensor):
        raise TypeError("o must be a tensor")
    dev = o.device
    _need("o", o, (B, T, H, dv), dtype, dev)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev, optional=True)
    _need("S_T", S_T, (B, H, dk, dv), torch.float32, dev, optional=True)
    _ws("ws", ws, dev)
    _on_gpu(dev)
    _run("gdr2_fwd_carry", dev, lib.gdr2_fwd_carry, B, T, H, dk, dv, dt, _ptr(S0), _ptr(o),
         _ptr(S_T), _ptr(ws), ws.numel())


def gdr2_bwd_state(B, T, H, dk, dv, dtype, fwd_ws, dO, bws, dS_T=None, dS0=None):
    """Stage 1 of the backward: per-chunk state gradients into ``bws`` and dS0."""
    lib = load_library()
    dt = _dt_code(dtype)
    if not isinstance(dO, torch.Tensor):
        raise TypeError("dO must be a tensor")
    dev = dO.device
    _need("dO", dO, (B, T, H, dv), dtype, dev)
    _need("dS_T", dS_T, (B, H, dk, dv), torch.float32, dev, optional=True)
    _need("dS0", dS0, (B, H, dk, dv), torch.float32, dev, optional=True)
    _ws("fwd_ws", fwd_ws, dev)
    _ws("bws", bws, dev)
    _on_gpu(dev)
    _run("gdr2_bwd_state", dev, lib.gdr2_bwd_state, B, T, H, dk, dv, dt, _ptr(fwd_ws),
         fwd_ws.numel(), _ptr(dO), _ptr(dS_T), _ptr(dS0), _ptr(bws), bws.numel())


def gdr2_bwd_grads(q, k, v, log_alpha, b, w, fwd_ws, dO, bws, g, prologue=None):
    """Stage 2 of the backward: fills g["dq"], g["dk"], g["dv"], g["dlog_alpha"], g["db"],
    g["dw"] (preallocated, each in the shape and dtype of its input)."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 4)
    B, T, H, dk, dv = _shapes(q, v)
    _need("dO", dO, (B, T, H, dv), q.dtype, dev)
    for name, like in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", log_alpha), ("db", b),
                       ("dw", w)):
        _need(name, g.get(name), like.shape, like.dtype, dev)
    _ws("fwd_ws", fwd_ws, dev)
    _ws("bws", bws, dev)
    _on_gpu(dev)
    _run("gdr2_bwd_grads", dev, lib.gdr2_bwd_grads_ex, B, T, H, dk, dv, _dtype(q), bits,
         _pro(prologue), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
         _ptr(fwd_ws), fwd_ws.numel(), _ptr(dO), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
         _ptr(g["dlog_alpha"]), _ptr(g["db"]), _ptr(g["dw"]), _ptr(bws), bws.numel())


def gdr2_decode_step(q, k, v, log_alpha, b, w, S_in=None, S_out=None, prologue=None):
    """One decode token for [N, H] sequences-heads.  S_out defaults to S_in (in place) or a new
    buffer.  Returns (o, S_out)."""
    lib = load_library()
    dev, bits = _inputs(q, k, v, log_alpha, b, w, 3)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype(q)
    _need("S_in", S_in, (N, H, dk, dv), torch.float32, dev, optional=True)
    _need("S_out", S_out, (N, H, dk, dv), torch.float32, dev, optional=True)
    _on_gpu(dev)
    if S_out is None:
        S_out = S_in if S_in is not None else torch.empty((N, H, dk, dv), dtype=torch.float32,
                                                          device=dev)
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _run("gdr2_decode_step", dev, lib.gdr2_decode_step_ex, N, H, dk, dv, dt, bits, _pro(prologue),
         _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S_in), _ptr(S_out),
         _ptr(o))
    return o, S_out


def _gate_inputs(o, g, weight):
    if not isinstance(o, torch.Tensor) or o.dim() < 1:
        raise ValueError("o must be a tensor [..., dv]")
    _dtype(o)
    dev, dv = o.device, o.shape[-1]
    _need("o", o, o.shape, o.dtype, dev)
    _need("g", g, o.shape, o.dtype, dev)
    _need("weight", weight, (dv,), torch.float32, dev)
    return dev, (o.numel() // dv if dv else 0), dv


def gdr2_out_gate_fwd(o, g, weight, eps=1e-6):
    """Output epilogue y = RMSNorm(o) * weight * silu(g) over the last (d_v) axis of o [..., dv];
    g has o's shape and dtype, weight is [dv] fp32.  Returns y."""
    lib = load_library()
    dev, rows, dv = _gate_inputs(o, g, weight)
    _on_gpu(dev)
    y = torch.empty_like(o)
    _run("gdr2_out_gate_fwd", dev, lib.gdr2_out_gate_fwd, rows, dv, _dtype(o), _ptr(o), _ptr(g),
         _ptr(weight), float(eps), _ptr(y))
    return y


def gdr2_out_gate_bwd(o, g, weight, dy, eps=1e-6, workspace=None):
    """Backward of gdr2_out_gate_fwd for the cotangent dy.  Returns dict do, dg, dweight."""
    lib = load_library()
    dev, rows, dv = _gate_inputs(o, g, weight)
    _need("dy", dy, o.shape, o.dtype, dev)
    if workspace is not None:
        _ws("workspace", workspace, dev)
    _on_gpu(dev)
    need = lib.gdr2_out_gate_bwd_workspace_bytes(rows, dv)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8,
                                                             device=dev)
    out = dict(do=torch.empty_like(o), dg=torch.empty_like(g),
               dweight=torch.empty((dv,), dtype=torch.float32, device=dev))
    _run("gdr2_out_gate_bwd", dev, lib.gdr2_out_gate_bwd, rows, dv, _dtype(o), _ptr(o), _ptr(g),
         _ptr(weight), float(eps), _ptr(dy), _ptr(out["do"]), _ptr(out["dg"]),
         _ptr(out["dweight"]), _ptr(ws), ws.numel())
    return out
