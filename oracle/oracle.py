"""fp64 CPU oracle for the Gated Delta Rule-2 layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module.  The product library (``gated_delta_rule_gdr_amd``) never imports it, and it imports
nothing from the product library: the two share no code.

What lives here:
  * a ctypes wrapper around ``gdr2_oracle.c`` (token-by-token fp64 recurrence, its hand-derived
    reverse mode, one decode step, and the KDA / Gated DeltaNet reduced rules written as explicit
    transition-matrix products);
  * ``la_closed_form``: causal linear attention written as masked matrix products (the textbook
    definition), which is what GDR-2 must reduce to at alpha = 1, b = 0, w = 1;
  * ``gla_closed_form``: the b = 0 case as an explicit double sum over (query token, key token)
    with cumulative decay products, i.e. channel-wise gated linear attention;
  * ``out_gate_forward`` / ``out_gate_backward``: the block's output epilogue (RMS normalisation
    of each head's output over its d_v channels, a per-channel weight, a SiLU output gate) and its
    hand-derived vector-Jacobian product -- ainews.random.gg article, section "Block design and
    hybrid model";
  * ``prologue_forward`` / ``prologue_backward``: the transforms between the block's projections and
    the mixer (L2 normalisation of q and k, sigmoid erase and write gates, a decay log alpha =
    -c * softplus(a)) and their chain rule -- same article, sections "Block design and hybrid
    model" and "Gated Delta Rule-2: two gates instead of one".

Citations (page title, section):
  * update rule and the KDA / Gated DeltaNet reductions -- forum summary "Gated DeltaNet-2:
    Decoupling Erase and Write Gates in Linear Attention for Better Memory Editing"
    (zhichai.net, English), section "Gated Delta Rule-2";
  * decay before the edit, erase gate on the key side, write gate on the value side -- the
    ainews.random.gg article on NVIDIA's Gated DeltaNet-2, section "Gated Delta Rule-2: two gates
    instead of one";
  * "basic linear attention only adds" -- forum summary, section "The Memory Dilemma".

Every function takes and returns float64 numpy arrays in the layouts of ``gdr2_oracle.c``:
q, k, log_alpha, b: [B,T,H,dk]; v, w, o, dO: [B,T,H,dv]; states [B,H,dk,dv].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdr2_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP) next to its source and return the path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", "-o", tmp, _SRC,
             "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        L, P = ctypes.c_long, ctypes.c_void_p
        lib.gdr2o_forward.argtypes = [L] * 5 + [P] * 9
        lib.gdr2o_forward.restype = None
        lib.gdr2o_backward.argtypes = [L] * 5 + [P] * 16
        lib.gdr2o_backward.restype = None
        lib.gdr2o_decode_step.argtypes = [L] * 4 + [P] * 9
        lib.gdr2o_decode_step.restype = None
        lib.gdr2o_kda_forward.argtypes = [L] * 5 + [ctypes.c_int] + [P] * 8
        lib.gdr2o_kda_forward.restype = None
        lib.gdr2o_num_threads.argtypes = []
        lib.gdr2o_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().gdr2o_num_threads())


def forward(q, k, v, log_alpha, b, w, S0=None):
    """Token-by-token GDR-2 forward.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv])."""
    q, k, v, la, b, w, S0 = map(_f64, (q, k, v, log_alpha, b, w, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    _load().gdr2o_forward(B, T, H, dk, dv, *map(_ptr, (q, k, v, la, b, w, S0, o, ST)))
    return o, ST


def backward(q, k, v, log_alpha, b, w, dO, S0=None, dST=None):
    """Reverse mode of ``forward``.

    Returns a dict with dq, dk, dv, dlog_alpha, db, dw (token layouts) and dS0 [B,H,dk,dv].
    ``dST`` is the cotangent of the final state (None = 0)."""
    q, k, v, la, b, w, dO, S0, dST = map(_f64, (q, k, v, log_alpha, b, w, dO, S0, dST))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {n: np.zeros(q.shape) for n in ("dq", "dk", "dlog_alpha", "db")}
    out.update({n: np.zeros(v.shape) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((B, H, dk, dv))
    _load().gdr2o_backward(
        B, T, H, dk, dv, *map(_ptr, (q, k, v, la, b, w, S0, dO, dST, out["dq"], out["dk"],
                                      out["dv"], out["dlog_alpha"], out["db"], out["dw"],
                                      out["dS0"])))
    return out


def decode_step(q, k, v, log_alpha, b, w, S_in=None, S_out=None):
    """One recurrent token for N sequences x H heads.

    q, k, log_alpha, b: [N,H,dk]; v, w: [N,H,dv]; S_in: [N,H,dk,dv] or None (= 0).  ``S_out``
    (optional, C-contiguous float64) receives the new state; it may be S_in itself (in place).
    Returns (o [N,H,dv], S_out [N,H,dk,dv])."""
    inplace = S_out is not None and S_in is S_out
    q, k, v, la, b, w = map(_f64, (q, k, v, log_alpha, b, w))
    N, H, dk = q.shape
    dv = v.shape[-1]
    if S_out is None:
        S_out = np.zeros((N, H, dk, dv))
    if not (S_out.dtype == np.float64 and S_out.flags.c_contiguous and S_out.shape == (N, H, dk, dv)):
        raise ValueError("S_out must be a C-contiguous float64 [N,H,dk,dv] array")
    S_in = S_out if inplace else _f64(S_in)
    o = np.zeros((N, H, dv))
    _load().gdr2o_decode_step(N, H, dk, dv, *map(_ptr, (q, k, v, la, b, w, S_in, S_out, o)))
    return o, S_out


def kda_forward(q, k, v, log_alpha, beta, S0=None, scalar_decay=False):
    """Reduced rules: KDA (channel-wise decay, one scalar edit strength beta per token and head)
    and, with ``scalar_decay``, Gated DeltaNet (alpha is log_alpha[..., 0] per token and head).

    beta: [B,T,H].  Returns (o, S_T)."""
    q, k, v, la, beta, S0 = map(_f64, (q, k, v, log_alpha, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    _load().gdr2o_kda_forward(B, T, H, dk, dv, 1 if scalar_decay else 0,
                              *map(_ptr, (q, k, v, la, beta, S0, o, ST)))
    return o, ST


def la_closed_form(q, k, v, S0=None):
    """Causal linear attention (the rule that "only adds"), per (batch, head):
    O = tril(Q K^T) V + Q S0,   S_T = S0 + K^T V.   Returns (o, S_T)."""
    q, k, v, S0 = map(_f64, (q, k, v, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    mask = np.tril(np.ones((T, T)))
    for bb in range(B):
        for h in range(H):
            Q, K, V = q[bb, :, h], k[bb, :, h], v[bb, :, h]
            s0 = np.zeros((dk, dv)) if S0 is None else S0[bb, h]
            o[bb, :, h] = ((Q @ K.T) * mask) @ V + Q @ s0
            ST[bb, h] = s0 + K.T @ V
    return o, ST


def la_backward_closed_form(q, k, v, dO, S0=None, dST=None):
    """Gradients of ``la_closed_form`` written out as matrix products:
    with M = tril mask, P = (Q K^T) * M, dP = (dO V^T) * M:
      dQ = dP K + dO S0^T;  dK = dP^T Q + V dST^T;  dV = P^T dO + K dST;  dS0 = Q^T dO + dST."""
    q, k, v, dO, S0, dST = map(_f64, (q, k, v, dO, S0, dST))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    g = {n: np.zeros(q.shape) for n in ("dq", "dk")}
    g["dv"] = np.zeros(v.shape)
    g["dS0"] = np.zeros((B, H, dk, dv))
    mask = np.tril(np.ones((T, T)))
    for bb in range(B):
        for h in range(H):
            Q, K, V, D = q[bb, :, h], k[bb, :, h], v[bb, :, h], dO[bb, :, h]
            s0 = np.zeros((dk, dv)) if S0 is None else S0[bb, h]
            ds = np.zeros((dk, dv)) if dST is None else dST[bb, h]
            P = (Q @ K.T) * mask
            dP = (D @ V.T) * mask
            g["dq"][bb, :, h] = dP @ K + D @ s0.T
            g["dk"][bb, :, h] = dP.T @ Q + V @ ds.T
            g["dv"][bb, :, h] = P.T @ D + K @ ds
            g["dS0"][bb, h] = Q.T @ D + ds
    return g


def gla_closed_form(q, k, v, log_alpha, w, S0=None):
    """GDR-2 with b = 0 (no erase): channel-wise gated linear attention as an explicit sum,
        o_t[j] = sum_i q_t[i] * A(0,t)[i] * S0[i,j]
               + sum_{s<=t} sum_i q_t[i] k_s[i] A(s,t)[i] * w_s[j] v_s[j],
    with A(s,t)[i] = prod_{u=s+1..t} alpha_u[i] (and A(0,t) including alpha_1..alpha_t).
    O(T^2 d^2) -- tiny inputs only.  Returns o."""
    q, k, v, la, w, S0 = map(_f64, (q, k, v, log_alpha, w, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    for bb in range(B):
        for h in range(H):
            alpha = np.exp(la[bb, :, h])  # [T, dk]
            for t in range(T):
                acc = np.zeros(dv)
                if S0 is not None:
                    dec = np.prod(alpha[: t + 1], axis=0)
                    acc += (q[bb, t, h] * dec) @ S0[bb, h]
                for s in range(t + 1):
                    dec = np.prod(alpha[s + 1: t + 1], axis=0) if s < t else np.ones(dk)
                    coef = float(np.sum(q[bb, t, h] * k[bb, s, h] * dec))
                    acc += coef * w[bb, s, h] * v[bb, s, h]
                o[bb, t, h] = acc
    return o


def _silu(x):
    return x / (1.0 + np.exp(-x))


def out_gate_forward(o, g, weight, eps):
    """Output epilogue, per row (last axis = d_v channels):
        y = o / sqrt(mean(o^2) + eps) * weight * silu(g).   Returns y (float64)."""
    o, g, weight = map(_f64, (o, g, weight))
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * weight * _silu(g)


def out_gate_backward(o, g, weight, eps, dy):
    """Vector-Jacobian product of out_gate_forward for the cotangent dy, derived by hand:
        r = (mean(o^2) + eps)^(-1/2),  a = dy * weight * silu(g)
        do = r * a - r^3 * o * mean(a * o)           (dr/do_j = -r^3 o_j / d_v)
        dg = dy * o * r * weight * silu'(g),  silu'(x) = s + x s (1 - s),  s = sigmoid(x)
        dweight = sum over all rows of dy * o * r * silu(g)
    Returns dict do, dg, dweight."""
    o, g, weight, dy = map(_f64, (o, g, weight, dy))
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    s = 1.0 / (1.0 + np.exp(-g))
    a = dy * weight * (g * s)
    do = r * a - r ** 3 * o * np.mean(a * o, axis=-1, keepdims=True)
    dg = dy * o * r * weight * (s + g * s * (1.0 - s))
    dweight = (dy * o * r * (g * s)).reshape(-1, o.shape[-1]).sum(axis=0)
    return {"do": do, "dg": dg, "dweight": dweight}


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def prologue_forward(q, k, a, b, w, decay_scale, norm_eps):
    """Pre-activations -> the mixer's inputs (elementwise on gates of any shape):
        q_hat = q / sqrt(sum_i q_i^2 + eps)   (and likewise k, over the last axis)
        log_alpha = -decay_scale * softplus(a),   b = sigmoid(b),   w = sigmoid(w)
    Returns dict q, k, log_alpha, b, w (float64)."""
    q, k, a, b, w = map(_f64, (q, k, a, b, w))
    nq = 1.0 / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + norm_eps)
    nk = 1.0 / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + norm_eps)
    return {"q": q * nq, "k": k * nk, "log_alpha": -decay_scale * _softplus(a),
            "b": _sigmoid(b), "w": _sigmoid(w)}


def prologue_backward(q, k, a, b, w, decay_scale, norm_eps, g):
    """Chain rule through prologue_forward: ``g`` holds the gradients with respect to its outputs
    (dq, dk, dlog_alpha, db, dw); returns them with respect to the pre-activations.
        n = (sum q^2 + eps)^(-1/2):  d(q n)/dq applied to g = n g - n^3 q (q . g)
        d softplus(a)/da = sigmoid(a),   d sigmoid(x)/dx = s (1 - s)"""
    q, k, a, b, w = map(_f64, (q, k, a, b, w))

    def l2(x, gx):
        n = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + norm_eps)
        return n * gx - n ** 3 * x * np.sum(x * gx, axis=-1, keepdims=True)

    sb, sw = _sigmoid(b), _sigmoid(w)
    return {"dq": l2(q, _f64(g["dq"])), "dk": l2(k, _f64(g["dk"])),
            "dlog_alpha": -decay_scale * _sigmoid(a) * _f64(g["dlog_alpha"]),
            "db": sb * (1.0 - sb) * _f64(g["db"]), "dw": sw * (1.0 - sw) * _f64(g["dw"])}
