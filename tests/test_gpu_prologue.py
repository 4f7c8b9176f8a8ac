"""GPU parity of the fused prologue: q, k, log alpha, b and w handed over as pre-activations, and
the kernels apply the L2 normalisation of q and k, the sigmoid erase and write gates and the
softplus decay themselves (ainews.random.gg article on Gated DeltaNet-2, sections "Block design
and hybrid model" and "Gated Delta Rule-2: two gates instead of one").

The oracle maps the same pre-activations through its own prologue (pinned by closed forms and
finite differences in tests/test_oracle.py), runs the layer, and takes the gradients back through
the prologue's chain rule."""
import numpy as np
import pytest
import torch

from gated_delta_rule_gdr_amd import (Prologue, gdr2_bwd_chunked, gdr2_decode_step, gdr2_fwd_chunked,
                                     gdr2_fwd_infer)
from gated_delta_rule_gdr_amd.inputs import decode_inputs, layer_inputs, to_f64
from oracle import oracle as orc
from tests._util import TOL, announce, assert_close, assert_close_chains, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def _widen(x, d, like):
    return np.ascontiguousarray(np.broadcast_to(x[..., None], x.shape + (d,))) if x.ndim == like - 1 else x


def _oracle(f, c, eps, want_bwd=True):
    """Post-activations from the oracle's prologue, the layer, and the chain rule back."""
    dk, dv = f["q"].shape[-1], f["v"].shape[-1]
    p = orc.prologue_forward(f["q"], f["k"], f["log_alpha"], f["b"], f["w"], c, eps)
    nd = f["q"].ndim
    la, b, w = _widen(p["log_alpha"], dk, nd), _widen(p["b"], dk, nd), _widen(p["w"], dv, nd)
    ro, rS = orc.forward(p["q"], p["k"], f["v"], la, b, w, f.get("S0"))
    if not want_bwd:
        return ro, rS, None
    g = orc.backward(p["q"], p["k"], f["v"], la, b, w, f["dO"], S0=f.get("S0"), dST=f.get("dST"))
    for n, gate in (("dlog_alpha", "log_alpha"), ("db", "b"), ("dw", "w")):
        if f[gate].ndim == nd - 1:
            g[n] = g[n].sum(-1)
    rg = orc.prologue_backward(f["q"], f["k"], f["log_alpha"], f["b"], f["w"], c, eps, g)
    rg["dv"], rg["dS0"] = g["dv"], g["dS0"]
    return ro, rS, rg


@pytest.mark.parametrize("dtype,dk,dv,T,scalar,c", [
    ("bf16", 128, 128, 130, "", 0.1),
    ("f32", 64, 64, 100, "", 0.1),
    ("f32", 128, 128, 70, "", 1.0),
    ("bf16", 64, 128, 65, "bwa", 0.1),
    ("bf16", 128, 128, 200, "b", 0.5),
    ("f32", 128, 64, 150, "a", 0.1),
    ("bf16", 128, 64, 1, "", 0.1),
    ("bf16", 64, 64, 90, "", 0.3),
    ("bf16", 64, 128, 66, "", 0.1),
])
def test_prologue_fwd_bwd(dtype, dk, dv, T, scalar, c):
    eps = 1e-6
    x = layer_inputs(2, T, 3, dk, dv, dtype=dtype, seed=700 + T + dk + len(scalar), s0_std=0.05,
                     dST=True, scalar=scalar, raw=True)
    tag = f"prologue {dtype} dk={dk} dv={dv} T={T} scalar={scalar} c={c}"
    announce(tag)
    g = _gpu(x)
    pro = Prologue(c, eps)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S0=g["S0"],
                                 prologue=pro)
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws,
                          dS_T=g["dST"], prologue=pro)
    torch.cuda.synchronize()
    ro, rS, rg = _oracle(to_f64(x), c, eps)
    tol = TOL[dtype]
    assert_close(f"{tag} o", to_np(o), ro, tol)
    assert_close(f"{tag} S_T", to_np(ST), rS, tol)
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        assert_close(f"{tag} {n}", to_np(gr[n]), rg[n], tol)


def test_prologue_large_and_small_rows():
    """Pre-activation rows far from unit scale (x 40 and x 1/40) normalise to the same q, k; large
    |a|, |b|, |w| drive the gates into saturation without overflow."""
    x = layer_inputs(1, 96, 2, 128, 128, dtype="f32", seed=731, raw=True)
    x["q"][:, ::2] *= 40.0
    x["k"][:, 1::2] /= 40.0
    x["log_alpha"][:, :8] *= 30.0
    x["b"][:, 8:16] *= 25.0
    x["w"][:, 16:24] *= 25.0
    announce("prologue saturation")
    g = _gpu(x)
    pro = Prologue(0.2, 1e-6)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], prologue=pro)
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws,
                          prologue=pro)
    torch.cuda.synchronize()
    ro, rS, rg = _oracle(to_f64(x), 0.2, 1e-6)
    assert_close("o", to_np(o), ro, TOL["f32"])
    assert_close("S_T", to_np(ST), rS, TOL["f32"])
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        assert_close(n, to_np(gr[n]), rg[n], TOL["f32"])


@pytest.mark.parametrize("scalar", ["", "bwa"])
def test_prologue_decode(scalar):
    N, H, dk, dv = 8, 4, 128, 128
    c, eps = 0.3, 1e-6
    announce(f"prologue decode scalar={scalar}")
    pro = Prologue(c, eps)
    S = None
    fS = None
    for step in range(3):
        x = decode_inputs(step, N=N, H=H, dk=dk, dv=dv, scalar=scalar, raw=True)
        g = _gpu(x)
        o, S = gdr2_decode_step(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S_in=S,
                                S_out=S, prologue=pro)
        torch.cuda.synchronize()
        f = to_f64(x)
        p = orc.prologue_forward(f["q"], f["k"], f["log_alpha"], f["b"], f["w"], c, eps)
        ro, fS = orc.decode_step(p["q"], p["k"], f["v"], _widen(p["log_alpha"], dk, 3),
                                 _widen(p["b"], dk, 3), _widen(p["w"], dv, 3), S_in=fS)
        assert_close(f"decode o step {step}", to_np(o), ro, TOL["bf16"])
        assert_close(f"decode S step {step}", to_np(S), fS, TOL["bf16"])


def test_prologue_decode_continues_chunked_prefill():
    """A prefill through the forward-only chunked forward (no chunk-entry states stored) and three
    decode steps, both with the prologue, equal the oracle's recurrence over the whole sequence."""
    B, T, H, dk, dv = 2, 77, 2, 128, 128
    c, eps = 0.1, 1e-6
    x = layer_inputs(B, T + 3, H, dk, dv, dtype="bf16", seed=741, raw=True, grads=False)
    announce("prologue prefill + decode")
    g = _gpu(x)
    pro = Prologue(c, eps)
    pre = {n: g[n][:, :T].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    o0, S = gdr2_fwd_infer(pre["q"], pre["k"], pre["v"], pre["log_alpha"], pre["b"], pre["w"],
                           prologue=pro)
    outs = []
    for t in range(T, T + 3):
        tok = {n: g[n][:, t].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
        o, S = gdr2_decode_step(tok["q"], tok["k"], tok["v"], tok["log_alpha"], tok["b"], tok["w"],
                                S_in=S, S_out=S, prologue=pro)
        outs.append(o)
    torch.cuda.synchronize()
    ro, rS, _ = _oracle(to_f64(x), c, eps, want_bwd=False)
    assert_close("prefill o", to_np(o0), ro[:, :T], TOL["bf16"])
    for i, o in enumerate(outs):
        assert_close(f"decode token {i}", to_np(o), ro[:, T + i], TOL["bf16"])
    assert_close("final state", to_np(S), rS, TOL["bf16"])


def test_prologue_layer_1p3b_all_chains():
    """Model-shaped 1.3B layer (B=4, T=4096, H=16, d=128) with the fused prologue, in the launch
    configuration of the benchmark; the oracle recomputes every (batch, head) chain."""
    x = layer_inputs(4, 4096, 16, 128, 128, dtype="bf16", seed=1001, raw=True)
    announce("layer_1p3b prologue")
    g = _gpu(x)
    pro = Prologue(0.1, 1e-6)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], prologue=pro)
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws,
                          prologue=pro)
    torch.cuda.synchronize()
    f = to_f64(x)
    ro, _, rg = _oracle(f, 0.1, 1e-6)
    assert_close_chains("o", to_np(o), ro, TOL["bf16"], "tok")
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        assert_close_chains(n, to_np(gr[n]), rg[n], TOL["bf16"], "tok")
