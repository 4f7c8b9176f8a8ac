"""GPU parity of the gate-aware backward (and the forward it depends on) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from gated_delta_rule_gdr_amd import gdr2_bwd_chunked, gdr2_fwd_chunked
from gated_delta_rule_gdr_amd.inputs import config_inputs, layer_inputs, strong_decay_inputs, to_f64
from oracle import oracle as orc
from tests._util import TOL, announce, assert_close, assert_close_chains, assert_close_rows, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def _run(x):
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S0=g["S0"])
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws,
                          dS_T=g.get("dST"))
    torch.cuda.synchronize()
    return o, ST, gr


def _oracle(x):
    f = to_f64(x)
    ro, rS = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["S0"])
    rg = orc.backward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["dO"], S0=f["S0"],
                      dST=f.get("dST"))
    return ro, rS, rg


def _check(x, tol, tag):
    announce(tag)
    o, ST, gr = _run(x)
    ro, rS, rg = _oracle(x)
    errs = {"o": assert_close_chains(f"{tag} o", to_np(o), ro, tol, "tok"),
            "S_T": assert_close_chains(f"{tag} S_T", to_np(ST), rS, tol, "state")}
    for n in GRADS:
        errs[n] = assert_close_chains(f"{tag} {n}", to_np(gr[n]), rg[n], tol,
                                      "state" if n == "dS0" else "tok")
    print("  " + tag + ": " + "  ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
    if tol <= TOL["f32"]:  # fp32: every row on its own as well
        rows = {"o": assert_close_rows(f"{tag} o rows", to_np(o), ro, tol, "tok"),
                "S_T": assert_close_rows(f"{tag} S_T rows", to_np(ST), rS, tol, "state")}
        for n in GRADS:
            rows[n] = assert_close_rows(f"{tag} {n} rows", to_np(gr[n]), rg[n], tol,
                                        "state" if n == "dS0" else "tok")
        print("  " + tag + " rows: " + "  ".join(f"{k} {v:.1e}" for k, v in rows.items()), flush=True)


@pytest.mark.parametrize("T", [1, 37, 64, 65, 130])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_bwd_bf16_shapes(T, dk, dv):
    x = layer_inputs(2, T, 3, dk, dv, dtype="bf16", seed=300 + T + dk + dv, s0_std=0.05, dST=True)
    _check(x, TOL["bf16"], f"bwd bf16 T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("T,dk,dv", [(1, 64, 64), (100, 64, 64), (130, 64, 128), (256, 64, 64),
                                     (200, 128, 128), (65, 128, 64)])
def test_bwd_fp32_shapes(T, dk, dv):
    x = layer_inputs(2, T, 2, dk, dv, dtype="f32", seed=400 + T + dk, s0_std=0.05, dST=True)
    _check(x, TOL["f32"], f"bwd f32 T={T} dk={dk} dv={dv}")


def test_bwd_pr1_fp32_workload():
    """The fp32 reference workload shape (B=1, H=1, T=256, d=64), with a backward."""
    c = dict(B=1, T=256, H=1, dk=64, dv=64)
    x = layer_inputs(**c, dtype="f32", seed=1000)
    _check(x, TOL["f32"], "bwd pr1 fp32")


def test_bwd_many_chains():
    """Enough chains that the state-gradient carry uses wide value slices."""
    x = layer_inputs(4, 130, 64, 128, 128, dtype="bf16", seed=7, dST=True)
    _check(x, TOL["bf16"], "bwd bf16 B=4 H=64")


def test_bwd_strong_decay():
    x = strong_decay_inputs(1, 192, 2, 128, 128, dtype="bf16", seed=11, floor=-5.0)
    x["dST"] = torch.randn(x["q"].shape[0], 2, 128, 128, generator=torch.Generator().manual_seed(3))
    _check(x, TOL["bf16"], "bwd bf16 strong decay")
    x = strong_decay_inputs(1, 192, 2, 64, 64, dtype="f32", seed=12, floor=-5.0)
    _check(x, TOL["f32"], "bwd f32 strong decay")


def _check_chains(tag, o, ST, gr, ro, rS, rg, tol):
    errs = {"o": assert_close_chains(f"{tag} o", to_np(o), ro, tol, "tok")}
    if ST is not None:
        errs["S_T"] = assert_close_chains(f"{tag} S_T", to_np(ST), rS, tol, "state")
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        errs[n] = assert_close_chains(f"{tag} {n}", to_np(gr[n]), rg[n], tol, "tok")
    errs["dS0"] = assert_close_chains(f"{tag} dS0", to_np(gr["dS0"]), rg["dS0"], tol, "state")
    print("  " + tag + " worst chain: " + "  ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)


def test_bwd_layer_1p3b_all_chains():
    """Model-shaped 1.3B layer (B=4, T=4096, H=16, d=128) in the launch configuration the bench
    times; the oracle recomputes forward and backward of all 64 (b, h) chains, each compared on
    its own."""
    x = config_inputs("layer_1p3b")
    announce("layer_1p3b fwd+bwd full size, all chains")
    o, ST, gr = _run(x)
    ro, rS, rg = _oracle(x)
    _check_chains("layer_1p3b", o, ST, gr, ro, rS, rg, TOL["bf16"])


def test_bwd_long_context_all_heads():
    """Long context (B=1, T=32768, H=16, d=128) with S0 ~ N(0, 0.02^2), returning the final state;
    the oracle recomputes all 16 chains."""
    x = config_inputs("long_ctx")
    announce("long_ctx fwd+bwd full size, all heads")
    o, ST, gr = _run(x)
    ro, rS, rg = _oracle(x)
    _check_chains("long_ctx", o, ST, gr, ro, rS, rg, TOL["bf16"])


@pytest.mark.parametrize("variant", ["tied_kda", "tied_gdn", "tied_la"])
def test_tied_gate_reductions(variant):
    """Tied-gate sweep (B=2, T=2048, H=16, d=128), all 32 chains: the forward must match the
    reduced rule's own oracle (KDA, Gated DeltaNet, or the linear-attention closed form), and the
    gradients of the tied parameters (sum of db and dw for beta; sum of dlog alpha for a scalar
    decay) must match the main oracle's."""
    x = config_inputs(variant)
    announce(variant)
    o, ST, gr = _run(x)
    f = to_f64(x)
    if variant == "tied_la":
        ro, rS = orc.la_closed_form(f["q"], f["k"], f["v"])
    else:
        ro, rS = orc.kda_forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"][..., 0],
                                 scalar_decay=(variant == "tied_gdn"))
    tol = TOL["bf16"]
    assert_close_chains(f"{variant} o", to_np(o), ro, tol, "tok")
    assert_close_chains(f"{variant} S_T", to_np(ST), rS, tol, "state")
    rg = orc.backward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["dO"])
    for n in ("dq", "dk", "dv"):
        assert_close_chains(f"{variant} {n}", to_np(gr[n]), rg[n], tol, "tok")
    gb = to_np(gr["db"]).sum(-1) + to_np(gr["dw"]).sum(-1)
    rb = rg["db"].sum(-1) + rg["dw"].sum(-1)
    assert_close_chains(f"{variant} dbeta", gb, rb, tol, "tok")
    gl = to_np(gr["dlog_alpha"])
    if variant == "tied_gdn":
        assert_close_chains(f"{variant} dlog_alpha (scalar)", gl.sum(-1), rg["dlog_alpha"].sum(-1), tol, "tok")
    else:
        assert_close_chains(f"{variant} dlog_alpha", gl, rg["dlog_alpha"], tol, "tok")


def test_bwd_split_sequence_handoff():
    """Forward and backward over [0, t1) and [t1, T) with S_T -> S0 and dS0 -> dS_T hand-off equal
    one pass over [0, T) (t1 not a multiple of the chunk)."""
    x = layer_inputs(1, 300, 2, 128, 128, dtype="bf16", seed=21, s0_std=0.05)
    announce("split hand-off")
    g = _gpu(x)
    o, ST, gr = _run(x)
    t1 = 141
    part = lambda a, sl: a[:, sl].contiguous()
    A = {n: (part(g[n], slice(0, t1)) if n not in ("S0", "dST") else g[n]) for n in g}
    Bp = {n: (part(g[n], slice(t1, None)) if n not in ("S0", "dST") else g[n]) for n in g}
    oA, SA, wsA = gdr2_fwd_chunked(A["q"], A["k"], A["v"], A["log_alpha"], A["b"], A["w"], S0=A["S0"])
    oB, SB, wsB = gdr2_fwd_chunked(Bp["q"], Bp["k"], Bp["v"], Bp["log_alpha"], Bp["b"], Bp["w"], S0=SA)
    gB = gdr2_bwd_chunked(Bp["q"], Bp["k"], Bp["v"], Bp["log_alpha"], Bp["b"], Bp["w"], Bp["dO"], wsB)
    gA = gdr2_bwd_chunked(A["q"], A["k"], A["v"], A["log_alpha"], A["b"], A["w"], A["dO"], wsA,
                          dS_T=gB["dS0"])
    torch.cuda.synchronize()
    assert_close("o", to_np(torch.cat([oA, oB], 1)), to_np(o), TOL["bf16"])
    assert_close("S_T", to_np(SB), to_np(ST), TOL["bf16"])
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        assert_close(n, to_np(torch.cat([gA[n], gB[n]], 1)), to_np(gr[n]), TOL["bf16"])
    assert_close("dS0", to_np(gA["dS0"]), to_np(gr["dS0"]), TOL["bf16"])


def test_bwd_deterministic():
    """Two runs give bitwise identical results (no floating-point atomics)."""
    x = layer_inputs(2, 200, 4, 128, 128, dtype="bf16", seed=31, dST=True)
    announce("determinism")
    _, _, g1 = _run(x)
    _, _, g2 = _run(x)
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_empty_sequence(dtype, d):
    """T = 0: no token is processed, so the forward returns S_T = S0 and the backward passes the
    state gradient straight through, dS0 = dS_T (both exactly); the token-shaped outputs are empty."""
    x = layer_inputs(2, 0, 3, d, d, dtype=dtype, seed=31, s0_std=0.05, dST=True)
    announce(f"empty sequence {dtype} d={d}")
    o, ST, gr = _run(x)
    assert o.shape == (2, 0, 3, d)
    assert torch.equal(ST.cpu(), x["S0"].float())
    assert torch.equal(gr["dS0"].cpu(), x["dST"].float())
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        assert gr[n].numel() == 0, n


@pytest.mark.parametrize("case", ["decay_only", "no_write", "full_erase"])
def test_degenerate_gates(case):
    """Degenerate gate settings from a random S0: pure decay (b = w = 0: the state only decays and
    o_t = S_t^T q_t), erase without write (w = 0), and a full-strength erase (b = 1); forward and
    backward against the oracle."""
    x = layer_inputs(2, 100, 3, 64, 64, dtype="bf16", seed=41, s0_std=0.05, dST=True)
    if case in ("decay_only", "no_write"):
        x["w"] = torch.zeros_like(x["w"])
    if case == "decay_only":
        x["b"] = torch.zeros_like(x["b"])
    if case == "full_erase":
        x["b"] = torch.ones_like(x["b"])
    _check(x, TOL["bf16"], f"degenerate gates {case}")
