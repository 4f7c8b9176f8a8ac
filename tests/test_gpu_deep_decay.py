"""GPU parity at decays far beyond the default recipe: channels whose decay across one 16-token
block is below exp(-88) (the fp32 range of a factor exp(-G) referenced to the block start), whole
chunks at log alpha = -20 per token, and channels with no decay at all, mixed.  The decay is a
per-channel diagonal gate with alpha anywhere in (0, 1] (ainews.random.gg article on Gated
DeltaNet-2, section "Gated Delta Rule-2: two gates instead of one"; forum summary on zhichai.net,
section "The Memory Dilemma"), so nothing bounds it from below.

Forward, backward and decode against the fp64 oracle; every output must be finite and within the
tolerance, checked chain by chain."""
import numpy as np
import pytest
import torch

from gated_delta_rule_gdr_amd import Prologue, gdr2_bwd_chunked, gdr2_decode_step, gdr2_fwd_chunked
from gated_delta_rule_gdr_amd.inputs import deep_decay_inputs, layer_inputs, to_f64
from oracle import oracle as orc
from tests._util import TOL, announce, assert_close_chains, assert_close_rows, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw")


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def _run(x, prologue=None):
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S0=g["S0"],
                                 prologue=prologue)
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws,
                          dS_T=g.get("dST"), prologue=prologue)
    torch.cuda.synchronize()
    return o, ST, gr


def _check_all(tag, o, ST, gr, ro, rS, rg, tol):
    errs = {"o": assert_close_chains(f"{tag} o", to_np(o), ro, tol, "tok"),
            "S_T": assert_close_chains(f"{tag} S_T", to_np(ST), rS, tol, "state")}
    for n in GRADS:
        errs[n] = assert_close_chains(f"{tag} {n}", to_np(gr[n]), rg[n], tol, "tok")
    errs["dS0"] = assert_close_chains(f"{tag} dS0", to_np(gr["dS0"]), rg["dS0"], tol, "state")
    print("  " + tag + ": " + "  ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
    if tol <= TOL["f32"]:  # fp32: every row on its own as well
        rows = {"o": assert_close_rows(f"{tag} o rows", to_np(o), ro, tol, "tok"),
                "S_T": assert_close_rows(f"{tag} S_T rows", to_np(ST), rS, tol, "state"),
                "dS0": assert_close_rows(f"{tag} dS0 rows", to_np(gr["dS0"]), rg["dS0"], tol, "state")}
        for n in GRADS:
            rows[n] = assert_close_rows(f"{tag} {n} rows", to_np(gr[n]), rg[n], tol, "tok")
        print("  " + tag + " rows: " + "  ".join(f"{k} {v:.1e}" for k, v in rows.items()), flush=True)


def _check(x, tol, tag):
    announce(tag)
    o, ST, gr = _run(x)
    f = to_f64(x)
    ro, rS = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["S0"])
    rg = orc.backward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["dO"], S0=f["S0"],
                      dST=f.get("dST"))
    _check_all(tag, o, ST, gr, ro, rS, rg, tol)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64),
                                         ("bf16", 64, 128), ("f32", 64, 64), ("f32", 128, 128),
                                         ("f32", 128, 64)])
def test_deep_decay_fwd_bwd(dtype, dk, dv):
    """Half the key channels at log alpha in [-30, -6] per token, a quarter at 0, chunk 1 at -20,
    ragged last chunk."""
    x = deep_decay_inputs(2, 200, 3, dk, dv, dtype=dtype, seed=900 + dk + dv)
    _check(x, TOL[dtype], f"deep decay {dtype} dk={dk} dv={dv}")


def test_deep_decay_threshold_mix():
    """Per-token log alpha in [-4.4, -3.2] on every channel: 16-token block totals straddle the
    point where the kernels switch to their deep-decay path, so neighbouring chunks of one chain
    take different paths."""
    x = layer_inputs(2, 256, 3, 128, 128, dtype="bf16", seed=931, s0_std=0.05, dST=True)
    g = torch.Generator().manual_seed(932)
    x["log_alpha"] = (-4.4 + 1.2 * torch.rand(x["log_alpha"].shape, generator=g)).contiguous()
    _check(x, TOL["bf16"], "deep decay threshold mix bf16")
    x = layer_inputs(1, 256, 2, 64, 64, dtype="f32", seed=933, s0_std=0.05, dST=True)
    g = torch.Generator().manual_seed(934)
    x["log_alpha"] = (-4.4 + 1.2 * torch.rand(x["log_alpha"].shape, generator=g)).contiguous()
    _check(x, TOL["f32"], "deep decay threshold mix f32")


def test_deep_decay_extreme():
    """Single tokens that wipe a channel (log alpha = -1000 per token on some channels, e^-1000
    underflows to zero in any precision), next to channels without decay."""
    x = layer_inputs(1, 130, 2, 128, 128, dtype="bf16", seed=941, s0_std=0.05, dST=True)
    la = x["log_alpha"].clone()
    la[:, 10::17, :, :32] = -1000.0
    la[:, :, :, 32:64] = 0.0
    la[:, 70:90, :, 64:96] = -50.0
    x["log_alpha"] = la.contiguous()
    _check(x, TOL["bf16"], "deep decay extreme bf16")


def test_deep_decay_scalar_decay():
    """Deep decays through the scalar-decay gate shape (one log alpha per token and head), the
    Gated DeltaNet form of the decay; the oracle receives it broadcast over the channels."""
    x = layer_inputs(2, 150, 3, 128, 128, dtype="bf16", seed=951, s0_std=0.05, dST=True, scalar="a")
    g = torch.Generator().manual_seed(952)
    x["log_alpha"] = (-30.0 + 24.0 * torch.rand(x["log_alpha"].shape, generator=g)).contiguous()
    tag = "deep decay scalar log alpha"
    announce(tag)
    o, ST, gr = _run(x)
    f = to_f64(x)
    la = np.ascontiguousarray(np.broadcast_to(f["log_alpha"][..., None], f["q"].shape))
    ro, rS = orc.forward(f["q"], f["k"], f["v"], la, f["b"], f["w"], f["S0"])
    rg = orc.backward(f["q"], f["k"], f["v"], la, f["b"], f["w"], f["dO"], S0=f["S0"], dST=f["dST"])
    rg["dlog_alpha"] = rg["dlog_alpha"].sum(-1)
    tol = TOL["bf16"]
    assert_close_chains(f"{tag} o", to_np(o), ro, tol, "tok")
    assert_close_chains(f"{tag} S_T", to_np(ST), rS, tol, "state")
    for n in GRADS:
        assert_close_chains(f"{tag} {n}", to_np(gr[n]), rg[n], tol, "tok")
    assert_close_chains(f"{tag} dS0", to_np(gr["dS0"]), rg["dS0"], tol, "state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deep_decay_prologue(dtype):
    """The fused prologue's decay -c softplus(a) with large pre-activations a (c = 1, a up to 40)."""
    c, eps = 1.0, 1e-6
    x = layer_inputs(2, 140, 2, 128, 128, dtype=dtype, seed=961, s0_std=0.05, dST=True, raw=True)
    g = torch.Generator().manual_seed(962)
    big = 5.0 + 35.0 * torch.rand(x["log_alpha"].shape, generator=g)
    mask = torch.rand((2, 1, 2, 128), generator=g) < 0.5
    x["log_alpha"] = torch.where(mask, big, x["log_alpha"]).contiguous()
    tag = f"deep decay prologue {dtype}"
    announce(tag)
    o, ST, gr = _run(x, prologue=Prologue(c, eps))
    f = to_f64(x)
    p = orc.prologue_forward(f["q"], f["k"], f["log_alpha"], f["b"], f["w"], c, eps)
    ro, rS = orc.forward(p["q"], p["k"], f["v"], p["log_alpha"], p["b"], p["w"], f["S0"])
    rg = orc.backward(p["q"], p["k"], f["v"], p["log_alpha"], p["b"], p["w"], f["dO"], S0=f["S0"],
                      dST=f["dST"])
    rgp = orc.prologue_backward(f["q"], f["k"], f["log_alpha"], f["b"], f["w"], c, eps, rg)
    rgp["dv"], rgp["dS0"] = rg["dv"], rg["dS0"]
    _check_all(tag, o, ST, gr, ro, rS, rgp, TOL[dtype])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_deep_decay_decode_and_prefill(dtype, d):
    """A chunked prefill over deep-decay tokens, then decode steps with deep decays from its final
    state, against the oracle's token recurrence over the whole sequence."""
    T0, steps = 150, 6
    x = deep_decay_inputs(2, T0 + steps, 3, d, d, dtype=dtype, seed=971 + d, dST=False)
    tag = f"deep decay prefill + decode {dtype} d={d}"
    announce(tag)
    g = _gpu(x)
    pre = {n: g[n][:, :T0].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    o0, S, _ = gdr2_fwd_chunked(pre["q"], pre["k"], pre["v"], pre["log_alpha"], pre["b"], pre["w"],
                                S0=g["S0"])
    outs = []
    for t in range(T0, T0 + steps):
        ot, S = gdr2_decode_step(*(g[n][:, t].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")),
                                 S_in=S, S_out=S)
        outs.append(ot)
    torch.cuda.synchronize()
    f = to_f64(x)
    ro, rS = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["S0"])
    tol = TOL[dtype]
    assert_close_chains(f"{tag} prefill o", to_np(o0), ro[:, :T0], tol, "tok")
    assert_close_chains(f"{tag} decode o", to_np(torch.stack(outs, 1)), ro[:, T0:], tol, "tok")
    assert_close_chains(f"{tag} final state", to_np(S), rS, tol, "state")


def test_deep_decay_layer_full_size():
    """The model-shaped layer (B=4, T=4096, H=16, d=128, bf16) with the deep-decay recipe, in the
    launch configuration the benchmark times; every chain against the oracle, forward and
    backward."""
    x = deep_decay_inputs(4, 4096, 16, 128, 128, dtype="bf16", seed=981, s0_std=0.0, dST=False)
    _check(x, TOL["bf16"], "deep decay 1.3B layer, all chains")
