"""GPU tests of the forward-only forward and the recomputing backward (bitwise against the
training calls), and two metamorphic properties of the chunked layer that the oracle-free
structure of the method fixes:

  * channel-permutation equivariance: the update acts on key channels through elementwise gates
    and dot products over the key axis, and on value channels column by column (the gates are
    per-channel diagonals: ainews.random.gg article on Gated DeltaNet-2, section "Gated Delta
    Rule-2: two gates instead of one"), so permuting the key channels of q, k, b, log alpha (and
    the value channels of v, w, dO) permutes every output and gradient the same way;
  * chain isolation: each (batch, head) chain has its own state, so a NaN planted in one chain's
    inputs leaves every other chain's outputs and gradients bitwise unchanged;
  * the write gate and the value enter only through their product w . v (same section), so
    (w, v) -> (c w, v / c) leaves the forward unchanged and scales dv by c and dw by 1 / c;
  * for fixed q, k, b, w and decay the recurrence is linear in (v, S0) (the update equation,
    same section), and the backward is linear in the incoming gradients (dO, dS_T).
"""
import pytest
import torch

from gated_delta_rule_gdr_amd import (Prologue, gdr2_bwd_chunked, gdr2_bwd_chunked_recompute,
                                      gdr2_fwd_chunked, gdr2_fwd_infer)
from gated_delta_rule_gdr_amd.inputs import config_inputs, layer_inputs
from tests._util import TOL, announce, assert_close, assert_close_chains, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("q", "k", "v", "log_alpha", "b", "w")
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


@pytest.mark.parametrize("dtype,dk,dv,T,scalar,pro", [
    ("bf16", 128, 128, 200, "", None),
    ("f32", 64, 64, 130, "", None),
    ("bf16", 64, 128, 65, "bwa", None),
    ("bf16", 128, 128, 150, "", (0.1, 1e-6)),
    ("f32", 128, 64, 1, "b", None),
    ("bf16", 128, 128, 64 * 256 + 17, "", None),     # pipelined chunk ranges (few chains)
    ("bf16", 64, 64, 64 * 257, "bw", (0.1, 1e-6)),
])
def test_forward_only_equals_training_forward(dtype, dk, dv, T, scalar, pro):
    """o and S_T of the forward-only call equal the training forward's bit for bit, and the
    recomputing backward's gradients equal those of the backward that reads the forward
    workspace."""
    x = layer_inputs(2, T, 3, dk, dv, dtype=dtype, seed=1100 + T + dk, s0_std=0.05, dST=True,
                     scalar=scalar, raw=pro is not None)
    tag = f"forward-only {dtype} dk={dk} dv={dv} T={T} scalar={scalar} pro={pro}"
    announce(tag)
    g = _gpu(x)
    P = Prologue(*pro) if pro else None
    o, ST, ws = gdr2_fwd_chunked(*(g[n] for n in NAMES), S0=g["S0"], prologue=P)
    gr = gdr2_bwd_chunked(*(g[n] for n in NAMES), g["dO"], ws, dS_T=g["dST"], prologue=P)
    o2, ST2 = gdr2_fwd_infer(*(g[n] for n in NAMES), S0=g["S0"], prologue=P)
    gr2 = gdr2_bwd_chunked_recompute(*(g[n] for n in NAMES), g["dO"], S0=g["S0"], dS_T=g["dST"],
                                     prologue=P)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    for n in GRADS:
        assert torch.equal(gr[n], gr2[n]), n


def test_forward_only_layer_1p3b():
    """At the 1.3B-layer size (B=4, T=4096, H=16, d=128): the forward-only call equals the
    training forward bitwise and the recomputing backward equals the stored-workspace backward."""
    x = config_inputs("layer_1p3b")
    announce("forward-only layer_1p3b")
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(*(g[n] for n in NAMES))
    gr = gdr2_bwd_chunked(*(g[n] for n in NAMES), g["dO"], ws)
    del ws
    o2, ST2 = gdr2_fwd_infer(*(g[n] for n in NAMES))
    gr2 = gdr2_bwd_chunked_recompute(*(g[n] for n in NAMES), g["dO"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    for n in GRADS:
        assert torch.equal(gr[n], gr2[n]), n


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 128)])
def test_channel_permutation_equivariance(dtype, dk, dv):
    """Permuted key channels (q, k, b, log alpha) and value channels (v, w, dO, and S0, dS_T on
    both axes) give the permuted outputs and gradients.  The chunked kernels group channels into
    MFMA tiles and rows of 16 lanes, so the permuted problem runs through different tile
    placements: equal within the tolerance (not bitwise)."""
    x = layer_inputs(2, 150, 3, dk, dv, dtype=dtype, seed=1200 + dk, s0_std=0.05, dST=True)
    gen = torch.Generator().manual_seed(1201)
    pk, pv = torch.randperm(dk, generator=gen), torch.randperm(dv, generator=gen)
    y = dict(x)
    for n in ("q", "k", "b", "log_alpha"):
        y[n] = x[n][..., pk].contiguous()
    for n in ("v", "w", "dO"):
        y[n] = x[n][..., pv].contiguous()
    for n in ("S0", "dST"):
        y[n] = x[n][:, :, pk][..., pv].contiguous()
    tag = f"permutation {dtype} dk={dk} dv={dv}"
    announce(tag)
    res = []
    for z in (x, y):
        g = _gpu(z)
        o, ST, ws = gdr2_fwd_chunked(*(g[n] for n in NAMES), S0=g["S0"])
        gr = gdr2_bwd_chunked(*(g[n] for n in NAMES), g["dO"], ws, dS_T=g["dST"])
        res.append((o, ST, gr))
    torch.cuda.synchronize()
    (o, ST, gr), (o2, ST2, gr2) = res
    tol = TOL[dtype]
    assert_close("o", to_np(o2), to_np(o[..., pv]), tol)
    assert_close("S_T", to_np(ST2), to_np(ST[:, :, pk][..., pv]), tol)
    for n in ("dq", "dk", "db", "dlog_alpha"):
        assert_close(n, to_np(gr2[n]), to_np(gr[n][..., pk]), tol)
    for n in ("dv", "dw"):
        assert_close(n, to_np(gr2[n]), to_np(gr[n][..., pv]), tol)
    assert_close("dS0", to_np(gr2["dS0"]), to_np(gr["dS0"][:, :, pk][..., pv]), tol)


def test_nan_isolated_to_its_chain():
    """At the benchmarked grid (B=4, T=4096, H=16, d=128: heads-fastest workgroup order, XCD
    swizzle of the value slices), a NaN in one chain's inputs leaves every other chain's outputs
    and gradients bitwise unchanged and does reach its own chain."""
    x = config_inputs("layer_1p3b")
    announce("NaN isolation, layer_1p3b grid")
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(*(g[n] for n in NAMES))
    gr = gdr2_bwd_chunked(*(g[n] for n in NAMES), g["dO"], ws)
    del ws
    bad = {n: g[n].clone() for n in NAMES}
    bb, hh, t = 2, 7, 1000
    bad["k"][bb, t, hh, 5] = float("nan")
    o2, ST2, ws2 = gdr2_fwd_chunked(*(bad[n] for n in NAMES))
    gr2 = gdr2_bwd_chunked(*(bad[n] for n in NAMES), g["dO"], ws2)
    torch.cuda.synchronize()
    keep = torch.ones((4, 16), dtype=torch.bool, device=DEV)
    keep[bb, hh] = False
    assert torch.equal(o.permute(0, 2, 1, 3)[keep], o2.permute(0, 2, 1, 3)[keep])
    assert torch.equal(ST[keep], ST2[keep])
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        assert torch.equal(gr[n].permute(0, 2, 1, 3)[keep], gr2[n].permute(0, 2, 1, 3)[keep]), n
    assert torch.equal(gr["dS0"][keep], gr2["dS0"][keep])
    assert torch.isnan(o2[bb, t:, hh]).any() and torch.isnan(ST2[bb, hh]).any()


@pytest.mark.parametrize("dtype,dk,dv,T", [("bf16", 128, 128, 200), ("f32", 64, 128, 130)])
def test_write_gate_value_rescaling(dtype, dk, dv, T):
    """(w, v) -> (4 w, v / 4): a power-of-two scale is exact in both dtypes and commutes with
    every rounding the kernels do on w . v, dX . w and dX . v, so the forward is bitwise the same
    and dv, dw come back scaled by exactly 4 and 1/4; the other gradients are bitwise the same."""
    x = layer_inputs(2, T, 3, dk, dv, dtype=dtype, seed=1300 + dk, s0_std=0.05, dST=True)
    y = dict(x)
    y["w"] = x["w"] * 4
    y["v"] = x["v"] / 4
    announce(f"write-gate rescaling {dtype} dk={dk} dv={dv} T={T}")
    res = []
    for z in (x, y):
        g = _gpu(z)
        o, ST, ws = gdr2_fwd_chunked(*(g[n] for n in NAMES), S0=g["S0"])
        gr = gdr2_bwd_chunked(*(g[n] for n in NAMES), g["dO"], ws, dS_T=g["dST"])
        res.append((o, ST, gr))
    torch.cuda.synchronize()
    (o, ST, gr), (o2, ST2, gr2) = res
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    for n in ("dq", "dk", "db", "dlog_alpha", "dS0"):
        assert torch.equal(gr[n], gr2[n]), n
    assert torch.equal(gr2["dv"], gr["dv"] * 4)
    assert torch.equal(gr2["dw"], gr["dw"] / 4)


@pytest.mark.parametrize("dtype,dk,dv,T", [("f32", 128, 128, 200), ("bf16", 64, 128, 130)])
def test_linearity_in_values_state_and_gradients(dtype, dk, dv, T):
    """Forward: (v, S0) -> (o, S_T) is linear for fixed q, k, b, w and decay.  Backward: every
    gradient is linear in (dO, dS_T) for fixed forward inputs.  The two summands live on disjoint
    halves of the sequence (values and dO) and of the key rows (S0 and dS_T), so their sums are
    exact inputs in both dtypes; the results agree within the dtype's tolerance, chain by chain."""
    x = layer_inputs(2, T, 3, dk, dv, dtype=dtype, seed=1400 + dk, s0_std=0.05, dST=True)
    half, kh = T // 2, dk // 2
    a, b_ = dict(x), dict(x)
    a["v"] = x["v"].clone(); a["v"][:, half:] = 0
    b_["v"] = x["v"].clone(); b_["v"][:, :half] = 0
    a["S0"] = x["S0"].clone(); a["S0"][:, :, kh:] = 0
    b_["S0"] = x["S0"].clone(); b_["S0"][:, :, :kh] = 0
    a["dO"] = x["dO"].clone(); a["dO"][:, :half] = 0
    b_["dO"] = x["dO"].clone(); b_["dO"][:, half:] = 0
    a["dST"] = x["dST"].clone(); a["dST"][:, :, :kh] = 0
    b_["dST"] = x["dST"].clone(); b_["dST"][:, :, kh:] = 0
    announce(f"linearity {dtype} dk={dk} dv={dv} T={T}")
    fwd, bwd = [], []
    for z in (x, a, b_):
        g = _gpu(z)
        o, ST, _ = gdr2_fwd_chunked(*(g[n] for n in NAMES), S0=g["S0"])
        fwd.append((o.double(), ST.double()))
    gx = _gpu(x)
    _, _, ws = gdr2_fwd_chunked(*(gx[n] for n in NAMES), S0=gx["S0"])
    for z in (x, a, b_):
        gz = _gpu(z)
        gr = gdr2_bwd_chunked(*(gx[n] for n in NAMES), gz["dO"], ws, dS_T=gz["dST"])
        bwd.append({n: gr[n].double() for n in GRADS})
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert_close_chains("o", to_np(fwd[1][0] + fwd[2][0]), to_np(fwd[0][0]), tol, "tok")
    assert_close_chains("S_T", to_np(fwd[1][1] + fwd[2][1]), to_np(fwd[0][1]), tol, "state")
    for n in GRADS:
        lay = "state" if n == "dS0" else "tok"
        assert_close_chains(n, to_np(bwd[1][n] + bwd[2][n]), to_np(bwd[0][n]), tol, lay)
