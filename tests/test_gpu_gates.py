"""GPU parity of the gate-shape variants: the erase gate b, the write gate w and/or the decay
log alpha given as one value per (batch, token, head) instead of one per channel (the ablation
arms of the forum summary on zhichai.net, section "Ablation: the erase gate matters more", and
Gated DeltaNet's scalar decay).

The oracle receives the same gates broadcast over their channels; a scalar gate's gradient is
then the sum over its channels of the oracle's channel-wise gradient (the chain rule of the
broadcast, pinned against finite differences in tests/test_oracle.py)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_gdr_amd import gdr2_bwd_chunked, gdr2_decode_step, gdr2_fwd_chunked
from gated_delta_rule_gdr_amd.inputs import decode_inputs, layer_inputs, to_f64
from oracle import oracle as orc
from tests._util import TOL, announce, assert_close, assert_close_chains, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def _broadcast(f, dk, dv):
    """Channel-wise copies of the scalar gates (what the oracle consumes)."""
    g = dict(f)
    for n, d in (("b", dk), ("log_alpha", dk), ("w", dv)):
        if g[n].ndim == f["q"].ndim - 1:
            g[n] = np.ascontiguousarray(np.broadcast_to(g[n][..., None], g[n].shape + (d,)))
    return g


def _reduce(name, ref, gpu_shape):
    """The oracle's gradient in the gate's own shape (sum over channels for a scalar gate)."""
    return ref.sum(-1) if len(gpu_shape) == ref.ndim - 1 else ref


@pytest.mark.parametrize("scalar", ["b", "w", "a", "bw", "ba", "wa", "bwa"])
@pytest.mark.parametrize("dtype,dk,dv,T", [("bf16", 128, 128, 130), ("f32", 64, 64, 100),
                                           ("bf16", 64, 128, 65), ("bf16", 128, 64, 70),
                                           ("bf16", 64, 64, 100)])
def test_scalar_gates_fwd_bwd(scalar, dtype, dk, dv, T):
    x = layer_inputs(2, T, 3, dk, dv, dtype=dtype, seed=500 + T + len(scalar), s0_std=0.05,
                     dST=True, scalar=scalar)
    tag = f"scalar={scalar} {dtype} dk={dk} dv={dv} T={T}"
    announce(tag)
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S0=g["S0"])
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws,
                          dS_T=g["dST"])
    torch.cuda.synchronize()
    f = _broadcast(to_f64(x), dk, dv)
    ro, rS = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["S0"])
    rg = orc.backward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["dO"], S0=f["S0"],
                      dST=f["dST"])
    tol = TOL[dtype]
    assert_close(f"{tag} o", to_np(o), ro, tol)
    assert_close(f"{tag} S_T", to_np(ST), rS, tol)
    for n in ("dq", "dk", "dv", "dS0"):
        assert_close(f"{tag} {n}", to_np(gr[n]), rg[n], tol)
    for n, gate in (("db", "b"), ("dw", "w"), ("dlog_alpha", "log_alpha")):
        assert tuple(gr[n].shape) == tuple(x[gate].shape), n
        assert_close(f"{tag} {n}", to_np(gr[n]), _reduce(n, rg[n], gr[n].shape), tol)


def test_scalar_gates_equal_broadcast_channel_gates():
    """The scalar-gate path and the channel-wise path fed the broadcast gates agree (same
    arithmetic up to the order of the channel sums)."""
    x = layer_inputs(2, 200, 4, 128, 128, dtype="bf16", seed=77, scalar="bwa")
    announce("scalar vs broadcast")
    g = _gpu(x)
    gb = dict(g)
    gb["b"] = g["b"][..., None].expand(*g["b"].shape, 128).contiguous()
    gb["w"] = g["w"][..., None].expand(*g["w"].shape, 128).contiguous()
    gb["log_alpha"] = g["log_alpha"][..., None].expand(*g["log_alpha"].shape, 128).contiguous()
    o1, S1, ws1 = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"])
    o2, S2, ws2 = gdr2_fwd_chunked(gb["q"], gb["k"], gb["v"], gb["log_alpha"], gb["b"], gb["w"])
    g1 = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws1)
    g2 = gdr2_bwd_chunked(gb["q"], gb["k"], gb["v"], gb["log_alpha"], gb["b"], gb["w"], gb["dO"], ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for n in ("dq", "dk", "dv", "dS0"):
        assert torch.equal(g1[n], g2[n]), n
    for n in ("db", "dw", "dlog_alpha"):
        assert_close(n, to_np(g1[n]), to_np(g2[n].float().sum(-1)), 1e-2)


def test_scalar_gates_kda_reduction():
    """b = w = beta (both scalar) is KDA; with a scalar decay as well it is Gated DeltaNet: the
    forward must match the reduced rules' own oracle."""
    for scalar, gdn in (("bw", False), ("bwa", True)):
        x = layer_inputs(2, 300, 3, 128, 128, dtype="bf16", seed=91, scalar=scalar, grads=False)
        x["w"] = x["b"].clone()
        announce(f"kda reduction scalar={scalar}")
        g = _gpu(x)
        o, ST, _ = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"])
        torch.cuda.synchronize()
        f = to_f64(x)
        la = f["log_alpha"]
        if gdn:
            la = np.ascontiguousarray(np.broadcast_to(la[..., None], la.shape + (128,)))
        ro, rS = orc.kda_forward(f["q"], f["k"], f["v"], la, f["b"], scalar_decay=gdn)
        assert_close(f"kda {scalar} o", to_np(o), ro, TOL["bf16"])
        assert_close(f"kda {scalar} S_T", to_np(ST), rS, TOL["bf16"])


@pytest.mark.parametrize("scalar", ["b", "w", "a", "bwa"])
def test_scalar_gates_decode(scalar):
    N, H, dk, dv = 8, 4, 128, 128
    announce(f"decode scalar={scalar}")
    S = None
    fS = None
    for step in range(3):
        x = decode_inputs(step, N=N, H=H, dk=dk, dv=dv, scalar=scalar)
        g = _gpu(x)
        o, S = gdr2_decode_step(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S_in=S,
                                S_out=S)
        torch.cuda.synchronize()
        f = _broadcast(to_f64(x), dk, dv)
        ro, fS = orc.decode_step(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], S_in=fS)
        assert_close(f"decode {scalar} o step {step}", to_np(o), ro, TOL["bf16"])
        assert_close(f"decode {scalar} S step {step}", to_np(S), fS, TOL["bf16"])


@pytest.mark.parametrize("scalar", ["bw", "bwa"])
def test_scalar_gates_layer_1p3b_all_chains(scalar):
    """Model-shaped 1.3B layer (B=4, T=4096, H=16, d=128) with scalar erase and write gates (and
    scalar decay), in the launch configuration of the benchmark; the oracle recomputes every
    chain."""
    x = layer_inputs(4, 4096, 16, 128, 128, dtype="bf16", seed=1001, scalar=scalar)
    announce(f"layer_1p3b scalar {scalar}, all chains")
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"])
    gr = gdr2_bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["dO"], ws)
    torch.cuda.synchronize()
    f = _broadcast(to_f64(x), 128, 128)
    ro, _ = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"])
    rg = orc.backward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["dO"])
    tol = TOL["bf16"]
    assert_close_chains("o", to_np(o), ro, tol, "tok")
    for n in ("dq", "dk", "dv"):
        assert_close_chains(n, to_np(gr[n]), rg[n], tol, "tok")
    for n in ("db", "dw", "dlog_alpha"):  # a scalar gate's gradient: the oracle's channel sum
        assert_close_chains(n, to_np(gr[n]), _reduce(n, rg[n], gr[n].shape), tol, "tok")
