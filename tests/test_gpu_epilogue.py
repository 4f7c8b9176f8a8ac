"""GPU parity of the output epilogue (RMS normalisation over d_v x per-channel weight x SiLU
output gate; ainews.random.gg article on Gated DeltaNet-2, section "Block design and hybrid
model") and of its backward, against the fp64 oracle."""
import numpy as np
import pytest
import torch

from gated_delta_rule_gdr_amd import gdr2_fwd_chunked, gdr2_out_gate_bwd, gdr2_out_gate_fwd
from gated_delta_rule_gdr_amd.inputs import layer_inputs
from oracle import oracle as orc
from tests._util import TOL, announce, assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(shape, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    o = torch.randn(shape, generator=gen).to(_DT[dtype])
    g = torch.randn(shape, generator=gen).to(_DT[dtype])
    dy = torch.randn(shape, generator=gen).to(_DT[dtype])
    w = (1.0 + 0.1 * torch.randn(shape[-1], generator=gen)).float()
    return o, g, w, dy


def _check(o, g, w, dy, eps, dtype, tag):
    announce(tag)
    od, gd, wd, dyd = (t.to(DEV) for t in (o, g, w, dy))
    y = gdr2_out_gate_fwd(od, gd, wd, eps)
    gr = gdr2_out_gate_bwd(od, gd, wd, dyd, eps)
    torch.cuda.synchronize()
    f = [t.double().numpy() for t in (o, g, w, dy)]
    ry = orc.out_gate_forward(f[0], f[1], f[2], eps)
    rg = orc.out_gate_backward(f[0], f[1], f[2], eps, f[3])
    tol = TOL[dtype]
    assert_close(f"{tag} y", to_np(y), ry, tol)
    assert_close(f"{tag} do", to_np(gr["do"]), rg["do"], tol)
    assert_close(f"{tag} dg", to_np(gr["dg"]), rg["dg"], tol)
    assert_close(f"{tag} dweight", to_np(gr["dweight"]), rg["dweight"], tol)
    return gr


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 37, 3), (1, 300, 5)])
def test_out_gate_shapes(dtype, dv, B, T, H):
    o, g, w, dy = _inputs((B, T, H, dv), dtype, seed=B * 1000 + T + H + dv)
    _check(o, g, w, dy, 1e-6, dtype, f"out gate {dtype} dv={dv} B={B} T={T} H={H}")


def test_out_gate_layer_1p3b_on_layer_output():
    """The epilogue on the mixer output of the 1.3B-layer workload (B=4, T=4096, H=16, d=128),
    every row checked."""
    x = layer_inputs(4, 4096, 16, 128, 128, dtype="bf16", seed=1001, grads=False)
    announce("out gate on layer output")
    gx = {n: (None if t is None else t.to(DEV)) for n, t in x.items()}
    o, _, _ = gdr2_fwd_chunked(gx["q"], gx["k"], gx["v"], gx["log_alpha"], gx["b"], gx["w"],
                               want_final_state=False)
    torch.cuda.synchronize()
    _, g, w, dy = _inputs(tuple(o.shape), "bf16", seed=42)
    _check(o.cpu(), g, w, dy, 1e-6, "bf16", "out gate 1.3B layer")


def test_out_gate_eps_and_zero_rows():
    """A zero row stays zero (eps keeps the scale finite); a large eps damps the output."""
    o, g, w, dy = _inputs((2, 8, 2, 128), "f32", seed=9)
    o[0, 3, 1] = 0.0
    gr = _check(o, g, w, dy, 1e-6, "f32", "zero row")
    assert torch.all(gr["do"][0, 3, 1].isfinite())
    _check(o, g, w, dy, 10.0, "f32", "large eps")


def test_out_gate_deterministic():
    o, g, w, dy = (t.to(DEV) for t in _inputs((4, 512, 16, 128), "bf16", seed=11))
    announce("out gate determinism")
    a = gdr2_out_gate_bwd(o, g, w, dy)
    b = gdr2_out_gate_bwd(o, g, w, dy)
    torch.cuda.synchronize()
    for n in ("do", "dg", "dweight"):
        assert torch.equal(a[n], b[n]), n


def test_out_gate_empty_input():
    """No rows (T = 0): the forward writes nothing and the weight gradient is exactly zero."""
    o, g, w, dy = (t.to(DEV) for t in _inputs((1, 0, 2, 128), "bf16", seed=5))
    announce("out gate empty input")
    y = gdr2_out_gate_fwd(o, g, w)
    gr = gdr2_out_gate_bwd(o, g, w, dy)
    torch.cuda.synchronize()
    assert y.shape == o.shape and gr["do"].shape == o.shape and gr["dg"].shape == g.shape
    assert torch.equal(gr["dweight"].cpu(), torch.zeros(128))
