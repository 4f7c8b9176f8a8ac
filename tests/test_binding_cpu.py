"""The Python binding's tensor checks, on host tensors.  The C ABI sees raw pointers only, so the
binding checks every tensor's shape, dtype, contiguity and device against the layout in
include/gdr2.h before it calls the library; a tensor of the wrong shape or dtype would otherwise
be read out of bounds by the kernels.  Every case here is rejected before any library call, and
a consistent set of host tensors is rejected only for not being on a GPU."""
import pytest
import torch

import gated_delta_rule_gdr_amd as g2

B, T, H, DK, DV = 1, 5, 2, 64, 128
BF, F32 = torch.bfloat16, torch.float32


def layer(dv=DV, scalar=""):
    tok = (B, T, H)
    x = dict(q=torch.zeros(tok + (DK,), dtype=BF), k=torch.zeros(tok + (DK,), dtype=BF),
             v=torch.zeros(tok + (dv,), dtype=BF),
             log_alpha=torch.zeros(tok if "a" in scalar else tok + (DK,), dtype=F32),
             b=torch.zeros(tok if "b" in scalar else tok + (DK,), dtype=BF),
             w=torch.zeros(tok if "w" in scalar else tok + (dv,), dtype=BF))
    return x


def fwd(x, **kw):
    return g2.gdr2_fwd_chunked(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], **kw)


@pytest.mark.parametrize("scalar", ["", "b", "w", "a", "bwa"])
def test_consistent_host_tensors_fail_only_on_device(scalar):
    with pytest.raises(ValueError, match="GPU tensors"):
        fwd(layer(scalar=scalar))


@pytest.mark.parametrize("name,bad,exc,msg", [
    ("k", torch.zeros(B, T, H, DK + 64, dtype=BF), ValueError, "k has shape"),
    ("v", torch.zeros(B, T + 1, H, DV, dtype=BF), ValueError, "v has shape"),
    ("b", torch.zeros(B, T, H, DV, dtype=BF), ValueError, "b has shape"),      # d_v channels, not d_k
    ("w", torch.zeros(B, T, H, DK, dtype=BF), ValueError, "w has shape"),      # d_k channels, not d_v
    ("log_alpha", torch.zeros(B, T, H, DK, dtype=BF), TypeError, "log_alpha has dtype"),
    ("k", torch.zeros(B, T, H, DK, dtype=F32), TypeError, "k has dtype"),
    ("w", torch.zeros(B, T, H, DV, dtype=F32), TypeError, "w has dtype"),
    ("b", torch.zeros(B, T, H, 2 * DK, dtype=BF)[..., ::2], ValueError, "b must be contiguous"),
    ("b", torch.zeros(B, T, H, DK, 1, dtype=BF), ValueError, "expected the token shape"),
    ("w", None, TypeError, "w must be a tensor"),
])
def test_layer_input_rejections(name, bad, exc, msg):
    x = layer()
    x[name] = bad
    with pytest.raises(exc, match=msg):
        fwd(x)


def test_optional_state_and_workspace_checks():
    x = layer()
    with pytest.raises(ValueError, match="S0 has shape"):
        fwd(x, S0=torch.zeros(B, H, DV, DK))
    with pytest.raises(TypeError, match="S0 has dtype"):
        fwd(x, S0=torch.zeros(B, H, DK, DV, dtype=BF))
    with pytest.raises(TypeError, match="workspace must be a 1-D uint8"):
        fwd(x, workspace=torch.zeros(16, dtype=F32))


def test_backward_checks():
    x = layer()
    dO = torch.zeros(B, T, H, DV, dtype=BF)
    ws = torch.zeros(16, dtype=torch.uint8)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"])
    with pytest.raises(ValueError, match="dO has shape"):
        g2.gdr2_bwd_chunked(*args, dO[:, :, :, :DK].contiguous(), ws)
    with pytest.raises(TypeError, match="dS_T has dtype"):
        g2.gdr2_bwd_chunked(*args, dO, ws, dS_T=torch.zeros(B, H, DK, DV, dtype=BF))
    with pytest.raises(TypeError, match="fwd_ws must be a 1-D uint8"):
        g2.gdr2_bwd_chunked(*args, dO, torch.zeros(4, 4, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensors"):
        g2.gdr2_bwd_chunked(*args, dO, ws)
    grads = {n: torch.zeros_like(x[s]) for n, s in (("dq", "q"), ("dk", "k"), ("dv", "v"),
                                                  ("dlog_alpha", "log_alpha"), ("db", "b"), ("dw", "w"))}
    bad = dict(grads, db=torch.zeros(B, T, H, dtype=BF))
    with pytest.raises(ValueError, match="db has shape"):
        g2.gdr2_bwd_grads(*args, ws, dO, ws, bad)
    with pytest.raises(ValueError, match="dw is required"):
        g2.gdr2_bwd_grads(*args, ws, dO, ws, {k: v for k, v in grads.items() if k != "dw"})
    with pytest.raises(ValueError, match="GPU tensors"):
        g2.gdr2_bwd_grads(*args, ws, dO, ws, grads)


def test_phase_entry_point_checks():
    ws = torch.zeros(16, dtype=torch.uint8)
    o = torch.zeros(B, T, H, DV, dtype=BF)
    with pytest.raises(ValueError, match="o has shape"):
        g2.gdr2_fwd_carry(B, T + 1, H, DK, DV, BF, ws, o)
    with pytest.raises(TypeError, match="o has dtype"):
        g2.gdr2_fwd_carry(B, T, H, DK, DV, F32, ws, o)
    with pytest.raises(TypeError, match="unsupported dtype"):
        g2.gdr2_fwd_carry(B, T, H, DK, DV, torch.float16, ws, o)
    with pytest.raises(ValueError, match="S_T has shape"):
        g2.gdr2_fwd_carry(B, T, H, DK, DV, BF, ws, o, S_T=torch.zeros(B, H, DK, DK))
    with pytest.raises(ValueError, match="GPU tensors"):
        g2.gdr2_fwd_carry(B, T, H, DK, DV, BF, ws, o)
    with pytest.raises(ValueError, match="dS0 has shape"):
        g2.gdr2_bwd_state(B, T, H, DK, DV, BF, ws, o, ws, dS0=torch.zeros(B, H, DK))
    with pytest.raises(ValueError, match="GPU tensors"):
        g2.gdr2_bwd_state(B, T, H, DK, DV, BF, ws, o, ws)
    x = layer()
    with pytest.raises(TypeError, match="ws must be a 1-D uint8"):
        g2.gdr2_fwd_factors(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], o)


def test_decode_checks():
    N = 3
    x = dict(q=torch.zeros(N, H, DK, dtype=BF), k=torch.zeros(N, H, DK, dtype=BF),
             v=torch.zeros(N, H, DV, dtype=BF), log_alpha=torch.zeros(N, H, DK),
             b=torch.zeros(N, H, DK, dtype=BF), w=torch.zeros(N, H, DV, dtype=BF))
    args = lambda: (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"])  # noqa: E731
    with pytest.raises(ValueError, match="S_in has shape"):
        g2.gdr2_decode_step(*args(), S_in=torch.zeros(N, H, DV, DK))
    with pytest.raises(TypeError, match="S_out has dtype"):
        g2.gdr2_decode_step(*args(), S_out=torch.zeros(N, H, DK, DV, dtype=BF))
    with pytest.raises(ValueError, match="GPU tensors"):
        g2.gdr2_decode_step(*args(), S_in=torch.zeros(N, H, DK, DV))
    x["q"] = torch.zeros(B, T, H, DK, dtype=BF)  # a chunked-layout tensor handed to decode
    with pytest.raises(ValueError, match="3-D"):
        g2.gdr2_decode_step(*args())


def test_out_gate_checks():
    o = torch.zeros(B, T, H, DV, dtype=BF)
    w = torch.ones(DV)
    with pytest.raises(TypeError, match="weight has dtype"):
        g2.gdr2_out_gate_fwd(o, o.clone(), w.to(BF))
    with pytest.raises(ValueError, match="weight has shape"):
        g2.gdr2_out_gate_fwd(o, o.clone(), torch.ones(DK))
    with pytest.raises(ValueError, match="g has shape"):
        g2.gdr2_out_gate_fwd(o, o[:, :1].contiguous(), w)
    with pytest.raises(TypeError, match="dy has dtype"):
        g2.gdr2_out_gate_bwd(o, o.clone(), w, o.float())
    with pytest.raises(ValueError, match="GPU tensors"):
        g2.gdr2_out_gate_fwd(o, o.clone(), w)
