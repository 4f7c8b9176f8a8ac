"""The no-allocation forward-only entry point (gdr2_fwd_infer_noalloc_ex, static device scratch)
against the forward-only entry point with a caller workspace (gdr2_fwd_infer_ex), through the C
ABI: two calls in a row, the second on a smaller problem (the scratch still holds the first
call's factors), each equal bit for bit to the workspace call on the same inputs; and a problem
whose factors exceed the scratch is refused before any launch."""
import pytest
import torch

from gated_delta_rule_gdr_amd import (Gdr2Error, Prologue, fwd_infer_noalloc_max_bytes,
                                      fwd_infer_workspace_bytes, gdr2_fwd_infer, gdr2_fwd_infer_noalloc)
from gated_delta_rule_gdr_amd.inputs import layer_inputs
from tests._util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("q", "k", "v", "log_alpha", "b", "w")


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def test_noalloc_equals_workspace_call_twice():
    cases = [  # (shape, dtype, scalar gates, prologue): the second is the smaller problem
        (dict(B=2, T=1000, H=8, dk=128, dv=128), "bf16", "", None),
        (dict(B=1, T=130, H=3, dk=64, dv=128), "f32", "b", Prologue(0.5, 1e-6)),
    ]
    for i, (shp, dt, scalar, pro) in enumerate(cases):
        tag = f"no-alloc call {i}: {shp} {dt} scalar={scalar} prologue={pro is not None}"
        announce(tag)
        need = fwd_infer_workspace_bytes(shp["B"], shp["T"], shp["H"], shp["dk"], shp["dv"],
                                         torch.bfloat16 if dt == "bf16" else torch.float32)
        assert need <= fwd_infer_noalloc_max_bytes()
        x = layer_inputs(**shp, dtype=dt, seed=1300 + i, s0_std=0.05, grads=False, scalar=scalar,
                         raw=pro is not None)
        g = _gpu(x)
        o_ref, S_ref = gdr2_fwd_infer(*(g[n] for n in NAMES), S0=g["S0"], prologue=pro)
        o = torch.full_like(o_ref, float("nan"))
        S = torch.full_like(S_ref, float("nan"))
        gdr2_fwd_infer_noalloc(*(g[n] for n in NAMES), S0=g["S0"], o=o, S_T=S, prologue=pro)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), tag
        assert torch.equal(S, S_ref), tag


def test_noalloc_refuses_problem_beyond_scratch():
    """T such that the factors need more than the scratch: GDR2_E_TOO_LARGE, nothing launched
    (the output buffer keeps its contents)."""
    H, d = 16, 128
    per_chunk = fwd_infer_workspace_bytes(1, 64, H, d, d, torch.bfloat16)
    T = 64 * (fwd_infer_noalloc_max_bytes() // per_chunk + 2)
    x = layer_inputs(1, T, H, d, d, dtype="bf16", seed=1310, grads=False, device=DEV)
    announce(f"no-alloc beyond scratch T={T}")
    o = torch.zeros((1, T, H, d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(Gdr2Error, match="GDR2_E_TOO_LARGE"):
        gdr2_fwd_infer_noalloc(*(x[n] for n in NAMES), o=o, want_final_state=False)
    torch.cuda.synchronize()
    assert not o.any()
