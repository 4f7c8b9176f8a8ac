"""GPU parity of the chunked forward and of decode against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_gdr_amd import gdr2_decode_step, gdr2_fwd_chunked
from gated_delta_rule_gdr_amd.inputs import (DECODE, config_inputs, decode_inputs, layer_inputs,
                                             strong_decay_inputs, to_f64)
from oracle import oracle as orc
from tests._util import TOL, announce, assert_close, assert_close_chains, assert_close_rows, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def _run_fwd(x):
    g = _gpu(x)
    o, ST, ws = gdr2_fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"],
                                 S0=g["S0"])
    torch.cuda.synchronize()
    return o, ST, ws


def _states_view(ws, B, T, H, dk, dv, dtype):
    """The chunk-entry states inside the forward workspace: the last region of the layout
    (-Y, Qbar, Ktilde [C][dk]; P, T [C][C]; U [C][dv]; gamma [dk] fp32; states [dv][dk]), each
    region rounded up to 256 bytes."""
    es = 2 if dtype == torch.bfloat16 else 4
    NC = (T + 63) // 64
    ncc = B * H * NC
    r = lambda n: (n + 255) // 256 * 256
    off = 3 * r(ncc * 64 * dk * es) + 2 * r(ncc * 64 * 64 * es) + r(ncc * 64 * dv * es) + r(ncc * dk * 4)
    n = ncc * dv * dk
    return ws[off:off + n * es].view(dtype).view(B, H, NC, dv, dk)


def _check_fwd(x, tol, tag):
    announce(tag)
    o, ST, _ = _run_fwd(x)
    f = to_f64(x)
    ro, rS = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], f["S0"])
    eo = assert_close_chains(f"{tag} o", to_np(o), ro, tol, "tok")
    eS = assert_close_chains(f"{tag} S_T", to_np(ST), rS, tol, "state")
    msg = f"  {tag}: o {eo:.2e}  S_T {eS:.2e}"
    if tol <= TOL["f32"]:  # fp32: every row on its own as well
        ro_ = assert_close_rows(f"{tag} o rows", to_np(o), ro, tol, "tok")
        rS_ = assert_close_rows(f"{tag} S_T rows", to_np(ST), rS, tol, "state")
        msg += f"  (rows: o {ro_:.2e}  S_T {rS_:.2e})"
    print(msg, flush=True)


def test_fwd_pr1_fp32():
    """The fp32 reference workload: B=1, H=1, T=256, d=64."""
    _check_fwd(config_inputs("pr1_fp32"), TOL["f32"], "pr1_fp32")


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_fwd_bf16_shapes(T, dk, dv):
    x = layer_inputs(2, T, 3, dk, dv, dtype="bf16", seed=10 + T + dk + dv, s0_std=0.05, grads=False)
    _check_fwd(x, TOL["bf16"], f"bf16 T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("T,dk,dv", [(1, 64, 64), (130, 64, 64), (130, 64, 128), (256, 64, 128),
                                     (200, 128, 128), (65, 128, 64)])
def test_fwd_fp32_shapes(T, dk, dv):
    x = layer_inputs(2, T, 2, dk, dv, dtype="f32", seed=20 + T + dv, s0_std=0.05, grads=False)
    _check_fwd(x, TOL["f32"], f"f32 T={T} dk={dk} dv={dv}")


def test_fwd_many_chains_slice_paths():
    """Enough (b, h) chains that the wider value slices (fewer workgroups per chain) are used."""
    x = layer_inputs(4, 130, 64, 128, 128, dtype="bf16", seed=5, grads=False)
    _check_fwd(x, TOL["bf16"], "bf16 B=4 H=64 (wide slices)")
    x = layer_inputs(4, 130, 64, 64, 128, dtype="bf16", seed=6, grads=False)
    _check_fwd(x, TOL["bf16"], "bf16 B=4 H=64 dk=64")


def test_fwd_strong_decay():
    """Half the key channels decaying by log alpha in [-5, -2.5] per token: far outside the range
    of one exp(+-G) factor over a whole chunk (|G| up to 320); the deeper decays are in
    tests/test_gpu_deep_decay.py."""
    x = strong_decay_inputs(1, 256, 2, 128, 128, dtype="bf16", seed=3, floor=-5.0)
    _check_fwd(x, TOL["bf16"], "bf16 strong decay")
    x = strong_decay_inputs(1, 256, 2, 64, 64, dtype="f32", seed=4, floor=-5.0)
    _check_fwd(x, TOL["f32"], "f32 strong decay")
    x = strong_decay_inputs(1, 256, 2, 128, 128, dtype="f32", seed=5, floor=-5.0)
    _check_fwd(x, TOL["f32"], "f32 strong decay d=128")


def test_fwd_chunk_states_checkpoint():
    """The chunk-entry checkpoint equals the oracle state after 64*c tokens (rounded to dtype)."""
    x = layer_inputs(1, 150, 2, 128, 64, dtype="bf16", seed=9, s0_std=0.05, grads=False)
    announce("chunk states")
    o, ST, ws = _run_fwd(x)
    NC = 3
    st = _states_view(ws, 1, 150, 2, 128, 64, torch.bfloat16).float().cpu().numpy()  # [B,H,NC,dv,dk]
    f = to_f64(x)
    for c in range(NC):
        if c == 0:
            ref = f["S0"]
        else:
            sub = {n: (a[:, :64 * c] if a is not None and n != "S0" else a) for n, a in f.items()}
            _, ref = orc.forward(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["b"],
                                 sub["w"], sub["S0"])
        got = np.swapaxes(st[:, :, c], -1, -2)
        assert_close(f"state entering chunk {c}", got, ref, TOL["bf16"])


def test_fwd_layer_1p3b_all_chains():
    """Full model-shaped layer (B=4, T=4096, H=16, d=128) in the launch configuration the bench
    times; the oracle recomputes every (b, h) chain, each compared on its own."""
    x = config_inputs("layer_1p3b")
    announce("layer_1p3b forward, full size, all chains")
    o, ST, _ = _run_fwd(x)
    f = to_f64(x)
    ro, rS = orc.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"])
    eo = assert_close_chains("o", to_np(o), ro, TOL["bf16"], "tok")
    eS = assert_close_chains("S_T", to_np(ST), rS, TOL["bf16"], "state")
    print(f"  worst chain: o {eo:.2e}  S_T {eS:.2e}", flush=True)


@pytest.mark.parametrize("dt,dk,dv", [("bf16", 128, 128), ("f32", 64, 128), ("bf16", 64, 64),
                                      ("f32", 128, 64)])
def test_decode_steps_vs_oracle(dt, dk, dv):
    N, H, steps = 5, 3, 6
    announce(f"decode {dt} dk={dk} dv={dv}")
    S = None
    Sref = None
    for s in range(steps):
        x = decode_inputs(s, N=N, H=H, dk=dk, dv=dv, dtype=dt)
        g = _gpu(x)
        o, S = gdr2_decode_step(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S_in=S)
        torch.cuda.synchronize()
        f = to_f64(x)
        ro, Sref = orc.decode_step(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], Sref, S_out=Sref)
        assert_close(f"decode o step {s}", to_np(o), ro, TOL[dt])
        assert_close(f"decode S step {s}", to_np(S), Sref, TOL[dt])


def test_decode_equals_chunked_forward():
    """T decode steps from S0 reproduce the chunked forward's outputs and final state."""
    x = layer_inputs(3, 70, 2, 128, 128, dtype="bf16", seed=77, s0_std=0.05, grads=False)
    announce("decode == chunked")
    o, ST, _ = _run_fwd(x)
    g = _gpu(x)
    S = g["S0"].clone()
    outs = []
    for t in range(70):
        ot, S = gdr2_decode_step(*(g[n][:, t].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")),
                                 S_in=S, S_out=S)
        outs.append(ot)
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=1)
    assert_close("decode vs chunked o", to_np(od), to_np(o), TOL["bf16"])
    assert_close("decode vs chunked S_T", to_np(S), to_np(ST), TOL["bf16"])


@pytest.mark.timeout(900)
def test_decode_full_workload_all_chains():
    """The decode workload at full size (256 sequences x 16 heads, d = 128, 1024 steps, bf16
    tokens, fp32 state updated in place in HBM, the launch the benchmark times): every chain
    against the oracle's token recurrence, o at every step and the state at eight checkpoints."""
    N, H, dk, dv, steps = DECODE["N"], DECODE["H"], DECODE["dk"], DECODE["dv"], DECODE["steps"]
    announce(f"decode full workload N={N} H={H} steps={steps}, all chains")
    S = torch.zeros((N, H, dk, dv), dtype=torch.float32, device=DEV)
    Sref = np.zeros((N, H, dk, dv))  # the oracle's state, updated in place
    worst_o = worst_S = 0.0
    for s in range(steps):
        x = decode_inputs(s, N=N, H=H, dk=dk, dv=dv, device=DEV)
        o, _ = gdr2_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S_in=S, S_out=S)
        f = {n: t.to("cpu", torch.float64).numpy() for n, t in x.items()}
        ro, Sref = orc.decode_step(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], Sref, S_out=Sref)
        # o[n, h, :] is chain (n, h) at this step: a one-token [N, 1, H, dv] view
        worst_o = max(worst_o, assert_close_chains(f"decode o step {s}", to_np(o)[:, None], ro[:, None],
                                                   TOL["bf16"], "tok"))
        if s % 128 == 127:
            worst_S = max(worst_S, assert_close_chains(f"decode S step {s}", to_np(S), Sref, TOL["bf16"],
                                                       "state"))
            print(f"  step {s + 1}: worst chain o {worst_o:.2e}  S {worst_S:.2e}", flush=True)
