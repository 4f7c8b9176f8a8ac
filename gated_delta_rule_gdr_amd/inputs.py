"""Seeded synthetic inputs for the Gated Delta Rule-2 layer.

This module only draws random numbers and shapes them into the input recipe; it holds none of the
layer's arithmetic.  Both the HIP path and the oracle consume exactly the tensors made here (the
oracle receives them widened to float64), so low-precision rounding happens once, here, by
round-to-nearest-even casts.

Recipe (the pages' layer shape and value structure, synthetic values):
  * q, k ~ N(0, 1), then L2-normalised over the key channels of each (token, head) -- the block
    normalises queries and keys (ainews.random.gg article on Gated DeltaNet-2, section "Block
    design and hybrid model");
  * v ~ N(0, 1);
  * log alpha = -softplus(N(0, 1)) * 0.1, one value per key channel, kept in fp32;
  * b = sigmoid(N(0, 1)) per key channel, w = sigmoid(N(0, 1)) per value channel -- the gates are
    sigmoid outputs in [0, 1] (same article, section "Gated Delta Rule-2: two gates instead of one");
  * S0 = 0, or N(0, std^2) in fp32 when ``s0_std`` > 0;  dO ~ N(0, 1);  dS_T ~ N(0, 1) on request.
Draw order per call: q, k, v, log alpha, b, w, S0, dO, dS_T, from one ``torch.Generator`` seeded
with ``seed``.

Scalar gates (``scalar`` containing "b", "w" and/or "a"): that gate -- b, w or log alpha -- is
drawn once per (batch, token, head), same distribution, and has shape [B, T, H] (the gate-shape
variants of the ablation in the forum summary on zhichai.net, section "Ablation: the erase gate
matters more", and Gated DeltaNet's scalar decay).

Pre-activations (``raw=True``, for the fused prologue): the same draws without their
activations -- q, k ~ N(0, 1) unnormalised, a ~ N(0, 1) in the log alpha slot (fp32), b, w ~ N(0, 1)
-- which the prologue maps to the recipe above (q/|q|, -c softplus(a), sigmoid(b), sigmoid(w)).

Variants (tied-gate reductions):
  * ``"kda"``: beta = sigmoid(N(0,1)) per (batch, token, head), b = w = beta broadcast;
  * ``"gdn"``: as ``"kda"`` plus one log alpha per (batch, token, head) broadcast over channels;
  * ``"la"``: log alpha = 0, b = 0, w = 1 exactly (plain causal linear attention).
"""
from __future__ import annotations

import torch

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}

# The workloads: name -> shape / dtype / pass / seed.  dtype is the dtype of q, k, v, b, w, o and
# of the bf16/fp32 gradients; log alpha and every state are fp32.
CONFIGS = {
    "pr1_fp32": dict(B=1, T=256, H=1, dk=64, dv=64, dtype="f32", s0_std=0.0, seed=1000,
                     passes="fwd"),
    "layer_1p3b": dict(B=4, T=4096, H=16, dk=128, dv=128, dtype="bf16", s0_std=0.0, seed=1001,
                       passes="fwd+bwd"),
    "long_ctx": dict(B=1, T=32768, H=16, dk=128, dv=128, dtype="bf16", s0_std=0.02, seed=1002,
                     passes="fwd+bwd"),
    "tied_kda": dict(B=2, T=2048, H=16, dk=128, dv=128, dtype="bf16", s0_std=0.0, seed=1003,
                     passes="fwd+bwd", variant="kda"),
    "tied_gdn": dict(B=2, T=2048, H=16, dk=128, dv=128, dtype="bf16", s0_std=0.0, seed=1003,
                     passes="fwd+bwd", variant="gdn"),
    "tied_la": dict(B=2, T=2048, H=16, dk=128, dv=128, dtype="bf16", s0_std=0.0, seed=1003,
                    passes="fwd+bwd", variant="la"),
}

DECODE = dict(N=256, H=16, dk=128, dv=128, steps=1024, dtype="bf16", seed_base=2000)


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def layer_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, variant="gdr2", s0_std=0.0,
                 grads=True, dST=False, device="cpu", decay_scale=0.1, scalar="", raw=False):
    """Draw one batch of layer inputs.  Returns a dict of tensors on ``device``:
    q, k, b: [B,T,H,dk] (dtype); v, w, dO: [B,T,H,dv] (dtype); log_alpha: [B,T,H,dk] fp32;
    S0: [B,H,dk,dv] fp32 or None; dST: [B,H,dk,dv] fp32 or None."""
    dt = _DT[dtype]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = _normal((B, T, H, dk), g, device)
    if not raw:
        q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    k = _normal((B, T, H, dk), g, device)
    if not raw:
        k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    v = _normal((B, T, H, dv), g, device)
    if raw:
        if variant != "gdr2":
            raise ValueError("raw inputs are drawn for the plain recipe only")
        la = _normal((B, T, H) if "a" in scalar else (B, T, H, dk), g, device)
        b = _normal((B, T, H) if "b" in scalar else (B, T, H, dk), g, device).to(dt)
        w = _normal((B, T, H) if "w" in scalar else (B, T, H, dv), g, device).to(dt)
    elif variant == "gdn":
        la = -torch.nn.functional.softplus(_normal((B, T, H, 1), g, device)) * decay_scale
        la = la.expand(B, T, H, dk).contiguous()
    elif variant == "la":
        la = torch.zeros((B, T, H, dk), device=device)
    elif "a" in scalar:
        la = -torch.nn.functional.softplus(_normal((B, T, H), g, device)) * decay_scale
    else:
        la = -torch.nn.functional.softplus(_normal((B, T, H, dk), g, device)) * decay_scale
    if raw:
        pass
    elif variant in ("kda", "gdn"):
        beta = torch.sigmoid(_normal((B, T, H, 1), g, device)).to(dt)
        b = beta.expand(B, T, H, dk).contiguous()
        w = beta.expand(B, T, H, dv).contiguous()
    elif variant == "la":
        b = torch.zeros((B, T, H, dk), device=device, dtype=dt)
        w = torch.ones((B, T, H, dv), device=device, dtype=dt)
    else:
        b = torch.sigmoid(_normal((B, T, H) if "b" in scalar else (B, T, H, dk), g, device)).to(dt)
        w = torch.sigmoid(_normal((B, T, H) if "w" in scalar else (B, T, H, dv), g, device)).to(dt)
    S0 = (_normal((B, H, dk, dv), g, device) * s0_std) if s0_std > 0 else None
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=la.float().contiguous(), b=b, w=w,
               S0=S0)
    if grads:
        out["dO"] = _normal((B, T, H, dv), g, device).to(dt)
        out["dST"] = _normal((B, H, dk, dv), g, device) if dST else None
    return out


def config_inputs(name, device="cpu", **override):
    """Inputs of one named workload (see CONFIGS); keyword overrides change shape or seed."""
    c = dict(CONFIGS[name])
    c.update(override)
    return layer_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], dtype=c["dtype"],
                        seed=c["seed"], variant=c.get("variant", "gdr2"), s0_std=c["s0_std"],
                        grads="bwd" in c["passes"], device=device)


def decode_inputs(step, N=DECODE["N"], H=DECODE["H"], dk=DECODE["dk"], dv=DECODE["dv"],
                  dtype=DECODE["dtype"], seed_base=DECODE["seed_base"], device="cpu", scalar="",
                  raw=False):
    """Per-step decode token inputs (one token for each of N sequences x H heads), same recipe as
    the layer inputs, seeded with seed_base + step.  q, k, b, log_alpha: [N,H,dk]; v, w: [N,H,dv]
    (a scalar gate: [N,H])."""
    x = layer_inputs(N, 1, H, dk, dv, dtype=dtype, seed=seed_base + step, grads=False,
                     device=device, scalar=scalar, raw=raw)
    return {n: x[n][:, 0].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}


def strong_decay_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, device="cpu", floor=-6.0):
    """Layer inputs whose key channels decay fast: log alpha = floor * U(0.5, 1) per token on a
    random half of the channels (at floor = -5: log alpha in [-5, -2.5], alpha ~ 0.007..0.08 per
    token), the usual recipe elsewhere."""
    x = layer_inputs(B, T, H, dk, dv, dtype=dtype, seed=seed, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 77)
    mask = torch.rand((B, 1, H, dk), generator=g, device=device) < 0.5
    fast = floor * (0.5 + 0.5 * torch.rand((B, T, H, dk), generator=g, device=device))
    x["log_alpha"] = torch.where(mask, fast, x["log_alpha"]).contiguous()
    return x


def deep_decay_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, device="cpu", lo=-30.0, hi=-6.0,
                      deep_chunk=1, s0_std=0.05, dST=True):
    """Layer inputs with decays far past exp(-88) across a 16-token block.  Per (batch, head,
    channel) a random half of the key channels draws log alpha ~ U(lo, hi) per token, a random
    quarter has no decay at all (log alpha = 0 exactly) and the rest keep the usual recipe; every
    channel of chunk ``deep_chunk`` (tokens 64 c .. 64 c + 63, if the sequence has them) decays by
    log alpha = -20 per token.  alpha may be any value in (0, 1] (the decay is a per-channel
    diagonal gate; ainews.random.gg article on Gated DeltaNet-2, section "Gated Delta Rule-2: two
    gates instead of one"), so a trained decay branch can saturate like this."""
    x = layer_inputs(B, T, H, dk, dv, dtype=dtype, seed=seed, device=device, s0_std=s0_std, dST=dST)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 91)
    u = torch.rand((B, 1, H, dk), generator=g, device=device)
    fast = lo + (hi - lo) * torch.rand((B, T, H, dk), generator=g, device=device)
    la = torch.where(u < 0.5, fast, x["log_alpha"])
    la = torch.where(u > 0.75, torch.zeros_like(la), la)
    c0, c1 = 64 * deep_chunk, min(64 * deep_chunk + 64, T)
    if c0 < T:
        la[:, c0:c1] = -20.0
    x["log_alpha"] = la.contiguous()
    return x


def to_f64(x):
    """float64 numpy copies of every tensor in ``x`` (None stays None): what the oracle consumes."""
    return {n: (None if t is None else t.detach().to("cpu", torch.float64).numpy())
            for n, t in x.items()}
