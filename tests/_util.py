"""Helpers shared by the GPU parity tests."""
import sys

import numpy as np

# Tolerances: normwise max relative error per output tensor, max|gpu - ref| / max|ref|.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def normwise(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - ref)) / den)


def announce(msg):
    """Name the case before a GPU step, so a crash still shows which one ran."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().to("cpu").double().numpy()


def assert_close(name, x, ref, tol):
    e = normwise(x, ref)
    assert np.all(np.isfinite(np.asarray(x, dtype=np.float64))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: normwise error {e:.3e} > {tol:.1e}"
    return e


def assert_close_chains(name, x, ref, tol, layout):
    """Normwise error of every (batch, head) chain on its own: max|x - ref| / max|ref| over one
    chain's elements, so that an error confined to a few chains, tokens or channels cannot hide
    under the scale of the whole tensor.  layout: "tok" for [B, T, H, ...] tensors, "state" for
    [B, H, dk, dv].  Returns the worst chain's error."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, f"{name}: shape {x.shape} vs {ref.shape}"
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    if layout == "tok":
        x = np.moveaxis(x, 2, 1)        # [B, H, T, ...]
        ref = np.moveaxis(ref, 2, 1)
    B, H = x.shape[:2]
    d = np.abs(x - ref).reshape(B, H, -1).max(-1)
    m = np.abs(ref).reshape(B, H, -1).max(-1)
    e = np.where(m > 0, d / np.where(m > 0, m, 1.0), d)
    b, h = np.unravel_index(int(e.argmax()), e.shape)
    assert e[b, h] <= tol, f"{name}: chain (b={b}, h={h}) normwise error {e[b, h]:.3e} > {tol:.1e}"
    return float(e.max())
