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


def assert_close_rows(name, x, ref, tol, layout, floor=0.1):
    """Row-wise check for the fp32 path, where the tolerance is tight enough to be applied per
    row: every (batch, token, head) row of a [B, T, H, ...] tensor ("tok"), or every key row of a
    [B, H, dk, dv] state ("state"), must satisfy max|x - ref| <= tol * max(max|ref row|,
    floor * max|ref chain|).  A row at least `floor` of its chain's scale must match to `tol` of
    itself; a smaller row to tol * floor of the chain's scale.  The floor is there because fp32
    cannot do better for small rows under deep decay: the cumulative log decay G of a chunk (up to
    a few hundred in magnitude) carries an absolute rounding error of about |G| * 2^-24, so every
    decay factor exp(G_r - G_s) does so relatively, about 1e-5 of the chain's scale in the
    gradients' terms, and a row that is a small remainder of such terms cannot be more accurate
    than that (measured: 7e-6 of the chain scale on a dlog alpha row at 0.7 % of it, with
    log alpha in [-4.4, -3.2] per token).  Returns the worst row's error in those units."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, f"{name}: shape {x.shape} vs {ref.shape}"
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    if layout == "tok":
        x = np.moveaxis(x, 2, 1)        # [B, H, T, ...]
        ref = np.moveaxis(ref, 2, 1)
    B, H = x.shape[:2]
    x = x.reshape(B, H, x.shape[2], -1)
    ref = ref.reshape(B, H, ref.shape[2], -1)
    d = np.abs(x - ref).max(-1)                        # [B, H, rows]
    m = np.abs(ref).max(-1)
    chain = m.max(-1, keepdims=True)
    den = np.maximum(m, floor * chain)
    e = np.where(den > 0, d / np.where(den > 0, den, 1.0), d)
    b, h, rr = np.unravel_index(int(e.argmax()), e.shape)
    assert e[b, h, rr] <= tol, (f"{name}: row (b={b}, h={h}, row={rr}) error {e[b, h, rr]:.3e} > "
                                f"{tol:.1e}")
    return float(e.max())
