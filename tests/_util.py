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
