"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each test compares the oracle with something other than itself: hand-worked examples, the
update written as an explicit transition-matrix product, textbook closed forms, invariants that
the pages' statements imply, the reduced rules written in their own form, and central finite
differences.  A plausible slip in the oracle (dropped term, wrong sign, transposed state, wrong
side of the erase gate, edit before decay, read-out before the update) fails at least one.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng


def _rand_inputs(B, T, H, dk, dv, seed, unit_qk=True, s0=True):
    r = rng0(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    if unit_qk:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    la = -np.log1p(np.exp(r.standard_normal((B, T, H, dk)))) * 0.3
    b = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dk))))
    w = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dv))))
    S0 = r.standard_normal((B, H, dk, dv)) * 0.5 if s0 else None
    return dict(q=q, k=k, v=v, log_alpha=la, b=b, w=w, S0=S0)


def _fwd(x):
    return orc.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"])


# ----------------------------------------------------------------------------- golden examples
def test_golden_scalar_T3():
    g = json.load(open(os.path.join(GOLD, "scalar_T3.json")))
    i = g["inputs"]
    sh = lambda a: np.array(a, dtype=np.float64).reshape(1, -1, 1, 1)
    x = dict(q=sh(i["q"]), k=sh(i["k"]), v=sh(i["v"]), log_alpha=sh(i["log_alpha"]),
             b=sh(i["b"]), w=sh(i["w"]), S0=np.full((1, 1, 1, 1), i["S0"]))
    o, ST = _fwd(x)
    e = g["expected"]
    np.testing.assert_allclose(o.ravel(), e["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST.ravel(), [e["S_T"]], rtol=0, atol=1e-12)
    gr = orc.backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], np.ones_like(o),
                      S0=x["S0"])
    for n in ("dq", "dk", "dv", "dw", "db", "dlog_alpha"):
        np.testing.assert_allclose(gr[n].ravel(), e[n], rtol=0, atol=1e-12, err_msg=n)
    np.testing.assert_allclose(gr["dS0"].ravel(), [e["dS0"]], rtol=0, atol=1e-12)


def test_golden_mat2x2_T2():
    g = json.load(open(os.path.join(GOLD, "mat2x2_T2.json")))
    i = g["inputs"]
    sh = lambda a: np.array(a, dtype=np.float64).reshape(1, 2, 1, 2)
    x = dict(q=sh(i["q"]), k=sh(i["k"]), v=sh(i["v"]), log_alpha=sh(i["log_alpha"]),
             b=sh(i["b"]), w=sh(i["w"]), S0=np.array(i["S0"]).reshape(1, 1, 2, 2))
    o, ST = _fwd(x)
    np.testing.assert_allclose(o.reshape(2, 2), g["expected"]["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST.reshape(2, 2), g["expected"]["S_T"], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- forward pins
@pytest.mark.parametrize("dk,dv,T", [(3, 2, 9), (4, 5, 16), (1, 3, 7)])
def test_bruteforce_transition_product(dk, dv, T):
    """The update exactly as printed: S_t = (I - k e^T) D S_{t-1} + k z^T, with the d_k x d_k
    transition matrix formed explicitly; o_t = S_t^T q_t."""
    x = _rand_inputs(2, T, 2, dk, dv, seed=11 + dk)
    o, ST = _fwd(x)
    for bb in range(2):
        for h in range(2):
            S = x["S0"][bb, h].copy()
            for t in range(T):
                kk, qq = x["k"][bb, t, h], x["q"][bb, t, h]
                e = x["b"][bb, t, h] * kk
                z = x["w"][bb, t, h] * x["v"][bb, t, h]
                M = (np.eye(dk) - np.outer(kk, e)) @ np.diag(np.exp(x["log_alpha"][bb, t, h]))
                S = M @ S + np.outer(kk, z)
                np.testing.assert_allclose(o[bb, t, h], S.T @ qq, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(ST[bb, h], S, rtol=1e-12, atol=1e-12)


def test_linear_attention_closed_form():
    """alpha = 1, b = 0, w = 1: the rule only adds (causal linear attention)."""
    x = _rand_inputs(2, 37, 3, 5, 4, seed=3)
    x["log_alpha"][:] = 0.0
    x["b"][:] = 0.0
    x["w"][:] = 1.0
    o, ST = _fwd(x)
    o2, ST2 = orc.la_closed_form(x["q"], x["k"], x["v"], x["S0"])
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(ST, ST2, rtol=1e-11, atol=1e-11)


def test_no_erase_closed_form():
    """b = 0: channel-wise gated linear attention as an explicit double sum."""
    x = _rand_inputs(1, 12, 2, 4, 3, seed=5)
    x["b"][:] = 0.0
    o, _ = _fwd(x)
    o2 = orc.gla_closed_form(x["q"], x["k"], x["v"], x["log_alpha"], x["w"], x["S0"])
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-11)


def test_exact_write_after_decay():
    """b = 1 and a unit key: the edit replaces exactly what the key reads after the decay, so
    S_t^T k_t = w_t . v_t; reading with q_t = k_t therefore returns the gated value.  Fails if the
    decay came after the edit or the read-out used the pre-update state."""
    x = _rand_inputs(1, 20, 2, 6, 5, seed=8)
    x["b"][:] = 1.0
    x["q"] = x["k"].copy()
    o, _ = _fwd(x)
    np.testing.assert_allclose(o, x["w"] * x["v"], rtol=1e-11, atol=1e-11)


def test_reduces_to_kda_and_gdn():
    """b = w = beta*1 is KDA; with a scalar decay as well it is Gated DeltaNet."""
    x = _rand_inputs(2, 23, 2, 5, 4, seed=21)
    beta = 1 / (1 + np.exp(-rng0(4).standard_normal((2, 23, 2))))
    x["b"] = np.repeat(beta[..., None], 5, axis=-1)
    x["w"] = np.repeat(beta[..., None], 4, axis=-1)
    o, ST = _fwd(x)
    o2, ST2 = orc.kda_forward(x["q"], x["k"], x["v"], x["log_alpha"], beta, x["S0"])
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(ST, ST2, rtol=1e-11, atol=1e-11)
    x["log_alpha"] = np.repeat(x["log_alpha"][..., :1], 5, axis=-1)
    o, ST = _fwd(x)
    o3, ST3 = orc.kda_forward(x["q"], x["k"], x["v"], x["log_alpha"], beta, x["S0"],
                              scalar_decay=True)
    np.testing.assert_allclose(o, o3, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(ST, ST3, rtol=1e-11, atol=1e-11)


def test_fast_weight_objective_minimiser():
    """S_t minimises f(S) = ||S - Sbar||_F^2 - 2 <S^T k, z - Sbar^T e> (forum summary, section
    "Gated Delta Rule-2", fast-weight view).  f is quadratic with Hessian 2I, so S_t is the
    minimiser iff f(S_t + P) - f(S_t) = ||P||_F^2 for every P."""
    x = _rand_inputs(1, 6, 1, 4, 3, seed=31)
    r = rng0(9)
    for t in range(1, 6):
        pre = {n: (a[:, :t] if a is not None and a.ndim == 4 and n != "S0" else a)
               for n, a in x.items()}
        cur = {n: (a[:, :t + 1] if a is not None and a.ndim == 4 and n != "S0" else a)
               for n, a in x.items()}
        _, Sprev = _fwd(pre)
        _, St = _fwd(cur)
        Sprev, St = Sprev[0, 0], St[0, 0]
        kk, bb, ww, vv = (x[n][0, t, 0] for n in ("k", "b", "w", "v"))
        Sbar = np.diag(np.exp(x["log_alpha"][0, t, 0])) @ Sprev
        e, z = bb * kk, ww * vv

        def f(S):
            return np.sum((S - Sbar) ** 2) - 2 * np.dot(S.T @ kk, z - Sbar.T @ e)

        for _ in range(3):
            P = r.standard_normal(St.shape)
            assert abs(f(St + P) - f(St) - np.sum(P ** 2)) < 1e-9


def test_scale_invariance_and_linearity():
    """o and S_T depend on (w, v) only through w . v, and are jointly linear in (v, S0)."""
    x = _rand_inputs(1, 15, 2, 4, 3, seed=41)
    o, ST = _fwd(x)
    y = dict(x)
    y["w"] = x["w"] * 2.5
    y["v"] = x["v"] / 2.5
    o2, ST2 = _fwd(y)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-11)
    x2 = _rand_inputs(1, 15, 2, 4, 3, seed=42)
    y = dict(x)
    y["v"] = 2.0 * x["v"] - 3.0 * x2["v"]
    y["S0"] = 2.0 * x["S0"] - 3.0 * x2["S0"]
    z = dict(x)
    z["v"], z["S0"] = x2["v"], x2["S0"]
    oy, Sy = _fwd(y)
    oz, Sz = _fwd(z)
    np.testing.assert_allclose(oy, 2 * o - 3 * oz, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(Sy, 2 * ST - 3 * Sz, rtol=1e-10, atol=1e-10)


def test_split_sequence_handoff():
    """Running [0, t1) then [t1, T) with the final state handed over equals one run, forward and
    backward (dS0 of the second half is the dS_T of the first)."""
    x = _rand_inputs(1, 70, 2, 4, 3, seed=51)
    dO = rng0(52).standard_normal(x["v"].shape)
    o, ST = _fwd(x)
    g = orc.backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO, S0=x["S0"])
    t1 = 29
    A = {n: (a[:, :t1] if n != "S0" else a) for n, a in x.items()}
    Bh = {n: (a[:, t1:] if n != "S0" else a) for n, a in x.items()}
    oA, SA = _fwd(A)
    Bh["S0"] = SA
    oB, SB = _fwd(Bh)
    np.testing.assert_allclose(np.concatenate([oA, oB], axis=1), o, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(SB, ST, rtol=1e-11, atol=1e-11)
    gB = orc.backward(Bh["q"], Bh["k"], Bh["v"], Bh["log_alpha"], Bh["b"], Bh["w"],
                      dO[:, t1:], S0=SA)
    gA = orc.backward(A["q"], A["k"], A["v"], A["log_alpha"], A["b"], A["w"], dO[:, :t1],
                      S0=x["S0"], dST=gB["dS0"])
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        np.testing.assert_allclose(np.concatenate([gA[n], gB[n]], axis=1), g[n], rtol=1e-10,
                                   atol=1e-10, err_msg=n)
    np.testing.assert_allclose(gA["dS0"], g["dS0"], rtol=1e-10, atol=1e-10)


def test_decode_matches_token_steps():
    """The decode step is one token of the recurrence, applied in place."""
    x = _rand_inputs(3, 9, 2, 5, 4, seed=61)
    o, ST = _fwd(x)
    S = x["S0"]
    for t in range(9):
        ot, S = orc.decode_step(*(x[n][:, t] for n in ("q", "k", "v", "log_alpha", "b", "w")),
                                S_in=S)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, ST, rtol=1e-12, atol=1e-12)
    o0, S0 = orc.decode_step(*(x[n][:, 0] for n in ("q", "k", "v", "log_alpha", "b", "w")))
    y = dict(x)
    y["S0"] = None
    oy, _ = _fwd({n: (a[:, :1] if n != "S0" else a) for n, a in y.items()})
    np.testing.assert_allclose(o0, oy[:, 0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- backward pins
def _loss(x, dO, dST):
    o, ST = _fwd(x)
    return float(np.sum(o * dO) + np.sum(ST * dST))


@pytest.mark.parametrize("T,dk,dv", [(1, 1, 1), (2, 3, 2), (5, 4, 3), (7, 1, 2), (17, 3, 3),
                                     (66, 2, 2)])
def test_backward_finite_differences(T, dk, dv):
    """Central differences (h = 1e-6) in fp64 for every input, with dO and dS_T both random."""
    x = _rand_inputs(1, T, 2, dk, dv, seed=100 + T + dk)
    r = rng0(200 + T)
    dO = r.standard_normal(x["v"].shape)
    dST = r.standard_normal(x["S0"].shape)
    g = orc.backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO, S0=x["S0"],
                     dST=dST)
    names = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "b": "db", "w": "dw",
             "S0": "dS0"}
    h = 1e-6
    for n, gn in names.items():
        fd = np.zeros_like(x[n])
        flat = fd.reshape(-1)
        # all entries for small tensors, a random subset otherwise
        idx = np.arange(flat.size) if flat.size <= 64 else r.choice(flat.size, 64, replace=False)
        for j in idx:
            xp = {m: (a.copy() if a is not None else None) for m, a in x.items()}
            xm = {m: (a.copy() if a is not None else None) for m, a in x.items()}
            xp[n].reshape(-1)[j] += h
            xm[n].reshape(-1)[j] -= h
            flat[j] = (_loss(xp, dO, dST) - _loss(xm, dO, dST)) / (2 * h)
        an = g[gn].reshape(-1)[idx]
        scale = max(1.0, np.max(np.abs(flat[idx])))
        assert np.max(np.abs(an - flat[idx])) / scale < 1e-6, (n, np.max(np.abs(an - flat[idx])))


def test_backward_linear_attention_closed_form():
    x = _rand_inputs(2, 40, 2, 5, 4, seed=7)
    x["log_alpha"][:] = 0.0
    x["b"][:] = 0.0
    x["w"][:] = 1.0
    r = rng0(8)
    dO = r.standard_normal(x["v"].shape)
    dST = r.standard_normal(x["S0"].shape)
    g = orc.backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO, S0=x["S0"],
                     dST=dST)
    c = orc.la_backward_closed_form(x["q"], x["k"], x["v"], dO, S0=x["S0"], dST=dST)
    for n in ("dq", "dk", "dv", "dS0"):
        np.testing.assert_allclose(g[n], c[n], rtol=1e-10, atol=1e-10, err_msg=n)


def test_tied_gate_chain_rules():
    """With b = w = beta*1 the KDA gradient in beta is sum_i db_i + sum_j dw_j; with one decay per
    token as well, the Gated DeltaNet gradient in that log-decay is sum_i dlog_alpha_i.  The
    reference gradients are finite differences of the reduced rules written in their own form."""
    B, T, H, dk, dv = 1, 9, 1, 3, 2
    x = _rand_inputs(B, T, H, dk, dv, seed=71)
    r = rng0(72)
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    ell = -np.log1p(np.exp(r.standard_normal((B, T, H)))) * 0.3
    la = np.repeat(ell[..., None], dk, axis=-1)
    dO = r.standard_normal((B, T, H, dv))
    bb = np.repeat(beta[..., None], dk, axis=-1)
    ww = np.repeat(beta[..., None], dv, axis=-1)
    g = orc.backward(x["q"], x["k"], x["v"], la, bb, ww, dO, S0=x["S0"])

    def L(beta_, ell_):
        o, _ = orc.kda_forward(x["q"], x["k"], x["v"], np.repeat(ell_[..., None], dk, axis=-1),
                               beta_, x["S0"], scalar_decay=True)
        return float(np.sum(o * dO))

    h = 1e-6
    for t in range(T):
        bp, bm = beta.copy(), beta.copy()
        bp[0, t, 0] += h
        bm[0, t, 0] -= h
        fd = (L(bp, ell) - L(bm, ell)) / (2 * h)
        assert abs(fd - (g["db"][0, t, 0].sum() + g["dw"][0, t, 0].sum())) < 1e-6
        ep, em = ell.copy(), ell.copy()
        ep[0, t, 0] += h
        em[0, t, 0] -= h
        fd = (L(beta, ep) - L(beta, em)) / (2 * h)
        assert abs(fd - g["dlog_alpha"][0, t, 0].sum()) < 1e-6


# ---- output epilogue (RMS normalisation x weight x SiLU gate)
def test_out_gate_special_values():
    """Hand-checkable rows: a constant row c normalises to c / sqrt(c^2 + eps); a zero gate
    closes the output; a large gate passes silu(g) ~ g; the row scale cancels (up to eps)."""
    d = 8
    w = np.linspace(0.5, 2.0, d)
    c, eps = 3.0, 1e-3
    o = np.full((1, d), c)
    g = np.full((1, d), 40.0)
    y = orc.out_gate_forward(o, g, w, eps)
    np.testing.assert_allclose(y[0], c / np.sqrt(c * c + eps) * w * 40.0, rtol=1e-12)
    assert np.all(orc.out_gate_forward(o, np.zeros((1, d)), w, eps) == 0.0)
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, d))
    g = rng.standard_normal((5, d))
    np.testing.assert_allclose(orc.out_gate_forward(o * 7.0, g, w, 1e-14),
                               orc.out_gate_forward(o, g, w, 1e-14), rtol=1e-9)
    # silu(g) = g * sigmoid(g): at g = ln(3), sigmoid = 3/4
    g1 = np.full((1, d), np.log(3.0))
    y1 = orc.out_gate_forward(np.ones((1, d)), g1, np.ones(d), 0.0 + 1e-300)
    np.testing.assert_allclose(y1[0], np.log(3.0) * 0.75, rtol=1e-12)


def test_out_gate_backward_finite_differences():
    rng = np.random.default_rng(5)
    R, d, eps = 3, 6, 1e-2
    o = rng.standard_normal((R, d))
    g = rng.standard_normal((R, d))
    w = rng.standard_normal(d)
    dy = rng.standard_normal((R, d))
    gr = orc.out_gate_backward(o, g, w, eps, dy)
    L = lambda o_, g_, w_: float(np.sum(dy * orc.out_gate_forward(o_, g_, w_, eps)))
    h = 1e-6
    for name, x in (("do", o), ("dg", g), ("dweight", w)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [o, g, w]
            args_m = [o, g, w]
            pos = {"do": 0, "dg": 1, "dweight": 2}[name]
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (L(*args_p) - L(*args_m)) / (2 * h)
        err = np.max(np.abs(num - gr[name])) / np.max(np.abs(num))
        assert err < 1e-7, (name, err)


# ---- fused prologue (L2-normalised q, k; sigmoid gates; softplus decay)
def test_prologue_special_values():
    """Closed forms: softplus(0) = ln 2, softplus(ln(e - 1)) = 1, softplus(a) -> a for large a;
    sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4; (3, 4) normalises to (3, 4) / sqrt(25 + eps); a
    normalised row has unit norm as eps -> 0 and does not change when the row is scaled."""
    c, eps = 0.7, 1e-3
    a = np.array([0.0, np.log(np.e - 1.0), 60.0])
    q = np.array([[3.0, 4.0]])
    p = orc.prologue_forward(q, q, a, np.array([0.0, np.log(3.0)]), np.array([0.0]), c, eps)
    np.testing.assert_allclose(p["log_alpha"], [-c * np.log(2.0), -c, -c * 60.0], rtol=1e-12)
    np.testing.assert_allclose(p["b"], [0.5, 0.75], rtol=1e-12)
    np.testing.assert_allclose(p["w"], [0.5], rtol=1e-12)
    np.testing.assert_allclose(p["q"], [[3.0 / np.sqrt(25 + eps), 4.0 / np.sqrt(25 + eps)]],
                               rtol=1e-12)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5, 16))
    z = np.zeros(1)
    p1 = orc.prologue_forward(x, x, z, z, z, 1.0, 1e-300)
    np.testing.assert_allclose(np.linalg.norm(p1["k"], axis=-1), 1.0, rtol=1e-12)
    p2 = orc.prologue_forward(x * 9.0, x, z, z, z, 1.0, 1e-300)
    np.testing.assert_allclose(p2["q"], p1["q"], rtol=1e-12)


@pytest.mark.parametrize("scalar", [False, True])
def test_prologue_backward_finite_differences(scalar):
    """The layer fed through the prologue: central differences of <o, dO> + <S_T, dS_T> with
    respect to every pre-activation, against prologue_backward(backward(prologue_forward(.)));
    ``scalar`` uses one gate value per (token, head), broadcast over the channels."""
    B, T, H, dk, dv = 1, 6, 2, 3, 2
    c, eps = 0.8, 1e-2
    r = rng0(310 + scalar)
    raw = {"q": r.standard_normal((B, T, H, dk)), "k": r.standard_normal((B, T, H, dk)),
           "v": r.standard_normal((B, T, H, dv))}
    gshape = (B, T, H) if scalar else None
    raw["a"] = r.standard_normal(gshape or (B, T, H, dk))
    raw["b"] = r.standard_normal(gshape or (B, T, H, dk))
    raw["w"] = r.standard_normal(gshape or (B, T, H, dv))
    S0 = r.standard_normal((B, H, dk, dv)) * 0.3
    dO = r.standard_normal((B, T, H, dv))
    dST = r.standard_normal((B, H, dk, dv))

    def widen(x, d):
        return np.repeat(x[..., None], d, axis=-1) if scalar else x

    def post(x):
        p = orc.prologue_forward(x["q"], x["k"], x["a"], x["b"], x["w"], c, eps)
        return p["q"], p["k"], widen(p["log_alpha"], dk), widen(p["b"], dk), widen(p["w"], dv)

    def L(x):
        q, k, la, b, w = post(x)
        o, ST = orc.forward(q, k, x["v"], la, b, w, S0)
        return float(np.sum(o * dO) + np.sum(ST * dST))

    q, k, la, b, w = post(raw)
    g = orc.backward(q, k, raw["v"], la, b, w, dO, S0=S0, dST=dST)
    if scalar:
        g = dict(g, dlog_alpha=g["dlog_alpha"].sum(-1), db=g["db"].sum(-1), dw=g["dw"].sum(-1))
    gr = orc.prologue_backward(raw["q"], raw["k"], raw["a"], raw["b"], raw["w"], c, eps, g)
    gr["dv"] = g["dv"]
    h = 1e-6
    for n, gn in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("a", "dlog_alpha"), ("b", "db"),
                  ("w", "dw")):
        num = np.zeros_like(raw[n])
        for idx in np.ndindex(raw[n].shape):
            xp = {m: t.copy() for m, t in raw.items()}
            xm = {m: t.copy() for m, t in raw.items()}
            xp[n][idx] += h
            xm[n][idx] -= h
            num[idx] = (L(xp) - L(xm)) / (2 * h)
        err = np.max(np.abs(num - gr[gn])) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-7, (n, err)
