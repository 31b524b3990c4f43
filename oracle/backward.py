"""Gradients of the token recurrence (reverse-mode), float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages give the forward pass only (they name chunkwise-parallel training but print
no backward), so this is the derivative of the plain definition used by the forward
oracle. Per token, with X = Diag(alpha_t) S_{t-1} and u = w_t - X^T b_t:

    S_t = X + a_t u^T,   o_t = S_t^T q_t

and, with G = dL/dS_t (the gradient from the later tokens plus q_t do_t^T):

    dq_t = S_t do_t                        dw = G^T a
    da   = G u                             db = -X dw
    dX   = G - b dw^T                      dalpha = rowsum(dX . S_{t-1})
    dL/dS_{t-1} = Diag(alpha_t) dX

then the chain rule through each variant's (a, b, w, alpha) map (FG2-GDN reading
notes, section 2.2 eq. (11) and section 2.3 eq. (13); GDN2-stability page, eq. (1)).
Pinned by central finite differences in tests/test_oracle_backward.py.

Inputs as for oracle.forward (library layouts, state [B, H, dk, dv]); d_o has the
shape of o, ds_final (optional) the shape of the state. Returns a dict of float64
gradients named after the inputs (dq, dk, dv, dalpha, dbeta, dbeta_v, dj, deta, ds0).
DeltaProduct (DeltaProduct summary, "Approach") runs as its sequence of n_h
Householder sub-steps per token (a = k_i, b = beta_i k_i, w = beta_i v_i, the gate
as alpha at the first sub-step, q read after the last), through the same loop.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _maps(inp):
    """Per-variant (a, b, w, alpha) as [B, T, H, d] float64 arrays."""
    var = inp["variant"]
    k, v = _f64(inp["k"]), _f64(inp["v"])
    dk = k.shape[-1]
    if var == "fg2":
        s = np.sqrt(_f64(inp["beta"]))
        sv = np.sqrt(_f64(inp["beta_v"])) if inp.get("beta_v") is not None else s
        return s * k, s * k, sv * v, _f64(inp["alpha"])
    if var in ("kda", "gdn"):
        s = np.sqrt(_f64(inp["beta"]))[..., None]
        al = _f64(inp["alpha"])
        if var == "gdn":
            al = np.repeat(al[..., None], dk, axis=-1)
        return s * k, s * k, s * v, al
    if var == "asym":
        e = _f64(inp["eta"])[..., None]
        return k, e * _f64(inp["j"]), e * v, _f64(inp["alpha"])
    raise ValueError(f"no backward for variant {var!r}")


def _deltaproduct(inp, d_o, s0, ds_final):
    k, v = _f64(inp["k"]), _f64(inp["v"])          # [B, T, H, n_h, d]
    beta, gate = _f64(inp["beta"]), _f64(inp["alpha"])
    B, T, H, n, dk = k.shape
    dv = v.shape[-1]
    flat = lambda x: np.moveaxis(x, 3, 2).reshape(B, T * n, H, x.shape[-1])  # noqa: E731
    a = flat(k)
    bsub = flat(beta[..., None] * k)
    w = flat(beta[..., None] * v)
    al = np.ones((B, T, n, H, dk))
    al[:, :, 0] = gate[..., None]
    al = al.reshape(B, T * n, H, dk)
    q = np.zeros((B, T, n, H, dk))
    q[:, :, n - 1] = _f64(inp["q"])
    do = np.zeros((B, T, n, H, dv))
    do[:, :, n - 1] = _f64(d_o)
    sub = {"variant": "sub", "a": a, "b": bsub, "w": w, "alpha": al,
           "q": q.reshape(B, T * n, H, dk)}
    g = _steps(sub, do.reshape(B, T * n, H, dv), s0, ds_final)
    unflat = lambda x: np.moveaxis(x.reshape(B, T, n, H, x.shape[-1]), 2, 3)  # noqa: E731
    da, db, dw, dal = unflat(g["da"]), unflat(g["db"]), unflat(g["dw"]), unflat(g["dal"])
    return {"dq": unflat(g["dq"])[:, :, :, n - 1], "ds0": g["ds0"],
            "dk": da + beta[..., None] * db, "dv": beta[..., None] * dw,
            "dbeta": np.sum(k * db, -1) + np.sum(v * dw, -1),
            "dalpha": np.sum(dal[:, :, :, 0], -1)}


def backward(inp: dict, d_o, s0=None, ds_final=None) -> dict:
    if inp["variant"] == "deltaproduct":
        return _deltaproduct(inp, d_o, s0, ds_final)
    a, b, w, al = _maps(inp)
    g = _steps({"a": a, "b": b, "w": w, "alpha": al, "q": _f64(inp["q"])}, d_o, s0, ds_final)
    da, db, dw, dal, dq = g["da"], g["db"], g["dw"], g["dal"], g["dq"]
    return _chain(inp, da, db, dw, dal, dq, g["ds0"])


def _steps(st: dict, d_o, s0, ds_final) -> dict:
    """The reverse sweep over steps given per-step (a, b, w, alpha) and q."""
    a, b, w, al, q = st["a"], st["b"], st["w"], st["alpha"], st["q"]
    do = _f64(d_o)
    B, T, H, dk = a.shape
    dv = w.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0).copy()

    # forward, keeping the state before every token
    prev = np.empty((T, B, H, dk, dv))
    for t in range(T):
        prev[t] = S
        X = al[:, t][..., None] * S
        u = w[:, t] - np.einsum("bhkv,bhk->bhv", X, b[:, t])
        S = X + a[:, t][..., None] * u[..., None, :]

    G = np.zeros((B, H, dk, dv)) if ds_final is None else _f64(ds_final).copy()
    da = np.zeros_like(a)
    db = np.zeros_like(b)
    dw = np.zeros_like(w)
    dal = np.zeros_like(al)
    dq = np.zeros_like(q)
    for t in reversed(range(T)):
        Sp = prev[t]
        X = al[:, t][..., None] * Sp
        u = w[:, t] - np.einsum("bhkv,bhk->bhv", X, b[:, t])
        St = X + a[:, t][..., None] * u[..., None, :]
        dq[:, t] = np.einsum("bhkv,bhv->bhk", St, do[:, t])
        G = G + q[:, t][..., None] * do[:, t][..., None, :]
        dw[:, t] = np.einsum("bhkv,bhk->bhv", G, a[:, t])
        da[:, t] = np.einsum("bhkv,bhv->bhk", G, u)
        db[:, t] = -np.einsum("bhkv,bhv->bhk", X, dw[:, t])
        dX = G - b[:, t][..., None] * dw[:, t][..., None, :]
        dal[:, t] = np.sum(dX * Sp, axis=-1)
        G = al[:, t][..., None] * dX

    return {"da": da, "db": db, "dw": dw, "dal": dal, "dq": dq, "ds0": G}


def _chain(inp, da, db, dw, dal, dq, ds0) -> dict:
    out = {"dq": dq, "ds0": ds0}
    var = inp["variant"]
    k, v = _f64(inp["k"]), _f64(inp["v"])
    if var == "fg2":
        beta = _f64(inp["beta"])
        s = np.sqrt(beta)
        out["dk"] = s * (da + db)
        out["dalpha"] = dal
        if inp.get("beta_v") is not None:
            sv = np.sqrt(_f64(inp["beta_v"]))
            out["dv"] = sv * dw
            out["dbeta_v"] = v * dw / (2.0 * sv)
            out["dbeta"] = k * (da + db) / (2.0 * s)
        else:
            out["dv"] = s * dw
            out["dbeta"] = (k * (da + db) + v * dw) / (2.0 * s)
    elif var in ("kda", "gdn"):
        beta = _f64(inp["beta"])
        s = np.sqrt(beta)
        out["dk"] = s[..., None] * (da + db)
        out["dv"] = s[..., None] * dw
        out["dbeta"] = (np.sum(k * (da + db), -1) + np.sum(v * dw, -1)) / (2.0 * s)
        out["dalpha"] = dal if var == "kda" else np.sum(dal, -1)
    else:  # asym
        e = _f64(inp["eta"])
        j = _f64(inp["j"])
        out["dk"] = da
        out["dj"] = e[..., None] * db
        out["dv"] = e[..., None] * dw
        out["deta"] = np.sum(j * db, -1) + np.sum(v * dw, -1)
        out["dalpha"] = dal
    return out
