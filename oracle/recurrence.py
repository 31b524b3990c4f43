"""Token-by-token float64 recurrences, one per model on the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every function takes float arrays laid out [B, T, H, ...] (the library's layout),
upcasts them to float64, and loops over tokens; each step is the rank-1 update
exactly as the cited passage writes it. Batch and heads are independent and
are processed together by numpy broadcasting. Each returns (o, S_T):
    o    [B, T, H, dv]  the read-out after each token's update
    S_T  the state after the last token
The state of every left-multiplied model is S in R^{dk x dv} ([B, H, dk, dv]),
read out as o_t = S_t^T q_t. GDN2 keeps the pages' own convention (S in
R^{dv x dk}, right-multiplied transition, o_t = S_t q_t); ``forward`` maps it to
the library's [dk, dv] state by a transpose.

Readings taken where the pages leave a step open:
  * no 1/sqrt(dk) scaling of q: o = S^T q as printed;
  * the forget gate acts before the erase, as printed: (I - k k^T) Diag(alpha) S;
  * the read-out uses the state after the token's update (S_t, not S_{t-1});
  * DeltaProduct applies its scalar gate once per token, before the n_h
    Householder steps, and reads q after the last step;
  * nothing is normalised here: inputs are used as given.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _init_state(s0, B, H, dk, dv):
    if s0 is None:
        return np.zeros((B, H, dk, dv))
    return np.array(s0, dtype=np.float64, copy=True)


def _readout(S, q_t):
    # o_t = S_t^T q_t  for S [B,H,dk,dv], q_t [B,H,dk]  ->  [B,H,dv]
    return np.einsum("bhkv,bhk->bhv", S, q_t)


def _erase_write(S, key_l, key_r, w):
    """(I - key_l key_r^T) S + key_l w^T, applied to S [B,H,dk,dv]."""
    pred = np.einsum("bhk,bhkv->bhv", key_r, S)             # key_r^T S
    S = S - key_l[..., :, None] * pred[..., None, :]
    return S + key_l[..., :, None] * w[..., None, :]


def deltanet(q, k, v, beta, s0=None):
    """DeltaNet, the delta rule as one online gradient step on 1/2||S^T k - v||^2:
    S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
    FG2-GDN reading notes, section 2.1, eq. (6). beta: [B, T, H] (scalar per token).
    """
    q, k, v, beta = map(_f64, (q, k, v, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = _init_state(s0, B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        bt = beta[:, t][..., None]
        S = _erase_write(S, bt * k[:, t], k[:, t], v[:, t])  # beta k (k^T S) and beta k v^T
        o[:, t] = _readout(S, q[:, t])
    return o, S


def gdn(q, k, v, alpha, beta, s0=None):
    """Gated DeltaNet: the forget matrix is a scalar, D_t = gamma_t I.
    S_t = (I - beta_t k_t k_t^T) gamma_t S_{t-1} + beta_t k_t v_t^T.
    GDN2-stability page (kexue translation 11945), 'Problem Description' (GDN as
    the special case D_t = gamma_t I); FG2-GDN reading notes, section 1 table.
    alpha (gamma): [B, T, H]; beta: [B, T, H].
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = _init_state(s0, B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S = alpha[:, t][..., None, None] * S
        bt = beta[:, t][..., None]
        S = _erase_write(S, bt * k[:, t], k[:, t], v[:, t])
        o[:, t] = _readout(S, q[:, t])
    return o, S


def kda(q, k, v, alpha, beta, s0=None):
    """Kimi Delta Attention: channel-wise forget Diag(alpha_t), scalar beta_t.
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
    FG2-GDN summary, section 1 (channel-wise decay vector, scalar beta); reading
    notes section 2.1. alpha: [B, T, H, dk]; beta: [B, T, H].
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = _init_state(s0, B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S = alpha[:, t][..., :, None] * S                   # Diag(alpha_t) S
        bt = beta[:, t][..., None]
        S = _erase_write(S, bt * k[:, t], k[:, t], v[:, t])
        o[:, t] = _readout(S, q[:, t])
    return o, S


def fg2(q, k, v, alpha, beta, s0=None, beta_v=None):
    """FG2-GDN, per-channel write rate beta_t in R^{dk} absorbed symmetrically:
    k~ = sqrt(beta) . k,  v~ = sqrt(beta) . v,
    S_t = (I - k~ k~^T) Diag(alpha_t) S_{t-1} + k~ v~^T,   o_t = S_t^T q_t.
    FG2-GDN summary section 2 ('FG2-GDN Update Rule'); reading notes section 2.2,
    eq. (11). With ``beta_v`` given this is FG2-GDN+ (reading notes section 2.3,
    eq. (13)): the erase and the write's key factor use sqrt(beta^k) . k and the
    written value is sqrt(beta^v) . v.
    alpha, beta: [B, T, H, dk]; beta_v: [B, T, H, dv]. Without beta_v, dk must
    equal dv (the value is scaled by the key-side vector).
    """
    q, k, v, alpha, beta, beta_v = map(_f64, (q, k, v, alpha, beta, beta_v))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    if beta_v is None and dk != dv:
        raise ValueError("FG2-GDN with one beta vector needs dk == dv")
    S = _init_state(s0, B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        kt = np.sqrt(beta[:, t]) * k[:, t]
        vt = np.sqrt(beta[:, t] if beta_v is None else beta_v[:, t]) * v[:, t]
        S = alpha[:, t][..., :, None] * S
        S = _erase_write(S, kt, kt, vt)
        o[:, t] = _readout(S, q[:, t])
    return o, S


def deltaproduct(q, k, v, alpha, beta, s0=None):
    """(Gated) DeltaProduct: per token, n_h generalised Householder steps, each an
    online gradient step with its own key, value and rate:
        S <- g_t S;   for i = 1..n_h:  S <- (I - beta_i k_i k_i^T) S + beta_i k_i v_i^T
        o_t = S^T q_t  (after the last step).
    DeltaProduct summary, 'Approach' and the forget-gate row of its results
    table; beta in (0, 2) gives the eigenvalue range [-1, 1].
    k: [B, T, H, n_h, dk]; v: [B, T, H, n_h, dv]; beta: [B, T, H, n_h];
    alpha (gate g): [B, T, H]; q: [B, T, H, dk].
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, T, H, n_h, dk = k.shape
    dv = v.shape[-1]
    S = _init_state(s0, B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S = alpha[:, t][..., None, None] * S
        for i in range(n_h):
            bi = beta[:, t, :, i][..., None]
            S = _erase_write(S, bi * k[:, t, :, i], k[:, t, :, i], v[:, t, :, i])
        o[:, t] = _readout(S, q[:, t])
    return o, S


def gdn2(q, k, v, j, eta, D, s0_pages=None):
    """GDN2 general form in the pages' convention (S in R^{dv x dk}):
    S_t = S_{t-1} D_t (I - eta_t j_t k_t^T) + eta_t v_t k_t^T,   o_t = S_t q_t.
    GDN2-stability page (kexue translation 11945), 'Problem Description', eq. (1).
    j, k, D: [B, T, H, dk]; eta: [B, T, H]; v: [B, T, H, dv].
    Returns (o [B, T, H, dv], S_T [B, H, dv, dk]).
    """
    q, k, v, j, eta, D = map(_f64, (q, k, v, j, eta, D))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = _init_state(s0_pages, B, H, dv, dk)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        SD = S * D[:, t][..., None, :]                     # S D_t (scales columns)
        e = eta[:, t][..., None, None]
        SDj = np.einsum("bhvk,bhk->bhv", SD, j[:, t])       # S D j
        S = SD - e * SDj[..., :, None] * k[:, t][..., None, :] \
            + e * v[:, t][..., :, None] * k[:, t][..., None, :]
        o[:, t] = np.einsum("bhvk,bhk->bhv", S, q[:, t])    # S_t q_t
    return o, S


def forward(inp: dict, s0=None):
    """Dispatch on ``inp['variant']`` (the dict built by gdn_inputs.make_inputs).

    s0 and the returned S_T use the library's layout [B, H, dk, dv]. For the
    asymmetric GDN2 variant the pages' state is its transpose.
    """
    var = inp["variant"]
    if var == "fg2":
        return fg2(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], s0,
                   beta_v=inp.get("beta_v"))
    if var == "kda":
        return kda(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], s0)
    if var == "gdn":
        return gdn(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], s0)
    if var == "deltaproduct":
        return deltaproduct(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], s0)
    if var == "asym":
        s0p = None if s0 is None else np.swapaxes(np.asarray(s0, dtype=np.float64), -1, -2)
        o, Sp = gdn2(inp["q"], inp["k"], inp["v"], inp["j"], inp["eta"], inp["alpha"], s0p)
        return o, np.swapaxes(Sp, -1, -2)
    raise ValueError(f"unknown variant {var!r}")
