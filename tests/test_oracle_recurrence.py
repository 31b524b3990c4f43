"""Pins of the float64 token-loop oracle by routes that do not go through it.

* every variant against explicit products of its dense transition matrices;
* reductions between the pages' models (uniform beta: FG2 -> KDA; gamma 1: KDA ->
  GDN; gamma = 1: GDN -> DeltaNet eq. (6); j = k: GDN2 -> KDA; n_h = 1:
  DeltaProduct -> GDN; beta_v = beta: FG2-GDN+ -> FG2-GDN);
* hand-derivable cases: overwrite memory with orthonormal keys; the DeltaNet
  limit S_1 = (1 - beta) S_0; the RWKV-7 (-1)^t channel at the secular boundary;
* invariants: non-expansiveness of FG2 with v = 0; linearity in (S_0, v) and q.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from oracle import dense


def _small(variant, seed, T=6, d=5, H=2, B=1, n_h=2, fg2_plus=False):
    return gdn_inputs.make_inputs(variant, B, T, H, d, d, dtype="f32", seed=seed, n_h=n_h,
                                  fg2_plus=fg2_plus)


def _dense_path(inp, s0):
    """States and outputs of one (b=0, h) from dense matrix products."""
    var = inp["variant"]
    T = inp["T"]
    out = []
    for h in range(inp["H"]):
        Phis, Ws = [], []
        for t in range(T):
            q = inp["q"][0, t, h]
            if var == "fg2":
                k, v, a, b = (inp[x][0, t, h] for x in ("k", "v", "alpha", "beta"))
                bv = inp["beta_v"][0, t, h] if "beta_v" in inp else None
                Phis.append(dense.fg2_transition(k, a, b))
                Ws.append(dense.fg2_write(k, v, b, bv))
            elif var == "kda":
                k, v, a, b = (inp[x][0, t, h] for x in ("k", "v", "alpha", "beta"))
                Phis.append(dense.householder(k, b) @ np.diag(np.asarray(a, np.float64)))
                Ws.append(float(b) * np.outer(k.astype(np.float64), v.astype(np.float64)))
            elif var == "gdn":
                k, v, a, b = (inp[x][0, t, h] for x in ("k", "v", "alpha", "beta"))
                Phis.append(float(a) * dense.householder(k, b))
                Ws.append(float(b) * np.outer(k.astype(np.float64), v))
            elif var == "deltaproduct":
                n_h = inp["n_h"]
                g = float(inp["alpha"][0, t, h])
                P = g * np.eye(k_dim(inp))
                W = np.zeros((k_dim(inp), inp["dv"]))
                for i in range(n_h):
                    k = inp["k"][0, t, h, i].astype(np.float64)
                    v = inp["v"][0, t, h, i].astype(np.float64)
                    b = float(inp["beta"][0, t, h, i])
                    Hh = dense.householder(k, b)
                    P = Hh @ P
                    W = Hh @ W + b * np.outer(k, v)
                Phis.append(P)
                Ws.append(W)
            elif var == "asym":
                k, v, j, D = (inp[x][0, t, h] for x in ("k", "v", "j", "alpha"))
                e = float(inp["eta"][0, t, h])
                # right-multiplied factor of the pages' S (dv x dk); on S^T it acts from the left
                Phis.append(dense.gdn2_transition(j, k, e, D).T)
                Ws.append(e * np.outer(k.astype(np.float64), v))
            del q
        S0 = np.zeros((k_dim(inp), inp["dv"])) if s0 is None else s0[0, h].astype(np.float64)
        states = dense.run_dense(Phis, Ws, S0)
        o = np.stack([St.T @ inp["q"][0, t, h].astype(np.float64) for t, St in enumerate(states)])
        out.append((o, states[-1]))
    return out


def k_dim(inp):
    return inp["dk"]


@pytest.mark.parametrize("variant", ["fg2", "kda", "gdn", "deltaproduct", "asym"])
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("with_s0", [False, True])
def test_oracle_vs_dense_products(variant, seed, with_s0):
    inp = _small(variant, seed)
    s0 = gdn_inputs.make_state(1, inp["H"], inp["dk"], inp["dv"], seed=seed) if with_s0 else None
    o, S = oracle.forward(inp, s0)
    for h, (o_ref, S_ref) in enumerate(_dense_path(inp, s0)):
        np.testing.assert_allclose(o[0, :, h], o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[0, h], S_ref, rtol=1e-12, atol=1e-12)


def test_fg2_plus_vs_dense_products():
    inp = _small("fg2", 4, fg2_plus=True)
    o, S = oracle.forward(inp)
    for h, (o_ref, S_ref) in enumerate(_dense_path(inp, None)):
        np.testing.assert_allclose(o[0, :, h], o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[0, h], S_ref, rtol=1e-12, atol=1e-12)


def test_reductions_between_models():
    rng = np.random.default_rng(5)
    inp = _small("fg2", 5, T=7, d=4, H=3, B=2)
    beta_s = rng.uniform(0.1, 0.9, (2, 7, 3))
    s0 = gdn_inputs.make_state(2, 3, 4, 4, seed=5)
    q, k, v, a = inp["q"], inp["k"], inp["v"], inp["alpha"]
    # FG2 with a beta vector that is constant over channels == KDA with that scalar
    o1, S1 = oracle.fg2(q, k, v, a, np.repeat(beta_s[..., None], 4, -1), s0)
    o2, S2 = oracle.kda(q, k, v, a, beta_s, s0)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-13)
    # KDA with alpha = gamma * 1 == GDN
    gam = rng.uniform(0.5, 1.0, (2, 7, 3))
    o3, S3 = oracle.kda(q, k, v, np.repeat(gam[..., None], 4, -1), beta_s, s0)
    o4, S4 = oracle.gdn(q, k, v, gam, beta_s, s0)
    np.testing.assert_allclose(o3, o4, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S3, S4, rtol=1e-13, atol=1e-13)
    # GDN with gamma = 1 == DeltaNet eq. (6)
    o5, S5 = oracle.gdn(q, k, v, np.ones_like(gam), beta_s, s0)
    o6, S6 = oracle.deltanet(q, k, v, beta_s, s0)
    np.testing.assert_allclose(o5, o6, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S5, S6, rtol=1e-13, atol=1e-13)
    # GDN2 with j = k == KDA with beta = eta (state transposed)
    o7, S7 = oracle.gdn2(q, k, v, k, beta_s, a, np.swapaxes(s0, -1, -2))
    np.testing.assert_allclose(o7, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.swapaxes(S7, -1, -2), S2, rtol=1e-12, atol=1e-12)
    # DeltaProduct with n_h = 1 == GDN
    o8, S8 = oracle.deltaproduct(q, k[:, :, :, None], v[:, :, :, None], gam,
                                 beta_s[..., None], s0)
    np.testing.assert_allclose(o8, o4, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S8, S4, rtol=1e-13, atol=1e-13)
    # FG2-GDN+ with beta_v = beta == FG2-GDN
    o9, S9 = oracle.fg2(q, k, v, a, inp["beta"], s0, beta_v=inp["beta"])
    o10, S10 = oracle.fg2(q, k, v, a, inp["beta"], s0)
    np.testing.assert_allclose(o9, o10, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(S9, S10, rtol=1e-15, atol=1e-15)


def test_overwrite_memory_orthonormal_keys():
    """k_t = e_{t mod d}, alpha = 1, beta = 1: each token replaces row (t mod d) of S
    with v_t; the read-out is then known by bookkeeping alone."""
    d, T = 4, 11
    rng = np.random.default_rng(11)
    k = np.zeros((1, T, 1, d))
    for t in range(T):
        k[0, t, 0, t % d] = 1.0
    v = rng.standard_normal((1, T, 1, d))
    q = rng.standard_normal((1, T, 1, d))
    s0 = rng.standard_normal((1, 1, d, d))
    o, S = oracle.fg2(q, k, v, np.ones((1, T, 1, d)), np.ones((1, T, 1, d)), s0)
    rows = [s0[0, 0, i].copy() for i in range(d)]
    for t in range(T):
        rows[t % d] = v[0, t, 0].copy()
        expect = sum(q[0, t, 0, i] * rows[i] for i in range(d))
        np.testing.assert_allclose(o[0, t, 0], expect, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(S[0, 0], np.stack(rows))


def test_deltanet_limit_single_step():
    """alpha = 1, scalar beta, v = 0 and S_0 = k e^T: S_1 = (1 - beta) S_0."""
    rng = np.random.default_rng(12)
    d = 6
    k = rng.standard_normal(d)
    k /= np.linalg.norm(k)
    e = rng.standard_normal(d)
    for beta in (0.25, 1.0, 1.5, 2.0):
        s0 = np.outer(k, e)[None, None]
        o, S = oracle.deltanet(np.zeros((1, 1, 1, d)), k[None, None, None], np.zeros((1, 1, 1, d)),
                               np.full((1, 1, 1), beta), s0)
        np.testing.assert_allclose(S[0, 0], (1.0 - beta) * s0[0, 0], atol=1e-15)


def test_secular_boundary_sign_flipping_channel():
    """RWKV-7 transition diag(w) - kappa (a.kappa)^T at budget 1, constant over tokens,
    v = 0: the state along the eigenvector of -1 flips sign every token. Written in
    GDN2 form (S in R^{dv x dk}, right-multiplied by D (I - eta j k^T)) with D = w,
    k = kappa, eta = 1 and j = a . kappa / w, whose transpose is the RWKV-7 matrix."""
    rng = np.random.default_rng(13)
    d, T = 5, 9
    w = rng.uniform(0.5, 0.95, d)
    kappa = rng.standard_normal(d)
    kappa /= np.linalg.norm(kappa)
    a = rng.uniform(0.2, 1.0, d)
    a = a / dense.secular_boundary_budget(w, kappa, a)
    A = dense.rwkv7_transition(w, kappa, a)
    ev, vecs = np.linalg.eig(A)
    i = int(np.argmin(ev.real))
    assert ev[i].real == pytest.approx(-1.0, abs=1e-12)
    x = vecs[:, i].real
    jvec = a * kappa / w
    np.testing.assert_allclose(dense.gdn2_transition(jvec, kappa, 1.0, w).T, A, atol=1e-15)
    e = rng.standard_normal(3)
    s0_pages = np.outer(e, x)[None, None]               # S_0 = e x^T (dv x dk)
    rep = lambda z: np.broadcast_to(z, (1, T, 1, d)).copy()  # noqa: E731
    o, S = oracle.gdn2(np.zeros((1, T, 1, d)), rep(kappa), np.zeros((1, T, 1, 3)), rep(jvec),
                       np.ones((1, T, 1)), rep(w), s0_pages)
    np.testing.assert_allclose(S[0, 0], (-1.0) ** T * s0_pages[0, 0], atol=1e-11)


def test_fg2_non_expansive_without_writes():
    inp = _small("fg2", 14, T=40, d=6, H=2)
    rng = np.random.default_rng(14)
    S = rng.standard_normal((1, 2, 6, 6))
    norms = [np.linalg.norm(S[0, h], 2) for h in range(2)]
    for t in range(40):
        sl = gdn_inputs.slice_tokens(inp, t, t + 1)
        sl["v"] = np.zeros_like(sl["v"])
        _, S = oracle.forward(sl, S)
        new = [np.linalg.norm(S[0, h], 2) for h in range(2)]
        assert all(n1 <= n0 + 1e-13 for n0, n1 in zip(norms, new))
        norms = new


@pytest.mark.parametrize("variant", ["fg2", "deltaproduct", "asym"])
def test_linearity(variant):
    a = _small(variant, 20)
    b = _small(variant, 21)
    b_in = dict(a)
    b_in["v"] = b["v"]
    s0a = gdn_inputs.make_state(1, a["H"], a["dk"], a["dv"], seed=1)
    s0b = gdn_inputs.make_state(1, a["H"], a["dk"], a["dv"], seed=2)
    oa, Sa = oracle.forward(a, s0a)
    ob, Sb = oracle.forward(b_in, s0b)
    mix = dict(a)
    mix["v"] = 2.0 * a["v"].astype(np.float64) - 3.0 * b["v"].astype(np.float64)
    om, Sm = oracle.forward(mix, 2.0 * s0a.astype(np.float64) - 3.0 * s0b.astype(np.float64))
    np.testing.assert_allclose(om, 2.0 * oa - 3.0 * ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sm, 2.0 * Sa - 3.0 * Sb, rtol=1e-12, atol=1e-12)
    q2 = dict(a)
    q2["q"] = -1.5 * a["q"].astype(np.float64)
    oq, _ = oracle.forward(q2, s0a)
    np.testing.assert_allclose(oq, -1.5 * oa, rtol=1e-13, atol=1e-13)


def test_split_sequence_state_passing():
    inp = _small("fg2", 30, T=13, d=4, H=2)
    o, S = oracle.forward(inp)
    o1, S1 = oracle.forward(gdn_inputs.slice_tokens(inp, 0, 5))
    o2, S2 = oracle.forward(gdn_inputs.slice_tokens(inp, 5, 13), S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(S2, S, rtol=1e-14, atol=1e-14)


def test_no_write_is_pure_decay():
    """beta = 0: S_t = Diag(prod alpha) S_0 and o_t = S_t^T q_t, channel by channel."""
    inp = _small("fg2", 15, T=12, d=5, H=2)
    inp["beta"] = np.zeros_like(inp["beta"])
    s0 = np.random.default_rng(15).standard_normal((1, 2, 5, 5))
    o, S = oracle.forward(inp, s0)
    cum = np.cumprod(np.asarray(inp["alpha"], np.float64), axis=1)[0]      # [T, H, dk]
    St = cum[:, :, :, None] * s0[0][None]
    np.testing.assert_allclose(S[0], St[-1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[0], np.einsum("thkv,thk->thv", St, np.asarray(inp["q"], np.float64)[0]),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("variant", ["fg2", "kda"])
def test_full_write_recalls_the_value(variant):
    """alpha = 1, beta = 1, unit keys and q_t = k_t: o_t = v_t for any earlier state."""
    inp = _small(variant, 16, T=9, d=6, H=2)
    inp["alpha"] = np.ones_like(inp["alpha"])
    inp["beta"] = np.ones_like(inp["beta"])
    k = np.asarray(inp["k"], np.float64)
    inp["k"] = k / np.linalg.norm(k, axis=-1, keepdims=True)
    inp["q"] = inp["k"].copy()
    s0 = np.random.default_rng(16).standard_normal((1, 2, 6, 6))
    o, _ = oracle.forward(inp, s0)
    np.testing.assert_allclose(o, np.asarray(inp["v"], np.float64), rtol=1e-12, atol=1e-12)
