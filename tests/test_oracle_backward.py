"""Pins of the backward oracle: every gradient against central finite differences of
the forward oracle (an independent code path: oracle.forward and its GDN2 form in the
page's transposed convention), on tiny inputs of each covered variant."""
import numpy as np
import pytest

import gdn_inputs
import oracle
from oracle import backward as bwd

CASES = [("fg2", False), ("fg2", True), ("kda", False), ("gdn", False), ("asym", False),
         ("deltaproduct", False)]


def _loss(inp, s0, do, dsf):
    o, S = oracle.forward(inp, s0)
    return float(np.sum(o * do) + np.sum(S * dsf))


@pytest.mark.parametrize("variant,plus", CASES, ids=lambda c: str(c))
def test_gradients_match_finite_differences(variant, plus):
    B, T, H, d = 1, 5, 2, 3
    inp = gdn_inputs.make_inputs(variant, B, T, H, d, d, dtype="f32", seed=80, fg2_plus=plus,
                                 n_h=3 if variant == "deltaproduct" else 1)
    for key in list(inp):
        if isinstance(inp[key], np.ndarray):
            inp[key] = inp[key].astype(np.float64)
    rng = np.random.default_rng(81)
    s0 = rng.standard_normal((B, H, d, d))
    do = rng.standard_normal((B, T, H, d))
    dsf = rng.standard_normal((B, H, d, d))
    g = bwd.backward(inp, do, s0, dsf)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta",
             "beta_v": "dbeta_v", "j": "dj", "eta": "deta"}
    h = 1e-6
    checked = 0
    for key, gname in names.items():
        if inp.get(key) is None:
            continue
        x = inp[key]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(inp, s0, do, dsf)
            x[idx] = old - h
            lm = _loss(inp, s0, do, dsf)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-7, err_msg=key)
        checked += 1
    num = np.zeros_like(s0)
    for idx in np.ndindex(s0.shape):
        old = s0[idx]
        s0[idx] = old + h
        lp = _loss(inp, s0, do, dsf)
        s0[idx] = old - h
        lm = _loss(inp, s0, do, dsf)
        s0[idx] = old
        num[idx] = (lp - lm) / (2 * h)
    np.testing.assert_allclose(g["ds0"], num, rtol=1e-6, atol=1e-7, err_msg="s0")
    assert checked >= 5


def test_no_state_gradient_without_upstream():
    """With do = 0 and dS_T = 0 every gradient is exactly zero."""
    inp = gdn_inputs.make_inputs("fg2", 1, 4, 1, 3, 3, dtype="f32", seed=82)
    g = bwd.backward(inp, np.zeros((1, 4, 1, 3)))
    for name, arr in g.items():
        assert not np.any(arr), name
