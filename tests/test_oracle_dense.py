"""Pins of the dense transition builders against the pages' closed forms.

Sources: GDN2-stability page (kexue translation 11945): 'The Spectral Norm',
'Modifying Itself', 'Proof Process'; secularmode README (RWKV-7 transition):
'An exact secular spectrum', 'Retention is safe...', 'Decay makes the instability
easier', 'Retention-stable can still be step-expansive'; FG2-GDN reading notes
section 2.2 (the symmetric rank-1 factor I - k~ k~^T).
"""
import os

import numpy as np
import pytest

from oracle import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x):
    return x / np.linalg.norm(x)


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_spectral_norm_golden_values():
    rows = _read_table("spectral_norm.txt")
    assert len(rows) >= 6
    rng = np.random.default_rng(0)
    for eta_s, c_s, norm_s, *_ in rows:
        eta, c, expect = float(eta_s), float(c_s), float(norm_s)
        assert dense.spectral_norm_closed_form(eta, c) == pytest.approx(expect, rel=1e-15)
        # build unit j, k with j^T k = c and measure the matrix itself
        k = _unit(rng.standard_normal(6))
        p = rng.standard_normal(6)
        p = _unit(p - (p @ k) * k)
        j = c * k + np.sqrt(max(0.0, 1.0 - c * c)) * p
        got = np.linalg.norm(dense.gdn2_A(j, k, eta), 2)
        assert got == pytest.approx(expect, rel=1e-12)


@pytest.mark.parametrize("seed", range(20))
def test_spectral_norm_closed_form_random(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.integers(2, 9))
    j, k = _unit(rng.standard_normal(d)), _unit(rng.standard_normal(d))
    eta = float(rng.uniform(0.0, 3.0))
    got = np.linalg.norm(dense.gdn2_A(j, k, eta), 2)
    assert got == pytest.approx(dense.spectral_norm_closed_form(eta, j @ k), rel=1e-12)


def test_spectral_norm_iff_and_lower_bound():
    rng = np.random.default_rng(1)
    k = _unit(rng.standard_normal(5))
    for eta in (0.3, 1.0, 1.7, 2.0):       # j = k, eta <= 2  =>  <= 1
        assert np.linalg.norm(dense.gdn2_A(k, k, eta), 2) <= 1.0 + 1e-12
    assert np.linalg.norm(dense.gdn2_A(k, k, 2.5), 2) > 1.0 + 1e-6
    assert np.linalg.norm(dense.gdn2_A(_unit(rng.standard_normal(5)), k, 0.0), 2) == \
        pytest.approx(1.0, abs=1e-14)
    for _ in range(50):                    # j != k, eta > 0  =>  > max(eta,2) - 1 >= 1
        j = _unit(rng.standard_normal(5))
        eta = float(rng.uniform(0.01, 3.0))
        n = np.linalg.norm(dense.gdn2_A(j, k, eta), 2)
        assert n > max(eta, 2.0) - 1.0
        assert n > 1.0


def test_modifying_itself_projection():
    """j* = c k + lambda* (j - c k) keeps j*^T k = c and brings ||I - j* k^T|| under
    1/gamma_max; gamma_max = 1 gives j* = c k (the KDA case)."""
    rng = np.random.default_rng(2)
    for _ in range(30):
        k = _unit(rng.standard_normal(6))
        p = rng.standard_normal(6)
        p = (p - (p @ k) * k) * rng.uniform(0.1, 3.0)
        j = rng.uniform(0.0, 1.5) * k + p            # c = j^T k in [0, 1.5]: tau >= c
        c = float(j @ k)
        gmax = float(rng.uniform(0.5, 1.0))
        tau = (c - 1.0) * gmax + 1.0 / gmax
        jn2 = float(j @ j)
        lam = min(1.0, np.sqrt(max(0.0, (tau * tau - c * c) / (jn2 - c * c))))
        js = c * k + lam * (j - c * k)
        assert js @ k == pytest.approx(c, abs=1e-12)
        n = np.linalg.norm(np.eye(6) - np.outer(js, k), 2)
        assert n == pytest.approx(dense.spectral_norm_closed_form_unnormalised(
            np.linalg.norm(js), c), rel=1e-12)
        assert n <= 1.0 / gmax + 1e-12
    k = _unit(rng.standard_normal(4))
    j = k * rng.uniform(0, 1, 4)
    c = float(j @ k)
    tau = (c - 1.0) * 1.0 + 1.0
    assert tau == pytest.approx(c)


def test_symmetric_factor_eigenvalues():
    """I - k~ k~^T has d-1 eigenvalues 1 and one 1 - ||k~||^2; with ||k~||^2 <= 2
    it is non-expansive (the tied rank-1 form kept by FG2-GDN)."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        d = int(rng.integers(2, 9))
        k = _unit(rng.standard_normal(d))
        beta = rng.uniform(0, 1, d)
        F = dense.fg2_transition(k, np.ones(d), beta)
        ev = np.sort(np.linalg.eigvalsh(F))
        kt2 = float(np.sum(beta * k * k))
        np.testing.assert_allclose(ev, np.sort(np.r_[np.ones(d - 1), 1.0 - kt2]), atol=1e-13)
        assert np.linalg.norm(F, 2) <= 1.0 + 1e-13


def _rwkv7(rng, d, a_const=None):
    w = np.sort(rng.uniform(0.2, 0.99, d))
    kappa = _unit(rng.standard_normal(d))
    a = np.full(d, a_const) if a_const is not None else rng.uniform(0.0, 1.0, d)
    return w, kappa, a


@pytest.mark.parametrize("seed", range(10))
def test_secular_roots_are_the_spectrum(seed):
    rng = np.random.default_rng(100 + seed)
    d = int(rng.integers(2, 9))
    w, kappa, a = _rwkv7(rng, d)
    A = dense.rwkv7_transition(w, kappa, a)
    ev = np.linalg.eigvals(A)
    assert np.max(np.abs(ev.imag)) < 1e-9                     # real spectrum
    roots = dense.secular_roots(w, a * kappa * kappa)
    np.testing.assert_allclose(np.sort(ev.real), roots, atol=1e-10)
    ws = np.sort(w)                                           # interlacing
    assert np.all(roots <= ws + 1e-12)
    assert np.all(roots[1:] >= ws[:-1] - 1e-12)
    assert roots[-1] <= ws.max() < 1.0                        # retention top pinned
    # det(A - lam I) = prod(w - lam) f(lam) at a point away from the poles
    lam = -0.37
    lhs = np.linalg.det(A - lam * np.eye(d))
    rhs = np.prod(w - lam) * dense.secular_f(lam, w, a * kappa * kappa)
    assert lhs == pytest.approx(rhs, rel=1e-10)


def test_secular_boundary_and_neighbours():
    facts = {r[0]: float(r[1]) for r in _read_table("secular_facts.txt")}
    rng = np.random.default_rng(7)
    for _ in range(10):
        d = int(rng.integers(3, 9))
        w, kappa, a = _rwkv7(rng, d)
        a = a / dense.secular_boundary_budget(w, kappa, a)    # budget exactly 1
        mn = np.min(np.linalg.eigvals(dense.rwkv7_transition(w, kappa, a)).real)
        assert mn == pytest.approx(facts["boundary_min_eig"], abs=1e-12)
        assert abs(mn + 1.0) < facts["boundary_tolerance"]
        lo = np.min(np.linalg.eigvals(dense.rwkv7_transition(w, kappa, 0.98 * a)).real)
        hi = np.min(np.linalg.eigvals(dense.rwkv7_transition(w, kappa, 1.02 * a)).real)
        assert np.sign(lo + 1.0) == facts["below_boundary_sign"]
        assert np.sign(hi + 1.0) == facts["above_boundary_sign"]
        assert dense.secular_f(-1.0, w, a * kappa * kappa) == pytest.approx(0.0, abs=1e-13)


def test_deltanet_limit():
    facts = {r[0]: float(r[1]) for r in _read_table("secular_facts.txt")}
    rng = np.random.default_rng(8)
    for beta in (0.3, 1.0, 1.5, 2.0):
        d = 5
        kappa = _unit(rng.standard_normal(d))
        A = dense.rwkv7_transition(np.ones(d), kappa, np.full(d, beta))
        np.testing.assert_allclose(A, dense.householder(kappa, beta), atol=1e-15)
        ev = np.sort(np.linalg.eigvalsh(A))
        assert ev[0] == pytest.approx(1.0 - beta, abs=1e-13)
        np.testing.assert_allclose(ev[1:], 1.0, atol=1e-13)
    assert 1.0 - 2.0 == facts["deltanet_limit_beta2_min_eig"]


def test_decay_lowers_the_budget_needed():
    """At fixed removal, smaller decay values raise sum a kappa^2/(w+1)."""
    rng = np.random.default_rng(9)
    d = 6
    kappa = _unit(rng.standard_normal(d))
    a = rng.uniform(0.2, 0.6, d)
    budgets = [dense.secular_boundary_budget(np.full(d, w), kappa, a)
               for w in (1.0, 0.7, 0.5, 0.3)]
    assert all(b1 < b2 for b1, b2 in zip(budgets, budgets[1:]))
    mins = [np.min(np.linalg.eigvals(dense.rwkv7_transition(np.full(d, w), kappa, a)).real)
            for w in (1.0, 0.7, 0.5, 0.3)]
    assert all(m1 > m2 for m1, m2 in zip(mins, mins[1:]))


def test_step_expansive_gap():
    """Constant a: symmetric, rho = sigma_max. Non-constant a: some transitions have
    rho <= 1 < sigma_max (the README's witness was 0.883 <= 1 < 1.003)."""
    rng = np.random.default_rng(10)
    w, kappa, _ = _rwkv7(rng, 5)
    A = dense.rwkv7_transition(w, kappa, np.full(5, 0.7))
    assert np.allclose(A, A.T)
    assert np.max(np.abs(np.linalg.eigvals(A))) == pytest.approx(np.linalg.norm(A, 2),
                                                                rel=1e-12)
    found = False
    for _ in range(2000):
        w = rng.uniform(0.6, 1.0, 4)
        kappa = _unit(rng.standard_normal(4))
        a = rng.uniform(0.0, 2.0, 4)
        A = dense.rwkv7_transition(w, kappa, a)
        rho = np.max(np.abs(np.linalg.eigvals(A)))
        if rho <= 1.0 and np.linalg.norm(A, 2) > 1.0:
            found = True
            break
    assert found
