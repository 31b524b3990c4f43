"""Pins of the GDN2 stabilisers in the oracle (GDN2-stability page, "The Spectral
Norm", "Simple Strategy", "Modifying Itself"): each property is checked by explicit
matrices and numpy's spectral norm, not through the closed forms being tested."""
import numpy as np
import pytest

from oracle import stabilize


def _rows(seed, n=200, d=12, eta_max=3.0, unit=False):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, d))
    j = rng.standard_normal((n, d)) + 0.5 * k
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        j /= np.linalg.norm(j, axis=-1, keepdims=True)
    eta = eta_max * rng.random(n)
    D = 1.0 / (1.0 + np.exp(-(3.0 + rng.standard_normal((n, d)))))
    return k, j, eta, D


def _A(k, j, eta):
    return np.eye(k.size) - eta * np.outer(j, k)


@pytest.mark.parametrize("unit", [True, False])
def test_spectral_norm_matches_numpy(unit):
    k, j, eta, _ = _rows(1, unit=unit)
    rho = stabilize.spectral_norm(k, j, eta)
    for i in range(len(eta)):
        assert rho[i] == pytest.approx(np.linalg.norm(_A(k[i], j[i], eta[i]), 2), rel=1e-12)


def test_clip_decay_bounds_the_transition():
    k, j, eta, D = _rows(2)
    Dc = stabilize.clip_decay(k, j, eta, D)
    rho = np.array([np.linalg.norm(_A(k[i], j[i], eta[i]), 2) for i in range(len(eta))])
    for i in range(len(eta)):
        assert np.linalg.norm(np.diag(Dc[i]) @ _A(k[i], j[i], eta[i]), 2) <= 1.0 + 1e-12
    # only the channels above 1/rho move, and they move to 1/rho exactly
    keep = D <= 1.0 / rho[:, None]
    assert np.array_equal(Dc[keep], D[keep])
    np.testing.assert_allclose(Dc[~keep], np.broadcast_to(1.0 / rho[:, None], D.shape)[~keep], rtol=1e-15)
    assert (~keep).any() and keep.any()


def test_project_j_keeps_the_erase_rate_and_bounds_the_norm():
    k, j, eta, D = _rows(3)
    jp = stabilize.project_j(k, j, eta, D)
    g = D.max(axis=-1)
    moved = 0
    for i in range(len(eta)):
        # erase rate eta j^T k unchanged
        assert eta[i] * jp[i] @ k[i] == pytest.approx(eta[i] * j[i] @ k[i], rel=1e-12, abs=1e-12)
        c = eta[i] * j[i] @ k[i]
        tau = (c - 1.0) * g[i] + 1.0 / g[i]
        if tau >= abs(c):
            assert np.linalg.norm(_A(k[i], jp[i], eta[i]), 2) <= 1.0 / g[i] + 1e-12
        if not np.allclose(jp[i], j[i]):
            moved += 1
            # a row is moved only when it was not already within 1/g
            assert np.linalg.norm(_A(k[i], j[i], eta[i]), 2) > 1.0 / g[i]
        else:
            assert np.linalg.norm(_A(k[i], j[i], eta[i]), 2) <= 1.0 / g[i] + 1e-12
    assert moved > 0


def test_project_j_at_full_retention_gives_kda():
    # g = 1: tau = c, so j_* = c k' and the update matrix is KDA's I - c k' k'^T
    k, j, eta, D = _rows(4, unit=True)
    D[:, 0] = 1.0
    c = eta * np.sum(j * k, axis=-1)
    ok = c >= 0
    jp = stabilize.project_j(k, j, eta, D)
    for i in np.flatnonzero(ok):
        np.testing.assert_allclose(eta[i] * np.outer(jp[i], k[i]), c[i] * np.outer(k[i], k[i]), atol=1e-12)


def test_project_j_special_cases():
    k = np.array([[1.0, 0.0, 0.0]])
    D = np.full((1, 3), 0.9)
    # eta = 0: nothing to move
    j = np.array([[0.3, 0.4, 0.5]])
    np.testing.assert_array_equal(stabilize.project_j(k, j, np.array([0.0]), D), j)
    # j parallel to k: nothing to move
    jk = np.array([[0.7, 0.0, 0.0]])
    np.testing.assert_allclose(stabilize.project_j(k, jk, np.array([1.0]), D), jk, rtol=1e-15)


def test_gated_key_parametrisation_reaches_the_bound():
    """'Modifying Itself' closes with j = k (.) b, b in [0, 1]^d: then c = eta j^T k >= 0,
    and for unit k and eta <= 1 the projected j' always meets ||I - eta j' k^T|| <= 1/g
    (no row falls in the case without a solution)."""
    rng = np.random.default_rng(6)
    n, d = 300, 10
    k = rng.standard_normal((n, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    j = k * rng.random((n, d))
    eta = rng.random(n)
    D = 1.0 / (1.0 + np.exp(-(3.0 + rng.standard_normal((n, d)))))
    assert (eta * np.sum(j * k, -1) >= 0).all()
    jp = stabilize.project_j(k, j, eta, D)
    for i in range(n):
        g = D[i].max()
        assert np.linalg.norm(_A(k[i], jp[i], eta[i]), 2) <= 1.0 / g + 1e-9
