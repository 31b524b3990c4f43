"""GDN2 stabilisers: token-wise transforms of the asymmetric variant's inputs
(GDN2-stability page, sections "Simple Strategy" and "Modifying Itself").

TEST INFRASTRUCTURE ONLY (see the package docstring).

Inputs in the library's ASYM layout: k, j and D (the forget diagonal, the library's
alpha) of shape [..., dk], eta of shape [...]. The page assumes unit j and k and
notes that their norms can be absorbed into eta; the functions below absorb them,
so unit vectors are not required.

  clip_decay  D' = min(D, 1 / rho) with rho = ||I - eta j k^T||_2 from the page's
              closed form; then ||D' (I - eta j k^T)||_2 <= 1.
  project_j   j' such that eta j' k^T = j_* k'^T, k' = k / ||k||, where j_* keeps the
              erase rate c = (eta ||k|| j)^T k' and has ||j_*|| <= tau = (c - 1) g + 1/g,
              g = max(D); then ||I - eta j' k^T||_2 <= 1 / g (when tau >= |c|).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def spectral_norm(k, j, eta):
    """rho = ||I - eta j k^T||_2 per row: the page's closed form
    (eta + sqrt(eta^2 - 4 eta c + 4)) / 2 for unit j, k and c = j^T k, with the norms
    absorbed, eta -> eta ||j|| ||k|| and eta c -> eta j^T k."""
    k, j, eta = _f64(k), _f64(j), _f64(eta)
    e = eta * np.linalg.norm(j, axis=-1) * np.linalg.norm(k, axis=-1)
    ejk = eta * np.sum(j * k, axis=-1)
    return 0.5 * (e + np.sqrt(e * e - 4.0 * ejk + 4.0))


def clip_decay(k, j, eta, D):
    """'Simple Strategy': D -> min(D, 1/rho), channel by channel."""
    rho = spectral_norm(k, j, eta)
    return np.minimum(_f64(D), 1.0 / rho[..., None])


def project_j(k, j, eta, D):
    """'Modifying Itself', with eta and ||k|| absorbed into j (jj = eta ||k|| j,
    k' = k / ||k||, so that eta j k^T = jj k'^T):
        c = jj^T k',  g = max(D),  tau = (c - 1) g + 1 / g,
        j_* = c k' + lam (jj - c k'),  lam = min(1, sqrt((tau^2 - c^2) / (||jj||^2 - c^2))),
    returned as j' = j_* / (eta ||k||) = c1 k' + lam (j - c1 k'), c1 = j^T k'.
    Readings where the page gives no value: ||jj||^2 = c^2 (jj parallel to k', or
    eta = 0) leaves j unchanged (lam = 1); tau^2 < c^2, possible only for c < 0 (the
    page's "no solution"), takes lam = 0, j_* = c k'."""
    k, j, eta, D = _f64(k), _f64(j), _f64(eta), _f64(D)
    nk = np.linalg.norm(k, axis=-1)
    kh = k / nk[..., None]
    c1 = np.sum(j * kh, axis=-1)
    c = eta * nk * c1
    jj2 = (eta * nk) ** 2 * np.sum(j * j, axis=-1)
    g = np.max(D, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        tau = c * g + (1.0 / g - g)  # (c - 1) g + 1/g, exact at g = 1
        num = tau * tau - c * c
        den = jj2 - c * c
        lam = np.where(den <= 0.0, 1.0,
                       np.where(num <= 0.0, 0.0, np.minimum(1.0, np.sqrt(num / den))))
    lam = np.where(np.isnan(lam), 1.0, lam)
    return c1[..., None] * kh + lam[..., None] * (j - c1[..., None] * kh)
