"""Explicit transition matrices and the closed forms the pages state about them.

TEST INFRASTRUCTURE ONLY (see the package docstring). These builders are used to
pin ``recurrence`` by a different route (explicit d x d matrix products instead
of rank-1 updates); they are themselves pinned by the pages' closed forms.
"""
from __future__ import annotations

import numpy as np


# --- single-token transitions -------------------------------------------------

def fg2_transition(k, alpha, beta):
    """(I - k~ k~^T) Diag(alpha), k~ = sqrt(beta) . k  (FG2-GDN reading notes,
    section 2.2, eq. (11)); acts on S in R^{dk x dv} from the left."""
    k, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (k, alpha, beta))
    kt = np.sqrt(beta) * k
    return (np.eye(k.size) - np.outer(kt, kt)) @ np.diag(alpha)


def fg2_write(k, v, beta, beta_v=None):
    """k~ v~^T with v~ = sqrt(beta_v or beta) . v  (eq. (11); eq. (13) with beta_v)."""
    k, v, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, beta))
    bv = beta if beta_v is None else np.asarray(beta_v, dtype=np.float64)
    return np.outer(np.sqrt(beta) * k, np.sqrt(bv) * v)


def householder(k, beta):
    """Generalised Householder factor I - beta k k^T (DeltaProduct summary)."""
    k = np.asarray(k, dtype=np.float64)
    return np.eye(k.size) - beta * np.outer(k, k)


def gdn2_A(j, k, eta):
    """A = I - eta j k^T (GDN2-stability page, 'The Spectral Norm')."""
    j, k = np.asarray(j, dtype=np.float64), np.asarray(k, dtype=np.float64)
    return np.eye(k.size) - eta * np.outer(j, k)


def gdn2_transition(j, k, eta, D):
    """D (I - eta j k^T): the factor that right-multiplies S in R^{dv x dk}
    (GDN2-stability page, eq. (1))."""
    return np.diag(np.asarray(D, dtype=np.float64)) @ gdn2_A(j, k, eta)


def rwkv7_transition(w, kappa, a):
    """diag(w) - kappa (a . kappa)^T (secularmode README, opening paragraph)."""
    w, kappa, a = (np.asarray(x, dtype=np.float64) for x in (w, kappa, a))
    return np.diag(w) - np.outer(kappa, a * kappa)


# --- closed forms ---------------------------------------------------------------

def spectral_norm_closed_form(eta, c):
    """||I - eta j k^T||_2 for unit j, k with c = j^T k:
    (eta + sqrt(eta^2 - 4 eta c + 4)) / 2  (GDN2-stability page, eq. 'spec')."""
    return 0.5 * (eta + np.sqrt(eta * eta - 4.0 * eta * c + 4.0))


def spectral_norm_closed_form_unnormalised(j_norm, c):
    """||I - j k^T||_2 with eta absorbed into j (unit k, c = j^T k):
    (||j|| + sqrt(||j||^2 - 4 c + 4)) / 2  (section 'Modifying Itself')."""
    return 0.5 * (j_norm + np.sqrt(j_norm * j_norm - 4.0 * c + 4.0))


def secular_f(lam, w, r):
    """f(lambda) = 1 - sum_i r_i / (w_i - lambda), r_i = a_i kappa_i^2
    (secularmode README, 'An exact secular spectrum')."""
    w, r = np.asarray(w, dtype=np.float64), np.asarray(r, dtype=np.float64)
    return 1.0 - np.sum(r / (w - lam))


def secular_roots(w, r, iters: int = 200):
    """All d roots of f(lambda) = 0 for distinct w and r > 0, by bisection.

    Classical rank-one-update theory: f rises from -inf to +inf between
    consecutive poles, so exactly one root lies in each gap (w_(i-1), w_(i)) and
    one below the smallest pole (f -> 1 as lambda -> -inf). No eigen-solver is
    used, so the result is independent of numpy.linalg.eigvals.
    """
    w = np.asarray(w, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    order = np.argsort(w)
    ws, rs = w[order], r[order]
    roots = []
    lo_bound = ws[0] - 1.0 - np.sum(rs) * 2.0     # f(lo_bound) > 0 there
    while secular_f(lo_bound, ws, rs) <= 0.0:
        lo_bound -= 2.0 * (ws[0] - lo_bound)
    brackets = [(lo_bound, ws[0])] + [(ws[i - 1], ws[i]) for i in range(1, ws.size)]
    for lo, hi in brackets:
        # on (lo, hi): f(lo+) > 0 (or finite positive), f(hi-) = -inf
        a, b = lo, hi
        for _ in range(iters):
            m = 0.5 * (a + b)
            if m <= a or m >= b:
                break
            if secular_f(m, ws, rs) > 0.0:
                a = m
            else:
                b = m
        roots.append(0.5 * (a + b))
    return np.array(roots)


def secular_boundary_budget(w, kappa, a):
    """sum_i a_i kappa_i^2 / (w_i + 1); -1 is an eigenvalue exactly when it is 1
    (secularmode README, 'Retention is safe; instability is only from below')."""
    w, kappa, a = (np.asarray(x, dtype=np.float64) for x in (w, kappa, a))
    return float(np.sum(a * kappa * kappa / (w + 1.0)))


# --- whole sequences by explicit products --------------------------------------

def run_dense(transitions, writes, S0):
    """S_t = Phi_t S_{t-1} + W_t evaluated as the closed sum
        S_t = (Phi_t ... Phi_1) S0 + sum_{s<=t} (Phi_t ... Phi_{s+1}) W_s
    with every partial product formed explicitly. Returns [S_1, ..., S_T]."""
    T = len(transitions)
    d = transitions[0].shape[0]
    states = []
    for t in range(T):
        acc = np.eye(d)
        for s in range(t, -1, -1):          # Phi_t ... Phi_0 applied to S0
            acc = acc @ transitions[s]
        St = acc @ S0
        for s in range(t + 1):
            prod = np.eye(d)
            for u in range(t, s, -1):       # Phi_t ... Phi_{s+1}
                prod = prod @ transitions[u]
            St = St + prod @ writes[s]
        states.append(St)
    return states
