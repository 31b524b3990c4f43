"""Error measures used to compare a result with the oracle (float64).

rel_l2  = ||x - y||_2 / ||y||_2 over the whole tensor.
max_rel = ||x - y||_inf / ||y||_inf, normwise so that entries near zero do not
          dominate.
Both return 0.0 when the reference is identically zero and x equals it.
"""
import numpy as np


def rel_l2(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    num = float(np.linalg.norm((x - y).ravel()))
    den = float(np.linalg.norm(y.ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def max_rel(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    num = float(np.max(np.abs(x - y))) if x.size else 0.0
    den = float(np.max(np.abs(y))) if y.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
