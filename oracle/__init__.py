"""Float64 CPU oracle for the gated delta rule forward pass.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, token-by-token
definition of what the library computes, used to check the HIP path. Only the
test suite, the package's smoke check and the CPU-baseline leg of the benchmark
may import it. It shares no code with the HIP path and imports nothing from it;
the HIP path never imports it.

Modules
  recurrence  one function per variant, each written from the passage that
              defines it (token loop, rank-1 updates, float64)
  dense       explicit transition matrices and the closed forms the pages give
              (spectral norm of I - eta j k^T, the RWKV-7 secular equation),
              used only to pin ``recurrence``
  stabilize   the GDN2 stabilisers (decay clip, j projection), token-wise
  backward    reverse-mode gradients of the token recurrence (all variants but
              DeltaProduct), pinned by finite differences of ``recurrence``
  metrics     rel-L2 and normwise max-rel error (pinned by hand-computed values
              in tests/test_oracle_metrics.py)

Parity status: every function in ``recurrence`` is pinned by tests that do not
go through it (explicit matrix products, special-case reductions between the
pages' models, closed forms, hand-derivable cases); see tests/test_oracle_*.py.
"""
from .recurrence import (deltanet, gdn, kda, fg2, deltaproduct, gdn2, forward)  # noqa: F401
from .metrics import rel_l2, max_rel  # noqa: F401
from . import stabilize, backward  # noqa: F401
