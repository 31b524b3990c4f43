"""Token-sequential kernel (gdn_recurrent_step) against the float64 oracle."""
import numpy as np
import pytest

import gdn_inputs
import oracle

pytestmark = pytest.mark.gpu

CASES = [
    # variant, dtype, B, T, H, dk, dv, n_h
    ("fg2", "f32", 1, 64, 1, 16, 16, 1),
    ("fg2", "f32", 2, 77, 3, 64, 64, 1),
    ("fg2", "bf16", 1, 300, 4, 128, 128, 1),
    ("kda", "f32", 1, 50, 2, 32, 64, 1),
    ("gdn", "bf16", 2, 90, 2, 64, 32, 1),
    ("deltaproduct", "f32", 1, 40, 2, 64, 64, 2),
    ("deltaproduct", "bf16", 1, 60, 2, 128, 128, 3),
    ("asym", "f32", 2, 64, 3, 64, 64, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("with_s0", [False, True])
def test_recurrent_vs_oracle(case, with_s0):
    from gpu_util import TOL, host, run_recurrent
    var, dt, B, T, H, dk, dv, n_h = case
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=7, n_h=n_h)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=3) if with_s0 else None
    print(f"recurrent {case} s0={with_s0}", flush=True)
    o, S = run_recurrent(inp, s0)
    o_ref, S_ref = oracle.forward(inp, s0)
    tol = TOL[dt]
    assert oracle.rel_l2(host(o), o_ref) <= tol["rel_l2"]
    assert oracle.max_rel(host(o), o_ref) <= tol["max_rel"]
    assert oracle.rel_l2(host(S), S_ref) <= tol["rel_l2"]
    assert oracle.max_rel(host(S), S_ref) <= tol["max_rel"]


def test_recurrent_fg2_plus():
    from gpu_util import TOL, host, run_recurrent
    inp = gdn_inputs.make_inputs("fg2", 1, 70, 2, 64, 32, dtype="f32", seed=9, fg2_plus=True)
    o, S = run_recurrent(inp)
    o_ref, S_ref = oracle.forward(inp)
    assert oracle.rel_l2(host(o), o_ref) <= TOL["f32"]["rel_l2"]
    assert oracle.rel_l2(host(S), S_ref) <= TOL["f32"]["rel_l2"]


def test_recurrent_split_equals_whole():
    """Two calls over [0, t1) and [t1, T) from the returned state equal one call."""
    from gpu_util import host, run_recurrent
    inp = gdn_inputs.make_inputs("fg2", 1, 41, 2, 32, 32, dtype="f32", seed=11)
    o, S = run_recurrent(inp)
    o1, S1 = run_recurrent(gdn_inputs.slice_tokens(inp, 0, 17))
    o2, S2 = run_recurrent(gdn_inputs.slice_tokens(inp, 17, 41), S1.cpu().numpy())
    np.testing.assert_array_equal(np.concatenate([host(o1), host(o2)], axis=1), host(o))
    np.testing.assert_array_equal(host(S2), host(S))
