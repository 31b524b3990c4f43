"""Chunkwise path (gdn_chunk_fwd / gdn_final_state) against the float64 oracle.

Tolerances (rel-L2 / normwise max-rel, for o and S_T): fp32 inputs 1e-5 / 1e-4,
bf16 inputs 5e-3 / 2e-2, both against the oracle run on the same (bf16-rounded)
inputs.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
import oracle

pytestmark = pytest.mark.gpu


def _check(o, S, o_ref, S_ref, dtype, what=""):
    from gpu_util import TOL, host
    tol = TOL[dtype]
    errs = dict(o_l2=oracle.rel_l2(host(o), o_ref), o_max=oracle.max_rel(host(o), o_ref),
                S_l2=oracle.rel_l2(host(S), S_ref), S_max=oracle.max_rel(host(S), S_ref))
    print(what, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["o_l2"] <= tol["rel_l2"], errs
    assert errs["o_max"] <= tol["max_rel"], errs
    assert errs["S_l2"] <= tol["rel_l2"], errs
    assert errs["S_max"] <= tol["max_rel"], errs


def _run_and_check(inp, s0=None, chunk=64, what=""):
    from gpu_util import run_chunk
    print(f"chunk_fwd {what} chunk={chunk}", flush=True)
    o, S = run_chunk(inp, s0, chunk=chunk)
    o_ref, S_ref = oracle.forward(inp, s0)
    _check(o, S, o_ref, S_ref, inp["dtype"], what)
    return o, S


# ---- the five workloads --------------------------------------------------------

def test_config0_full():
    inp = gdn_inputs.config_inputs(0)
    _run_and_check(inp, chunk=gdn_inputs.CONFIGS[0]["chunk"], what="config0")


def test_config1_full():
    inp = gdn_inputs.config_inputs(1)
    _run_and_check(inp, chunk=64, what="config1")


def test_config2_full_size_sampled_heads():
    """The 32K prefill at its full shape; the oracle checks two (batch, head) pairs."""
    from gpu_util import TOL, host, run_chunk
    inp = gdn_inputs.config_inputs(2)
    o, S = run_chunk(inp, chunk=64)
    torch.cuda.synchronize()
    for b, h in ((0, 3), (1, 14)):
        sub = {k: (v[b:b + 1, :, h:h + 1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        sub["B"], sub["H"] = 1, 1
        o_ref, S_ref = oracle.forward(sub)
        _check(o[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1], o_ref, S_ref, "bf16", f"config2 b{b} h{h}")
    assert np.isfinite(host(o)).all() and np.isfinite(host(S)).all()
    del TOL


def test_config3_deltaproduct_cut():
    inp = gdn_inputs.config_inputs(3, B=1, T=1024)
    _run_and_check(inp, chunk=64, what="config3 (B=1, T=1024)")


def test_config4_asym_cut():
    inp = gdn_inputs.config_inputs(4, B=1, T=512)
    _run_and_check(inp, chunk=gdn_inputs.CONFIGS[4]["chunk"], what="config4 (B=1, T=512)")


@pytest.mark.parametrize("idx,pairs", [(3, ((0, 2), (3, 7))), (4, ((0, 5), (7, 30)))])
def test_config_full_size_sampled_heads(idx, pairs):
    """DeltaProduct (B4 H8 T8192, n_h 2) and GDN2 (B8 H32 T2048 fp32) at their full
    shapes, in the launch configuration of bench.py --configs; the oracle checks two
    (batch, head) pairs of each."""
    from gpu_util import host, run_chunk
    cfg = gdn_inputs.CONFIGS[idx]
    inp = gdn_inputs.config_inputs(idx)
    o, S = run_chunk(inp, chunk=cfg["chunk"])
    torch.cuda.synchronize()
    for b, h in pairs:
        sub = {k: (v[b:b + 1, :, h:h + 1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        sub["B"], sub["H"] = 1, 1
        o_ref, S_ref = oracle.forward(sub)
        _check(o[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1], o_ref, S_ref, cfg["dtype"],
               f"config{idx} b{b} h{h}")
    assert np.isfinite(host(o)).all() and np.isfinite(host(S)).all()


# ---- variants, dtypes, shapes, chunk sizes --------------------------------------

CASES = [
    # variant, dtype, B, T, H, dk, dv, n_h, chunk
    ("fg2", "f32", 1, 200, 2, 64, 64, 1, 64),
    ("fg2", "f32", 2, 100, 2, 32, 32, 1, 32),
    ("fg2", "f32", 1, 90, 2, 16, 16, 1, 16),
    ("fg2", "f32", 1, 150, 2, 128, 128, 1, 32),
    ("fg2", "f32", 1, 150, 2, 128, 128, 1, 64),          # runs with 32-step chunks
    ("deltaproduct", "f32", 1, 70, 2, 128, 128, 2, 64),  # likewise
    ("deltaproduct", "f32", 1, 45, 2, 64, 32, 3, 64),     # 3 steps padded to 4
    ("deltaproduct", "bf16", 2, 50, 2, 64, 64, 3, 64),
    ("fg2", "bf16", 1, 517, 3, 128, 128, 1, 64),
    ("fg2", "bf16", 2, 333, 2, 64, 64, 1, 32),
    ("fg2", "bf16", 1, 257, 2, 32, 32, 1, 16),
    ("kda", "f32", 1, 130, 2, 64, 128, 1, 64),
    ("kda", "bf16", 1, 300, 2, 128, 64, 1, 64),
    ("gdn", "f32", 2, 97, 2, 32, 64, 1, 32),
    ("gdn", "bf16", 1, 260, 4, 128, 128, 1, 64),
    ("deltaproduct", "f32", 1, 100, 2, 64, 64, 2, 64),
    ("deltaproduct", "f32", 1, 70, 2, 32, 32, 1, 16),
    ("deltaproduct", "bf16", 1, 300, 2, 128, 128, 2, 64),
    ("deltaproduct", "bf16", 1, 130, 2, 64, 64, 4, 64),
    ("deltaproduct", "bf16", 1, 99, 2, 128, 128, 2, 32),
    ("asym", "f32", 1, 200, 2, 64, 64, 1, 32),
    ("asym", "f32", 1, 100, 2, 64, 64, 1, 64),
    ("asym", "f32", 1, 100, 2, 64, 64, 1, 16),
    ("asym", "bf16", 1, 256, 2, 128, 128, 1, 64),
    # bf16, dk 128, chunk 64: fragment-format records and the row-split scan,
    # every value width and output-row count it handles
    ("kda", "bf16", 1, 200, 2, 128, 32, 1, 64),
    ("gdn", "bf16", 2, 150, 2, 128, 16, 1, 64),
    ("deltaproduct", "bf16", 1, 100, 2, 128, 64, 4, 64),
    ("asym", "bf16", 1, 190, 3, 128, 64, 1, 64),
    # bf16, dk = dv = 128, chunk 64, DeltaProduct with 2 or 4 steps per token (ragged
    # ends): two-workgroup prepare kernel with multi-step rows
    ("deltaproduct", "bf16", 2, 77, 2, 128, 128, 4, 64),
    ("deltaproduct", "bf16", 1, 90, 2, 128, 128, 3, 64),   # 3 steps padded to 4
    ("deltaproduct", "bf16", 1, 161, 3, 128, 128, 2, 64),
    # bf16, dk = dv = 128, chunk 64, one step per token: two-workgroup prepare kernel
    ("kda", "bf16", 2, 170, 2, 128, 128, 1, 64),
    ("deltaproduct", "bf16", 1, 200, 2, 128, 128, 1, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("with_s0", [False, True])
def test_chunk_vs_oracle(case, with_s0):
    var, dt, B, T, H, dk, dv, n_h, chunk = case
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=5, n_h=n_h)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=4) if with_s0 else None
    _run_and_check(inp, s0, chunk=chunk, what=f"{case} s0={with_s0}")


# DeltaProduct chunks with 8 output rows (half of one 16-row tile): 8 steps a token
# (n_h 5..7 padded with identity steps), or 4 (n_h 3, 4) in 32-step chunks, or 2 in
# 16-step chunks; both scans (fragment records at bf16 dk 128, image records else)
EIGHT_ROWS = [
    # variant, dtype, B, T, H, dk, dv, n_h, chunk
    ("deltaproduct", "bf16", 1, 50, 2, 128, 128, 8, 64),
    ("deltaproduct", "bf16", 2, 37, 2, 128, 128, 5, 64),
    ("deltaproduct", "f32", 1, 41, 2, 64, 64, 6, 64),
    ("deltaproduct", "f32", 1, 20, 1, 16, 16, 7, 64),
    ("deltaproduct", "f32", 1, 40, 2, 128, 128, 4, 64),   # fp32 dk 128: 32-step chunks
    ("deltaproduct", "bf16", 1, 45, 2, 64, 64, 3, 32),
    ("deltaproduct", "bf16", 1, 33, 2, 32, 32, 2, 16),
]


@pytest.mark.parametrize("case", EIGHT_ROWS, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("with_s0", [False, True])
def test_deltaproduct_eight_output_rows(case, with_s0):
    var, dt, B, T, H, dk, dv, n_h, chunk = case
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=60 + n_h, n_h=n_h)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=61) if with_s0 else None
    _run_and_check(inp, s0, chunk=chunk, what=f"{case} s0={with_s0}")


def test_deltaproduct_eight_steps_strong_decay():
    inp = gdn_inputs.make_inputs("deltaproduct", 1, 60, 2, 128, 128, dtype="bf16", seed=62, n_h=8,
                                 alpha_mean=-3.0)
    s0 = gdn_inputs.make_state(1, 2, 128, 128, seed=63)
    _run_and_check(inp, s0, chunk=64, what="dp n_h 8 strong decay")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fg2_plus(dt):
    inp = gdn_inputs.make_inputs("fg2", 1, 211, 2, 64, 128, dtype=dt, seed=12, fg2_plus=True)
    _run_and_check(inp, chunk=64 if dt == "bf16" else 32, what=f"fg2+ {dt}")


def test_fg2_plus_fragment_records():
    """FG2+ (separate value-side beta) with dk 128, dv 64, chunk 64, bf16."""
    inp = gdn_inputs.make_inputs("fg2", 1, 300, 2, 128, 64, dtype="bf16", seed=14, fg2_plus=True)
    s0 = gdn_inputs.make_state(1, 2, 128, 64, seed=14)
    _run_and_check(inp, s0, chunk=64, what="fg2+ dk128 dv64")


@pytest.mark.parametrize("T,alpha_mean", [(1, 3.0), (130, 3.0), (300, 3.0), (300, -3.0)])
def test_fg2_plus_two_workgroup_prepare(T, alpha_mean):
    """FG2+ with dk = dv = 128, chunk 64, bf16: the two-workgroup prepare kernel with a
    value-side beta row, on mild decay (the mid-chunk pass) and on strong decay (the
    flagged chunks' tile-referenced pass), ragged ends and a nonzero initial state."""
    inp = gdn_inputs.make_inputs("fg2", 1, T, 2, 128, 128, dtype="bf16", seed=15 + T, fg2_plus=True,
                                 alpha_mean=alpha_mean)
    s0 = gdn_inputs.make_state(1, 2, 128, 128, seed=16)
    _run_and_check(inp, s0, chunk=64, what=f"fg2+ dk128 dv128 T={T} alpha_mean={alpha_mean}")


@pytest.mark.parametrize("T", [1, 63, 65, 130])
def test_short_and_ragged_fragment_records(T):
    inp = gdn_inputs.make_inputs("fg2", 1, T, 2, 128, 128, dtype="bf16", seed=40 + T)
    s0 = gdn_inputs.make_state(1, 2, 128, 128, seed=T)
    _run_and_check(inp, s0, chunk=64, what=f"T={T} dk128")


def test_wide_beta_and_strong_decay():
    """Write rates spread like trained FG2 gates (5th/95th pct 0.04/0.96) and a
    faster forget gate (mean alpha ~0.73)."""
    inp = gdn_inputs.make_inputs("fg2", 1, 400, 2, 128, 128, dtype="bf16", seed=13,
                                 beta_scale=1.93, alpha_mean=1.0)
    _run_and_check(inp, chunk=64, what="wide beta, strong decay")


# ---- strong decay ------------------------------------------------------------------
# alpha in (0, 1) is the whole domain (FG2-GDN reading notes, section 2.2 eq. (11);
# GDN2-stability page, "Problem Description"). Forget-gate logits centred at -2, -3
# and -6 put the mean alpha near 0.15, 0.07 and 0.0035, so a chunk's decay reaches
# far below the float32 range; every case runs with a nonzero initial state.
STRONG = [
    # variant, dtype, B, T, H, dk, dv, n_h, chunk
    ("fg2", "bf16", 1, 300, 2, 128, 128, 1, 64),       # two-workgroup prepare kernel
    ("kda", "bf16", 1, 300, 2, 128, 128, 1, 64),
    ("gdn", "bf16", 1, 300, 2, 128, 128, 1, 64),
    ("asym", "bf16", 1, 300, 2, 128, 128, 1, 64),
    ("deltaproduct", "bf16", 1, 150, 2, 128, 128, 2, 64),
    ("deltaproduct", "bf16", 1, 90, 2, 128, 128, 3, 64),  # 3 steps padded to 4 a token
    ("fg2", "f32", 1, 300, 2, 64, 64, 1, 32),          # generic prepare kernel, fp32
    ("kda", "f32", 1, 300, 2, 64, 64, 1, 32),
    ("gdn", "f32", 1, 300, 2, 64, 64, 1, 32),
    ("asym", "f32", 1, 300, 2, 64, 64, 1, 32),
    ("fg2", "f32", 1, 200, 2, 32, 32, 1, 64),          # generic, chunk 64 (four tiles)
    ("kda", "bf16", 1, 300, 2, 64, 64, 1, 64),
    ("fg2", "bf16", 1, 200, 2, 64, 64, 1, 16),         # one tile per chunk
    ("deltaproduct", "f32", 1, 100, 2, 64, 64, 2, 64),  # several steps per token, fp32
    ("deltaproduct", "bf16", 1, 100, 2, 64, 64, 2, 32),
]


@pytest.mark.parametrize("alpha_mean", [-2.0, -3.0, -6.0])
@pytest.mark.parametrize("case", STRONG, ids=lambda c: "-".join(map(str, c)))
def test_strong_decay(case, alpha_mean):
    var, dt, B, T, H, dk, dv, n_h, chunk = case
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=81, n_h=n_h, alpha_mean=alpha_mean)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=81, scale=1.0)
    _run_and_check(inp, s0, chunk=chunk, what=f"strong decay {case} alpha_mean={alpha_mean}")


@pytest.mark.parametrize("case", [
    ("fg2", "bf16", 1, 400, 2, 128, 128, 64),
    ("kda", "bf16", 1, 400, 2, 128, 128, 64),
    ("asym", "bf16", 1, 300, 2, 128, 128, 64),
    ("fg2", "bf16", 1, 300, 2, 64, 64, 64),
    ("fg2", "f32", 1, 300, 2, 64, 64, 32),
    ("kda", "f32", 1, 200, 2, 32, 32, 64),
], ids=lambda c: "-".join(map(str, c)))
def test_some_channels_forget_at_once(case):
    """Every seventh key channel has alpha = 1e-4 at every step (ordinary gates on the
    rest): those channels lose almost all of the state at each step while the others
    keep it, inside the same chunk."""
    var, dt, B, T, H, dk, dv, chunk = case
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=82)
    al = inp["alpha"].copy()
    al[..., ::7] = 1e-4
    inp["alpha"] = gdn_inputs.round_bf16(al) if dt == "bf16" else al.astype(np.float32)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=82, scale=1.0)
    _run_and_check(inp, s0, chunk=chunk, what=f"alpha 1e-4 channels {case}")


# ---- magnitudes of the caller's values -----------------------------------------------
# The bf16 path feeds v, q, the state and U to fp16 MFMAs with exact power-of-two
# scales (per chunk for the written values, per output row for q, per wave block and
# column for the state and U), so its relative accuracy must not depend on how large
# or small the caller's values are, nor on a change of magnitude between chunks.
# Powers of two keep the bf16 inputs exact; the oracle sees the same values.
MAG_SHAPES = [
    # variant, dtype, dk, dv, chunk
    ("fg2", "bf16", 128, 128, 64),    # two-workgroup prepare, row-split scan
    ("kda", "bf16", 128, 32, 64),     # general prepare, row-split scan
    ("fg2", "bf16", 64, 64, 64),      # image records, image scan
    ("gdn", "bf16", 32, 64, 32),
]
MAGNITUDES = [
    # scale of v, of q, of the initial state (0: none)
    (2.0 ** 14, 1.0, 0.0),
    (2.0 ** -14, 1.0, 0.0),
    (1.0, 2.0 ** 14, 0.0),
    (1.0, 2.0 ** -14, 1.0),
    (2.0 ** -12, 1.0, 2.0 ** 10),        # the state dominates every write
    (2.0 ** 12, 2.0 ** -12, 2.0 ** -12),  # the writes dominate the state
]


@pytest.mark.parametrize("mag", MAGNITUDES, ids=lambda m: "v%g-q%g-s%g" % m)
@pytest.mark.parametrize("shape", MAG_SHAPES, ids=lambda c: "-".join(map(str, c)))
def test_value_magnitudes(shape, mag):
    var, dt, dk, dv, chunk = shape
    vs, qs, ss = mag
    inp = gdn_inputs.make_inputs(var, 1, 200, 2, dk, dv, dtype=dt, seed=91)
    inp["v"] = (inp["v"] * np.float32(vs)).astype(np.float32)
    inp["q"] = (inp["q"] * np.float32(qs)).astype(np.float32)
    s0 = gdn_inputs.make_state(1, 2, dk, dv, seed=91, scale=1.0) * np.float32(ss) if ss else None
    _run_and_check(inp, s0, chunk=chunk, what=f"magnitudes {shape} v {vs:g} q {qs:g} s0 {ss:g}")


@pytest.mark.parametrize("shape", MAG_SHAPES, ids=lambda c: "-".join(map(str, c)))
def test_value_magnitude_changes_between_chunks(shape):
    """The written values jump by 2^12 for one chunk, then fall to 2^-12 of their
    size: every chunk's outputs are checked on their own (a whole-tensor norm would
    be dominated by the loud chunk)."""
    from gpu_util import TOL, host, run_chunk
    var, dt, dk, dv, chunk = shape
    T = 6 * chunk
    inp = gdn_inputs.make_inputs(var, 1, T, 2, dk, dv, dtype=dt, seed=92)
    v = inp["v"].copy()
    v[:, 2 * chunk:3 * chunk] *= np.float32(2.0 ** 12)
    v[:, 4 * chunk:] *= np.float32(2.0 ** -12)
    inp["v"] = v
    s0 = gdn_inputs.make_state(1, 2, dk, dv, seed=92, scale=1.0)
    print(f"chunk_fwd magnitude jumps {shape}", flush=True)
    o, S = run_chunk(inp, s0, chunk=chunk)
    o_ref, S_ref = oracle.forward(inp, s0)
    got, tol = host(o), TOL[dt]
    for c in range(T // chunk):
        seg = slice(c * chunk, (c + 1) * chunk)
        e = oracle.rel_l2(got[:, seg], o_ref[:, seg])
        m = oracle.max_rel(got[:, seg], o_ref[:, seg])
        assert e <= tol["rel_l2"] and m <= tol["max_rel"], (c, e, m)
    assert oracle.rel_l2(host(S), S_ref) <= tol["rel_l2"]
    assert oracle.max_rel(host(S), S_ref) <= tol["max_rel"]


@pytest.mark.parametrize("T", [1, 5, 16, 63, 64, 65])
def test_short_and_ragged(T):
    inp = gdn_inputs.make_inputs("fg2", 1, T, 2, 64, 64, dtype="bf16", seed=T)
    s0 = gdn_inputs.make_state(1, 2, 64, 64, seed=T)
    _run_and_check(inp, s0, chunk=64, what=f"T={T}")


def test_T_zero_copies_state():
    from gpu_util import host, run_chunk
    inp = gdn_inputs.make_inputs("fg2", 1, 0, 2, 32, 32, dtype="f32", seed=1)
    s0 = gdn_inputs.make_state(1, 2, 32, 32, seed=1)
    _, S = run_chunk(inp, s0, chunk=32)
    np.testing.assert_array_equal(host(S), s0.astype(np.float64))
    _, S = run_chunk(inp, None, chunk=32)
    assert not host(S).any()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chunk_size_invariance(dt):
    """C = 16, 32, 64 give the same result up to the tolerance of each."""
    from gpu_util import host, run_chunk
    inp = gdn_inputs.make_inputs("kda", 1, 300, 2, 64, 64, dtype=dt, seed=21)
    outs = [run_chunk(inp, chunk=c) for c in (16, 32, 64)]
    o0, S0 = host(outs[0][0]), host(outs[0][1])
    tol = 3e-6 if dt == "f32" else 4e-3
    for o, S in outs[1:]:
        assert oracle.rel_l2(host(o), o0) <= tol
        assert oracle.rel_l2(host(S), S0) <= tol


def test_split_sequence_state_passing():
    from gpu_util import host, run_chunk
    inp = gdn_inputs.make_inputs("fg2", 1, 300, 2, 64, 64, dtype="f32", seed=31)
    o, S = run_chunk(inp, chunk=64)
    o1, S1 = run_chunk(gdn_inputs.slice_tokens(inp, 0, 128), chunk=64)
    o2, S2 = run_chunk(gdn_inputs.slice_tokens(inp, 128, 300), S1.cpu().numpy(), chunk=64)
    assert oracle.rel_l2(np.concatenate([host(o1), host(o2)], axis=1), host(o)) <= 1e-6
    assert oracle.rel_l2(host(S2), host(S)) <= 1e-6


def test_chunk_matches_recurrent():
    from gpu_util import host, run_chunk, run_recurrent
    inp = gdn_inputs.make_inputs("asym", 1, 150, 2, 64, 64, dtype="f32", seed=41)
    s0 = gdn_inputs.make_state(1, 2, 64, 64, seed=41)
    o1, S1 = run_chunk(inp, s0, chunk=32)
    o2, S2 = run_recurrent(inp, s0)
    assert oracle.rel_l2(host(o1), host(o2)) <= 1e-5
    assert oracle.rel_l2(host(S1), host(S2)) <= 1e-5


def test_final_state_entry_and_aliasing():
    import gated_delta_rule_69_amd as gdn
    from gpu_util import host, run_chunk, state_to_dev, to_dev
    inp = gdn_inputs.make_inputs("fg2", 1, 333, 2, 128, 128, dtype="bf16", seed=51)
    s0 = gdn_inputs.make_state(1, 2, 128, 128, seed=51)
    _, S = run_chunk(inp, s0, chunk=64)
    d = to_dev(inp)
    S_only = gdn.gdn_final_state("fg2", d["k"], d["v"], d["alpha"], d["beta"], chunk=64,
                                 s0=state_to_dev(s0))
    np.testing.assert_array_equal(host(S_only), host(S))
    st = state_to_dev(s0)
    gdn.gdn_chunk_fwd("fg2", d["q"], d["k"], d["v"], d["alpha"], d["beta"], chunk=64, s0=st,
                      s_final=st)
    np.testing.assert_array_equal(host(st), host(S))


def test_bitwise_determinism():
    from gpu_util import host, run_chunk
    inp = gdn_inputs.make_inputs("fg2", 2, 700, 4, 128, 128, dtype="bf16", seed=61)
    o1, S1 = run_chunk(inp, chunk=64)
    o2, S2 = run_chunk(inp, chunk=64)
    np.testing.assert_array_equal(host(o1), host(o2))
    np.testing.assert_array_equal(host(S1), host(S2))


# ---- degenerate gates and the largest head count ----------------------------------

def test_no_write_keeps_decayed_state():
    """beta = 0: nothing is written or erased, so S_T = Diag(prod_t alpha_t) S_0 and
    o_t = S_t^T q_t (closed form, float64)."""
    from gpu_util import host, run_chunk
    inp = gdn_inputs.make_inputs("fg2", 1, 130, 2, 64, 64, dtype="f32", seed=71)
    inp["beta"] = np.zeros_like(inp["beta"])
    s0 = gdn_inputs.make_state(1, 2, 64, 64, seed=71, scale=1.0)
    o, S = run_chunk(inp, s0, chunk=32)
    al = inp["alpha"].astype(np.float64)                   # [1, T, H, dk]
    cum = np.cumprod(al, axis=1)                           # decay through token t
    St = cum[0][:, :, :, None] * s0[0][None].astype(np.float64)   # [T, H, dk, dv]
    o_ref = np.einsum("thkv,thk->thv", St, inp["q"][0].astype(np.float64))[None]
    assert oracle.rel_l2(host(S), St[-1][None]) <= 1e-5
    assert oracle.rel_l2(host(o), o_ref) <= 1e-5


@pytest.mark.parametrize("variant", ["fg2", "kda"])
def test_full_write_recalls_the_value(variant):
    """alpha = 1, beta = 1 and unit keys: each step replaces the value stored along k_t,
    so reading with q_t = k_t returns v_t exactly (the delta rule's defining case)."""
    from gpu_util import host, run_chunk
    inp = gdn_inputs.make_inputs(variant, 1, 100, 2, 32, 32, dtype="f32", seed=72)
    inp["alpha"] = np.ones_like(inp["alpha"])
    inp["beta"] = np.ones_like(inp["beta"])
    inp["q"] = inp["k"].copy()
    s0 = gdn_inputs.make_state(1, 2, 32, 32, seed=72)
    o, _ = run_chunk(inp, s0, chunk=32)
    assert oracle.rel_l2(host(o), inp["v"].astype(np.float64)) <= 1e-5


def test_largest_head_count():
    """B * H = 65536 heads (H at its limit) with a ragged two-chunk sequence: the grids
    of the prepare and scan kernels run past 65,535 workgroups; sampled heads against
    the oracle, the recurrent path against the chunked one."""
    from gpu_util import host, run_chunk, run_recurrent
    inp = gdn_inputs.make_inputs("fg2", 1, 20, 65536, 16, 16, dtype="f32", seed=73)
    o, S = run_chunk(inp, chunk=16)
    o2, S2 = run_recurrent(inp)
    torch.cuda.synchronize()
    for h in (0, 40961, 65535):
        sub = {k: (v[:, :, h:h + 1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        sub["H"] = 1
        o_ref, S_ref = oracle.forward(sub)
        _check(o[:, :, h:h + 1], S[:, h:h + 1], o_ref, S_ref, "f32", f"head {h} of 65536")
    assert oracle.rel_l2(host(o2), host(o)) <= 1e-5
    assert oracle.rel_l2(host(S2), host(S)) <= 1e-5
