"""Backward pass of the token recurrence (gdn_recurrent_bwd) against the float64
oracle's gradients (oracle.backward, itself pinned by finite differences).

The kernel computes in float32 from the (bf16-rounded, for bf16) inputs, as the oracle
does in float64 from the same values, so one tolerance covers both input dtypes:
rel-L2 1e-5 and normwise max-rel 1e-4 for every gradient. The pass runs on 16-step
chunks; the cases span one to several chunks, ragged last chunks and several sub-steps
per token.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
import oracle
from oracle import backward as obwd

pytestmark = pytest.mark.gpu

CASES = [  # variant, fg2_plus, dtype, B, T, H, dk, dv
    ("fg2", False, "f32", 1, 70, 2, 16, 16),
    ("fg2", True, "f32", 1, 90, 2, 32, 64),
    ("kda", False, "bf16", 2, 65, 2, 64, 32),
    ("gdn", False, "f32", 1, 130, 3, 32, 16),
    ("asym", False, "f32", 1, 100, 2, 64, 64),
    ("fg2", False, "bf16", 1, 150, 2, 128, 128),
    ("asym", False, "bf16", 1, 66, 1, 128, 64),
    ("deltaproduct", False, "f32", 1, 50, 2, 64, 64),     # 2 steps a token
    ("deltaproduct", False, "bf16", 1, 27, 2, 128, 128),  # 3 steps a token
    # one step, one chunk and a step, exactly four chunks (one operand-ring group of the
    # recursions), several groups and a ragged chunk
    ("fg2", False, "bf16", 1, 1, 2, 128, 128),    # one token
    ("kda", False, "f32", 2, 17, 3, 32, 16),      # one chunk and one step
    ("gdn", False, "bf16", 1, 64, 2, 64, 64),     # four chunks: one ring group
    ("fg2", True, "bf16", 1, 129, 1, 128, 32),    # FG2+, two groups and one step
    ("asym", False, "f32", 1, 48, 2, 16, 128),    # dk 16: lanes past dk idle
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_vs_oracle(case):
    var, plus, dt, B, T, H, dk, dv = case
    n_h = (2 if T % 2 == 0 else 3) if var == "deltaproduct" else 1
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=90, fg2_plus=plus, n_h=n_h)
    _check_backward(inp, case)


def _check_backward(inp, case):
    import gated_delta_rule_69_amd as gdn
    from gpu_util import DEV, host, state_to_dev, to_dev
    var, dt, B, T, H, dk, dv = (inp[k] for k in ("variant", "dtype", "B", "T", "H", "dk", "dv"))
    rng = np.random.default_rng(91)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=92)
    do = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    if dt == "bf16":
        do = gdn_inputs.round_bf16(do)
    dsf = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    ref = obwd.backward(inp, do, s0, dsf)
    d = to_dev(inp)
    io = torch.bfloat16 if dt == "bf16" else torch.float32
    got = gdn.gdn_recurrent_bwd(var, d["q"], d["k"], d["v"], d["alpha"], d.get("beta"),
                                d_o=torch.from_numpy(do).to(DEV).to(io), s0=state_to_dev(s0),
                                ds_final=torch.from_numpy(dsf).to(DEV), beta_v=d.get("beta_v"),
                                j=d.get("j"), eta=d.get("eta"))
    torch.cuda.synchronize()
    assert set(ref) <= set(got), (sorted(ref), sorted(got))
    for name, r in ref.items():
        x = host(got[name])
        e2, em = oracle.rel_l2(x, r), oracle.max_rel(x, r)
        print(case, name, f"rel_l2={e2:.2e} max_rel={em:.2e}", flush=True)
        assert e2 <= 1e-5 and em <= 1e-4, (name, e2, em)


# Strong decay: the backward pass runs in 16-step chunks whose decay factors are split
# at the chunk's step 8, so none spans more than 8 steps (the same window as the
# chunked forward pass). Forget-gate logits centred at -2, -3 and -6 (mean alpha 0.15,
# 0.07, 0.0035) for every variant.
STRONG = [  # variant, dtype, B, T, H, dk, dv
    ("fg2", "bf16", 1, 100, 2, 128, 128),
    ("kda", "f32", 1, 70, 2, 64, 64),
    ("gdn", "f32", 1, 70, 2, 32, 32),
    ("asym", "f32", 1, 70, 2, 64, 64),
    ("deltaproduct", "f32", 1, 40, 2, 64, 64),
]


@pytest.mark.parametrize("alpha_mean", [-2.0, -3.0, -6.0])
@pytest.mark.parametrize("case", STRONG, ids=lambda c: "-".join(map(str, c)))
def test_backward_strong_decay(case, alpha_mean):
    var, dt, B, T, H, dk, dv = case
    n_h = 2 if var == "deltaproduct" else 1
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=97, n_h=n_h, alpha_mean=alpha_mean)
    _check_backward(inp, (case, alpha_mean))


@pytest.mark.parametrize("case", [("fg2", "bf16", 1, 100, 2, 128, 128), ("kda", "f32", 1, 70, 2, 64, 32)],
                         ids=lambda c: "-".join(map(str, c)))
def test_backward_some_channels_forget_at_once(case):
    """Every seventh key channel has alpha = 1e-4 at every step, the others ordinary
    gates, inside the same chunk."""
    var, dt, B, T, H, dk, dv = case
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=98)
    al = inp["alpha"].copy()
    al[..., ::7] = 1e-4
    inp["alpha"] = gdn_inputs.round_bf16(al) if dt == "bf16" else al.astype(np.float32)
    _check_backward(inp, case)


def test_backward_deterministic():
    import gated_delta_rule_69_amd as gdn
    from gpu_util import DEV, to_dev
    inp = gdn_inputs.make_inputs("fg2", 2, 80, 2, 64, 64, dtype="bf16", seed=93)
    d = to_dev(inp)
    do = torch.randn((2, 80, 2, 64), device=DEV).bfloat16()
    r1 = gdn.gdn_recurrent_bwd("fg2", d["q"], d["k"], d["v"], d["alpha"], d["beta"], d_o=do)
    r2 = gdn.gdn_recurrent_bwd("fg2", d["q"], d["k"], d["v"], d["alpha"], d["beta"], d_o=do)
    for name in r1:
        assert torch.equal(r1[name], r2[name]), name


def test_backward_deltaproduct_eight_steps():
    """DeltaProduct with n_h = 8 (72 sub-steps for 9 tokens): q and do act after the
    eighth sub-step of each token, the gate at the first."""
    import gated_delta_rule_69_amd as gdn
    from gpu_util import DEV, host, state_to_dev, to_dev
    inp = gdn_inputs.make_inputs("deltaproduct", 1, 9, 2, 64, 32, dtype="f32", seed=94, n_h=8)
    rng = np.random.default_rng(95)
    s0 = gdn_inputs.make_state(1, 2, 64, 32, seed=96)
    do = rng.standard_normal((1, 9, 2, 32)).astype(np.float32)
    ref = obwd.backward(inp, do, s0, None)
    d = to_dev(inp)
    got = gdn.gdn_recurrent_bwd("deltaproduct", d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                d_o=torch.from_numpy(do).to(DEV), s0=state_to_dev(s0))
    torch.cuda.synchronize()
    for name, r in ref.items():
        x = host(got[name])
        e2, em = oracle.rel_l2(x, r), oracle.max_rel(x, r)
        print("dp n_h 8", name, f"rel_l2={e2:.2e} max_rel={em:.2e}", flush=True)
        assert e2 <= 1e-5 and em <= 1e-4, (name, e2, em)


def test_backward_empty_sequence():
    """T = 0: no step to differentiate; dL/dS_0 is dL/dS_T (zero without it)."""
    import gated_delta_rule_69_amd as gdn
    from gpu_util import DEV
    B, H, d = 2, 3, 64
    z = lambda *sh: torch.zeros(sh, device=DEV, dtype=torch.bfloat16)  # noqa: E731
    q, k, v, al, be = z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d)
    dsf = torch.randn((B, H, d, d), device=DEV)
    got = gdn.gdn_recurrent_bwd("fg2", q, k, v, al, be, d_o=z(B, 0, H, d), ds_final=dsf)
    torch.cuda.synchronize()
    assert torch.equal(got["ds0"], dsf)
    assert all(got[n].numel() == 0 for n in ("dq", "dk", "dv", "dalpha", "dbeta"))
    got = gdn.gdn_recurrent_bwd("fg2", q, k, v, al, be, d_o=z(B, 0, H, d))
    torch.cuda.synchronize()
    assert torch.count_nonzero(got["ds0"]) == 0


@pytest.mark.parametrize("index,pairs", [(1, [(0, 0), (0, 15)]), (3, [(3, 7)]), (4, [(0, 5), (7, 31)])],
                         ids=["workload1", "workload3", "workload4"])
def test_backward_full_size_sampled_heads(index, pairs):
    """Workloads 1 (FG2, bf16, T 4096, H 16, d 128), 3 (DeltaProduct n_h 2, T 8192) and 4
    (ASYM, fp32, d 64, B 8, H 32) at full size: every gradient of the sampled
    (sequence, head) pairs against the oracle, run on that pair alone."""
    import gated_delta_rule_69_amd as gdn
    from gpu_util import DEV, host
    cfg = gdn_inputs.CONFIGS[index]
    inp = gdn_inputs.config_inputs(index)
    B, T, H, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dv"]
    io = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    rng = np.random.default_rng(100 + index)
    do = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    if cfg["dtype"] == "bf16":
        do = gdn_inputs.round_bf16(do)
    t = {n: torch.from_numpy(inp[n]).to(DEV).to(io) for n in ("q", "k", "v", "alpha", "beta", "beta_v", "j", "eta")
         if inp.get(n) is not None}
    got = gdn.gdn_recurrent_bwd(cfg["variant"], t["q"], t["k"], t["v"], t["alpha"], t.get("beta"),
                                d_o=torch.from_numpy(do).to(DEV).to(io), beta_v=t.get("beta_v"),
                                j=t.get("j"), eta=t.get("eta"))
    torch.cuda.synchronize()
    for b, h in pairs:
        sub = {k: (v[b:b + 1, :, h:h + 1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        sub["B"], sub["H"] = 1, 1
        ref = obwd.backward(sub, do[b:b + 1, :, h:h + 1])
        for name, r in ref.items():
            x = host(got[name])
            x = x[b:b + 1, :, h:h + 1] if name != "ds0" else x[b:b + 1, h:h + 1]
            e2, em = oracle.rel_l2(x, r), oracle.max_rel(x, r)
            print(cfg["name"], (b, h), name, f"rel_l2={e2:.2e} max_rel={em:.2e}", flush=True)
            assert e2 <= 1e-5 and em <= 1e-4, (cfg["name"], b, h, name, e2, em)
