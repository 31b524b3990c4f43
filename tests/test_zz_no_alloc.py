"""gdn_chunk_fwd_static (the library's own record buffer, no allocation in the call)
against gdn_chunk_fwd with a workspace, through the C ABI: o and the final state must
be bitwise equal. Two calls in a row, the second on a smaller input, so the second
runs on a buffer that still holds the first call's records."""
import numpy as np
import pytest
import torch

import gdn_inputs

pytestmark = pytest.mark.gpu


def _pair(var, dt, B, T, H, dk, dv, chunk, *, with_sfinal, seed, n_h=1, alpha_mean=3.0, fg2_plus=False):
    import gated_delta_rule_69_amd as gdn
    from gpu_util import DEV, host, run_chunk, state_to_dev, to_dev
    inp = gdn_inputs.make_inputs(var, B, T, H, dk, dv, dtype=dt, seed=seed, n_h=n_h, alpha_mean=alpha_mean,
                                 fg2_plus=fg2_plus)
    s0 = gdn_inputs.make_state(B, H, dk, dv, seed=seed)
    print(f"static entry: {var} {dt} B{B} T{T} H{H} dk{dk} dv{dv} C{chunk} s_final={with_sfinal}", flush=True)
    o_ref, S_ref = run_chunk(inp, s0, chunk=chunk)
    d = to_dev(inp)
    o = torch.full_like(o_ref, float("nan"))
    s_final = torch.full((B, H, dk, dv), float("nan"), device=DEV) if with_sfinal else None
    a = gdn.make_args(var, d["q"], d["k"], d["v"], d["alpha"], d.get("beta"), chunk=chunk, j=d.get("j"),
                      eta=d.get("eta"), beta_v=d.get("beta_v"), s0=state_to_dev(s0), s_final=s_final, o=o)
    gdn.gdn_chunk_fwd_static(a)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o), host(o_ref))
    if with_sfinal:
        np.testing.assert_array_equal(host(s_final), host(S_ref))


def test_static_entry_two_calls_second_smaller():
    # 32 sequences of 128 chunks: the buffer holds 28 chunks of each, five blocks
    _pair("fg2", "bf16", 2, 8192, 16, 128, 128, 64, with_sfinal=True, seed=91)
    # smaller, the state carried inside the buffer (no s_final), one block
    _pair("kda", "f32", 1, 300, 4, 64, 64, 32, with_sfinal=False, seed=92)


def test_static_entry_blocks_without_s_final_and_strong_decay():
    # several blocks with the carried state inside the buffer, then a smaller call
    _pair("fg2", "bf16", 2, 4096, 16, 128, 128, 64, with_sfinal=False, seed=93, alpha_mean=-3.0)
    _pair("deltaproduct", "bf16", 1, 500, 4, 128, 128, 64, with_sfinal=True, seed=94, n_h=2)


def test_static_entry_value_side_beta_and_eight_row_chunks():
    # FG2+ on the two-workgroup prepare kernel over several blocks, then DeltaProduct
    # with eight steps a token (8 output rows a chunk) over several blocks
    _pair("fg2", "bf16", 2, 4096, 16, 128, 128, 64, with_sfinal=True, seed=95, fg2_plus=True)
    _pair("deltaproduct", "bf16", 1, 1200, 8, 128, 128, 64, with_sfinal=True, seed=96, n_h=8)
