"""Helpers for the GPU tests: move seeded numpy inputs to the device and call the
library through its C ABI binding."""
import numpy as np
import torch

import gated_delta_rule_69_amd as gdn

DEV = torch.device("cuda:0")

TOL = {"f32": dict(rel_l2=1e-5, max_rel=1e-4), "bf16": dict(rel_l2=5e-3, max_rel=2e-2)}


def to_dev(inp: dict) -> dict:
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v", "alpha", "beta", "beta_v", "j", "eta"):
        if key in inp:
            out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(DEV).to(dt).contiguous()
    return out


def state_to_dev(s0):
    return None if s0 is None else torch.from_numpy(np.ascontiguousarray(s0, np.float32)).to(DEV)


def run_chunk(inp: dict, s0=None, chunk=None, **kw):
    d = to_dev(inp)
    return gdn.gdn_chunk_fwd(inp["variant"], d.get("q"), d["k"], d["v"], d["alpha"], d.get("beta"),
                             chunk=chunk or 64, beta_v=d.get("beta_v"), j=d.get("j"),
                             eta=d.get("eta"), s0=state_to_dev(s0), **kw)


def run_recurrent(inp: dict, s0=None):
    d = to_dev(inp)
    B, H, dk, dv = inp["B"], inp["H"], inp["dk"], inp["dv"]
    state = state_to_dev(s0) if s0 is not None else torch.zeros((B, H, dk, dv), device=DEV)
    state = state.clone()
    o = gdn.gdn_recurrent_step(inp["variant"], d["q"], d["k"], d["v"], d["alpha"], d.get("beta"),
                               state=state, beta_v=d.get("beta_v"), j=d.get("j"), eta=d.get("eta"))
    return o, state


def host(t):
    return t.float().cpu().numpy().astype(np.float64)
