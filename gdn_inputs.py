"""Seeded synthetic inputs for the gated delta rule forward pass.

This module draws random numbers and shapes them into the arrays a caller hands
to the library (and to the float64 checker). It holds none of the recurrence's
arithmetic: no decay, no key/value scaling, no state update. It is the one
module that both the HIP path's tests/bench and the CPU oracle's tests import.

Recipe (the same for every caller):
  * generator: ``numpy.random.default_rng(seed)``;
  * draw order: q, k, v, alpha-logits, beta-logits, beta_v-logits, j-noise,
    eta-logits, gate-logits (each only where the variant uses it);
  * draws are float64; keys (and j) are L2-normalised per token and head in
    float64; everything is then cast to float32 and, for bf16 workloads,
    rounded to bfloat16 (round to nearest even). The arrays returned are float32
    holding exactly the values the device will see.

Distributions follow the workload definitions of the FG2-GDN, DeltaProduct and
GDN2/RWKV-7 pages: q, v ~ N(0,1); k ~ N(0,1) then unit L2 norm; per-channel
alpha = sigmoid(N(3,1)); beta = sigmoid(N(0,1)); DeltaProduct beta_j =
2*sigmoid(N(0,1)) with a per-(token, head) gate sigmoid(N(3,1)); GDN2 D =
sigmoid(N(3,1)) per channel, eta = 0.5*sigmoid(N(0,1)) per (token, head) and
j = normalize(k + 0.3*N(0, I)).
"""
from __future__ import annotations

import numpy as np

VARIANTS = ("fg2", "kda", "gdn", "deltaproduct", "asym")

# The workloads. Index 2 is the long-context prefill that throughput is quoted on.
CONFIGS = [
    dict(index=0, name="fg2_tiny_f32", variant="fg2", B=1, H=1, T=64, dk=16, dv=16,
         chunk=16, n_h=1, dtype="f32"),
    dict(index=1, name="fg2_prefill_4k_bf16", variant="fg2", B=1, H=16, T=4096, dk=128,
         dv=128, chunk=64, n_h=1, dtype="bf16"),
    dict(index=2, name="fg2_prefill_32k_bf16", variant="fg2", B=2, H=16, T=32768, dk=128,
         dv=128, chunk=64, n_h=1, dtype="bf16"),
    dict(index=3, name="deltaproduct2_8k_bf16", variant="deltaproduct", B=4, H=8, T=8192,
         dk=128, dv=128, chunk=64, n_h=2, dtype="bf16"),
    dict(index=4, name="gdn2_asym_2k_f32", variant="asym", B=8, H=32, T=2048, dk=64, dv=64,
         chunk=32, n_h=1, dtype="f32"),
]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _finish(x64: np.ndarray, dtype: str) -> np.ndarray:
    x = x64.astype(np.float32)
    if dtype == "bf16":
        x = round_bf16(x)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_inputs(variant: str, B: int, T: int, H: int, dk: int, dv: int, *,
                dtype: str = "f32", seed: int = 0, n_h: int = 1,
                fg2_plus: bool = False, alpha_mean: float = 3.0,
                beta_scale: float = 1.0) -> dict:
    """Draw one batch of inputs for ``variant``.

    Layouts (row-major):
      q, k, v, o:        [B, T, H, d]   (DeltaProduct k, v: [B, T, H, n_h, d])
      fg2   alpha, beta: [B, T, H, dk]; beta_v [B, T, H, dv] when fg2_plus
      kda   alpha [B, T, H, dk], beta [B, T, H]
      gdn   alpha, beta: [B, T, H]
      deltaproduct  beta [B, T, H, n_h], alpha (the forget gate) [B, T, H]
      asym  alpha (the diagonal D) [B, T, H, dk], j [B, T, H, dk], eta [B, T, H]

    ``alpha_mean`` moves the mean of the forget-gate logits (3.0 in every
    workload); ``beta_scale`` widens the write-rate logits (1.0 in every workload;
    1.93 gives the 5th/95th percentiles 0.04/0.96 reported for trained FG2 gates).
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    rng = np.random.default_rng(seed)
    out = {"variant": variant, "dtype": dtype, "B": B, "T": T, "H": H, "dk": dk,
           "dv": dv, "n_h": n_h}
    kshape = (B, T, H, n_h, dk) if variant == "deltaproduct" else (B, T, H, dk)
    vshape = (B, T, H, n_h, dv) if variant == "deltaproduct" else (B, T, H, dv)
    out["q"] = _finish(rng.standard_normal((B, T, H, dk)), dtype)
    k64 = _unit(rng.standard_normal(kshape))
    out["k"] = _finish(k64, dtype)
    out["v"] = _finish(rng.standard_normal(vshape), dtype)
    if variant in ("fg2", "kda", "asym"):
        out["alpha"] = _finish(_sigmoid(alpha_mean + rng.standard_normal((B, T, H, dk))), dtype)
    elif variant == "gdn":
        out["alpha"] = _finish(_sigmoid(alpha_mean + rng.standard_normal((B, T, H))), dtype)
    if variant == "fg2":
        out["beta"] = _finish(_sigmoid(beta_scale * rng.standard_normal((B, T, H, dk))), dtype)
        if fg2_plus:
            out["beta_v"] = _finish(_sigmoid(beta_scale * rng.standard_normal((B, T, H, dv))),
                                    dtype)
    elif variant in ("kda", "gdn"):
        out["beta"] = _finish(_sigmoid(beta_scale * rng.standard_normal((B, T, H))), dtype)
    elif variant == "deltaproduct":
        out["beta"] = _finish(2.0 * _sigmoid(beta_scale * rng.standard_normal((B, T, H, n_h))),
                              dtype)
    if variant == "asym":
        j64 = _unit(k64 + 0.3 * rng.standard_normal((B, T, H, dk)))
        out["j"] = _finish(j64, dtype)
        out["eta"] = _finish(0.5 * _sigmoid(rng.standard_normal((B, T, H))), dtype)
    if variant == "deltaproduct":
        out["alpha"] = _finish(_sigmoid(alpha_mean + rng.standard_normal((B, T, H))), dtype)
    return out


def make_state(B: int, H: int, dk: int, dv: int, *, seed: int = 0,
               scale: float = 0.1) -> np.ndarray:
    """A nonzero initial state [B, H, dk, dv], float32, ``scale * N(0, 1)``."""
    rng = np.random.default_rng(10_000 + seed)
    return (scale * rng.standard_normal((B, H, dk, dv))).astype(np.float32)


def config_inputs(index: int, *, seed: int | None = None, T: int | None = None,
                  B: int | None = None) -> dict:
    """Inputs of workload ``index`` (seed defaults to the index); T and B may be cut."""
    c = CONFIGS[index]
    return make_inputs(c["variant"], B if B is not None else c["B"],
                       T if T is not None else c["T"], c["H"], c["dk"], c["dv"],
                       dtype=c["dtype"], seed=index if seed is None else seed,
                       n_h=c["n_h"])


def slice_tokens(inp: dict, t0: int, t1: int) -> dict:
    """The same inputs restricted to tokens [t0, t1) (axis 1 of every array)."""
    out = dict(inp)
    for key in ("q", "k", "v", "alpha", "beta", "beta_v", "j", "eta"):
        if key in inp:
            out[key] = np.ascontiguousarray(inp[key][:, t0:t1])
    out["T"] = t1 - t0
    return out
