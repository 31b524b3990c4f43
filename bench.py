#!/usr/bin/env python3
"""Throughput of the FG2-GDN chunkwise forward pass on one MI355X.

Workload: the long-context prefill B=2, H=16, T=32768, dk=dv=128, chunk 64, bf16
inputs, fp32 state, final states returned. One step = one gdn_chunk_fwd call (its
two stages, gdn_chunk_prepare and gdn_chunk_scan, launched back to back) over
inputs already resident in HBM.

Prints one JSON line on stdout: tokens/s (B*T per step time), the roofline of the
dominant kernel from HIP events around each stage inside the timed region, the
whole path's HBM roofline, a parity check of sampled heads against the float64
oracle, and the oracle's own throughput on the host cores (a reported baseline).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
    python bench.py --sweep     # the pages' prefill sweep (fixed 32,768 tokens), FG2 and KDA
    python bench.py --decode    # one-token decode step over 512 sequences (state in HBM)
    python bench.py --configs   # workloads 0, 1, 3, 4: time per call, both roofline fractions
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn_inputs  # noqa: E402

METRIC = "FG²-GDN chunked prefill tokens/s at 32K (H=16,d=128); % of MFMA/HBM roofline"
WORKLOAD = gdn_inputs.CONFIGS[2]
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "chunk_traffic_fg2_32k.json")
CSRC = os.path.join(ROOT, "gated_delta_rule_69_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work per token-head (dk = dv = d, chunk C, bf16 I/O) ----------------
# prepare: reads q, k, v, alpha, beta (5 d elements); chunk-local products
#          M, P (C d each, triangular halves), W = T B+, U~ = T Wv (C d each).
# scan:    W S, A^T U, Q+ S (2 d^2 each) and P U (C d, triangular); writes o (d).
def prep_bytes_per_th(d, es=2):
    return 5 * d * es


def prep_flops_per_th(d, C):
    return 4 * C * d


def scan_flops_per_th(d, C):
    return 6 * d * d + C * d


def scan_bytes_per_th(d, es=2):
    return d * es


# ---- CPU baseline: the float64 oracle on a bounded sample ---------------------------
_CPU_INP = None


def _oracle_one(args):
    b, h, T = args
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(1):
        sub = {k: (v[b:b + 1, :T, h:h + 1] if isinstance(v, np.ndarray) else v)
               for k, v in _CPU_INP.items()}
        sub["B"], sub["H"], sub["T"] = 1, 1, T
        t0 = time.perf_counter()
        o, S = oracle.forward(sub)
        return b, h, o[0, :, 0].astype(np.float32), S[0, 0], time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Worker processes of the CPU leg: every core the process may run on, up to the 16
# host cores that go with one GPU on the measurement boxes.
CPU_WORKERS_MAX = 16


def cpu_baseline(inp, T_sample):
    """The oracle over every (batch, head) sequence of the workload, first T_sample
    tokens each; returns the baseline record and the per-head results (o, S)."""
    global _CPU_INP
    _CPU_INP = inp
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    workers = max(1, min(CPU_WORKERS_MAX, ncpu))
    pairs = [(b, h) for b in range(inp["B"]) for h in range(inp["H"])]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_one, [(b, h, T_sample) for b, h in pairs])
    wall = time.perf_counter() - t0
    tokens = len(pairs) * T_sample / inp["H"]     # metric tokens carry all H heads
    return dict(value=tokens / wall, unit="tokens/s", cores=workers, affinity_cores=ncpu, kind="oracle",
                cpu_model=cpu_model(),
                sample=f"all {len(pairs)} (batch, head) sequences of the workload, first {T_sample} "
                       f"of {inp['T']} tokens each (B*{T_sample} metric tokens); float64 token "
                       f"loop, {workers} worker processes, one thread each; wall {wall:.1f} s"), res


def parity_check(o_dev, s_dev, res, tol):
    """o and S_T of every sequence the oracle ran, against it: rel-L2 and normwise
    max-rel over the whole tensors and the worst single sequence."""
    import oracle
    o_host = o_dev.float().cpu().numpy()
    s_host = s_dev.float().cpu().numpy()
    T = res[0][2].shape[0]
    got_o = np.stack([o_host[b, :T, h] for b, h, _, _, _ in res])
    ref_o = np.stack([r[2] for r in res])
    got_s = np.stack([s_host[b, h] for b, h, _, _, _ in res])
    ref_s = np.stack([r[3] for r in res])
    out = dict(sequences=len(res), tokens=int(T), tolerance=dict(tol),
               o_rel_l2=oracle.rel_l2(got_o, ref_o), o_max_rel=oracle.max_rel(got_o, ref_o),
               S_rel_l2=oracle.rel_l2(got_s, ref_s), S_max_rel=oracle.max_rel(got_s, ref_s),
               worst_sequence_o_rel_l2=max(oracle.rel_l2(g, r) for g, r in zip(got_o, ref_o)),
               worst_sequence_S_rel_l2=max(oracle.rel_l2(g, r) for g, r in zip(got_s, ref_s)))
    out["pass"] = bool(max(out["o_rel_l2"], out["S_rel_l2"], out["worst_sequence_o_rel_l2"],
                           out["worst_sequence_S_rel_l2"]) <= tol["rel_l2"]
                       and max(out["o_max_rel"], out["S_max_rel"]) <= tol["max_rel"])
    return out


# Sources the two measured kernels (chunk_prep2_kernel for FG2, chunk_scan_rows_kernel)
# are built from, with the launch and argument code around them.
TRAFFIC_SOURCES = ("gdn_chunk.h", "gdn_chunk.hip", "gdn_prep_fg2.hip", "gdn_device.h", "gdn_internal.h",
                   "gdn_api.cpp", os.path.join("..", "..", "include", "gdn.h"))


def source_sha256():
    """Hash of the measured kernels' sources (the PMC traffic figures are only valid for
    the sources they were measured on)."""
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(os.path.basename(name).encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def write_traffic(pmc_dir):
    """Write profiles/chunk_traffic_fg2_32k.json from two rocprofv3 runs of
    `bench.py --profile-driver`, one with --pmc FETCH_SIZE (output under
    pmc_dir/fetch, prefix fetch) and one with --pmc WRITE_SIZE (pmc_dir/write, prefix
    write). The driver's 1 GiB device copy calibrates both counters."""
    import collections
    import csv
    import re
    # per dispatch, averaged over the steps for each instantiation; a stage's launches
    # (the prepare stage's mild and flagged passes) are summed
    vals = collections.defaultdict(list)
    for name in ("fetch", "write"):
        with open(os.path.join(pmc_dir, name, f"{name}_counter_collection.csv")) as f:
            for row in csv.DictReader(f):
                nm = row["Kernel_Name"]
                m = re.search(r"::(\w+)(<[^(]*>)?\(", nm)
                key = m.group(1) if m else ("copy" if "copyBuffer" in nm else nm[:30])
                inst = m.group(2) if m else ""
                vals[(key, inst, row["Counter_Name"])].append(float(row["Counter_Value"]))
    avg = collections.defaultdict(float)
    for (key, _, counter), v in vals.items():
        avg[(key, counter)] += sum(v) / len(v)
    cf, cw = avg[("copy", "FETCH_SIZE")], avg[("copy", "WRITE_SIZE")]
    ff, wf = 1048576.0 / cf, 1048576.0 / cw  # KiB the copy moves each way / KiB counted
    rec = {"source_sha256": source_sha256(),
           "workload": "fg2_prefill_32k_bf16 (B=2, T=32768, H=16, dk=dv=128, chunk 64)",
           "calibration": {"copy_bytes": 1 << 30, "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw,
                           "fetch_factor": ff, "write_factor": wf},
           "kernels": {}}
    for k in ("chunk_prep2_kernel", "chunk_scan_rows_kernel"):
        fk, wk = avg[(k, "FETCH_SIZE")], avg[(k, "WRITE_SIZE")]
        rb, wb = fk * 1024 * ff, wk * 1024 * wf
        rec["kernels"][k] = {"FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk, "read_bytes": rb,
                             "write_bytes": wb, "traffic_bytes_per_launch": rb + wb}
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def read_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC summary,
    if it was taken on the current kernel sources; else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
        if rec.get("source_sha256") != source_sha256():
            return None
        return rec["kernels"][kernel]["traffic_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def profile_driver(args):
    """Workload for the rocprofv3 counter runs: a few prepare + scan steps and a
    device-to-device copy of exactly 1 GiB (the calibration of FETCH_SIZE and
    WRITE_SIZE)."""
    import torch
    import gated_delta_rule_69_amd as gdn
    W = WORKLOAD
    inp = gdn_inputs.config_inputs(W["index"])
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous()
         for k in ("q", "k", "v", "alpha", "beta")}
    o = torch.empty_like(t["q"])
    s_final = torch.empty((W["B"], W["H"], W["dk"], W["dv"]), dtype=torch.float32, device=dev)
    a = gdn.make_args("fg2", t["q"], t["k"], t["v"], t["alpha"], t["beta"], chunk=W["chunk"],
                      s_final=s_final, o=o)
    ws = torch.empty(gdn.gdn_workspace_bytes(a), dtype=torch.uint8, device=dev)
    for _ in range(args.steps):
        gdn.gdn_chunk_prepare(a, ws)
        gdn.gdn_chunk_scan(a, ws)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"profile driver: {args.steps} steps and a 1 GiB copy done")


# ---- the pages' prefill timing protocol: a fixed 32,768 tokens per step, sequence
# length x batch from 2K x 16 to 32K x 1, H = 16, d = 128, FG2 and KDA inputs ------
SWEEP = [(2048, 16), (4096, 8), (8192, 4), (16384, 2), (32768, 1)]


def sweep(args):
    """Tokens/s of one gdn_chunk_fwd step (prepare + scan, final states returned) at
    each (T, B) of the sweep, for FG2, FG2+ (a value-side beta of its own) and KDA
    inputs. Each variant's inputs are drawn once as one 32,768-token sequence per head
    and cut into B sequences of T tokens. Parity: the first 1024 tokens of sequence 0,
    head 0 against the float64 oracle."""
    import torch
    import gated_delta_rule_69_amd as gdn
    import oracle
    dev = torch.device("cuda:0")
    H, d, C, total = 16, 128, 64, 32768
    rows = []
    for variant in ("fg2", "fg2_plus", "kda"):
        log(f"sweep: generating {variant} inputs (32,768 tokens x {H} heads)")
        base = "fg2" if variant == "fg2_plus" else variant
        inp = gdn_inputs.make_inputs(base, 1, total, H, d, d, dtype="bf16", seed=20,
                                     fg2_plus=variant == "fg2_plus")
        for T, B in SWEEP:
            cut = {k: (inp[k].reshape((B, T) + inp[k].shape[2:]) if isinstance(inp[k], np.ndarray) else inp[k])
                   for k in inp}
            cut["B"], cut["T"] = B, T
            tens = {k: torch.from_numpy(np.ascontiguousarray(cut[k])).to(dev).to(torch.bfloat16)
                    for k in ("q", "k", "v", "alpha", "beta", "beta_v") if k in cut}
            o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
            s_final = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
            a = gdn.make_args(base, tens["q"], tens["k"], tens["v"], tens["alpha"], tens["beta"],
                              chunk=C, beta_v=tens.get("beta_v"), s_final=s_final, o=o)
            ws = torch.empty(gdn.gdn_workspace_bytes(a), dtype=torch.uint8, device=dev)
            for _ in range(args.warmup):
                gdn.gdn_chunk_fwd_args(a, ws)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                gdn.gdn_chunk_fwd_args(a, ws)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / args.steps
            Tp = min(T, 1024)
            sub = {k: (v[0:1, :Tp, 0:1] if isinstance(v, np.ndarray) else v) for k, v in cut.items()}
            sub["B"], sub["H"], sub["T"] = 1, 1, Tp
            o_ref, _ = oracle.forward(sub)
            got = o[0, :Tp, 0].float().cpu().numpy()
            err = float(np.linalg.norm(got - o_ref[0, :, 0]) / np.linalg.norm(o_ref[0, :, 0]))
            rows.append(dict(variant=variant, T=T, B=B, ms=ms, tokens_per_s=B * T / (ms * 1e-3),
                             o_rel_l2_sample=err))
            log(f"sweep: {variant} T={T} B={B}: {ms:.3f} ms, {B * T / (ms * 1e-3):.3e} tokens/s, "
                f"parity rel-L2 {err:.2e}")
            del tens, o, s_final, ws, a
            torch.cuda.empty_cache()
    tok = {(r["variant"], r["T"]): r["tokens_per_s"] for r in rows}
    out = {
        "metric": "prefill tokens/s at a fixed 32,768 tokens per step (H=16, d=128, chunk 64, bf16)",
        "unit": "tokens/s",
        "rows": rows,
        "long_over_short": {v: tok[(v, 32768)] / tok[(v, 2048)] for v in ("fg2", "fg2_plus", "kda")},
        "fg2_over_kda_time": {str(T): tok[("kda", T)] / tok[("fg2", T)] for T, _ in SWEEP},
        "fg2_plus_over_kda_time": {str(T): tok[("kda", T)] / tok[("fg2_plus", T)] for T, _ in SWEEP},
        "data": "synthetic",
        "n_gpus": 1,
    }
    print(json.dumps(out), flush=True)


def copy_bandwidth_gbs():
    """Measured device-to-device copy bandwidth (1 GiB, read + write counted), GB/s:
    what a plain streaming kernel reaches on this GPU, beside the 8 TB/s spec."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(5):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 5
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


# ---- the other workloads: time per gdn_chunk_fwd call and both roofline fractions --
def alg_per_th(cfg):
    """Algorithmic bytes and flops per token-head of a workload (inputs + output,
    never the workspace; the chunkwise method's triangular work)."""
    es = 2 if cfg["dtype"] == "bf16" else 4
    d, C, n_h, var = cfg["dk"], cfg["chunk"], cfg["n_h"], cfg["variant"]
    if var == "deltaproduct":
        nbytes = (d + n_h * 2 * d + n_h + 1 + d) * es          # q, k_j, v_j, beta_j, gate, o
        flops = n_h * (4 * d * d + 3 * C * d) + 2 * d * d + 2 * C * d
    else:
        per_row = {"fg2": 5 * d, "kda": 4 * d + 1, "gdn": 3 * d + 2, "asym": 5 * d + 1}[var]
        nbytes = (per_row + d) * es
        flops = 6 * d * d + 5 * C * d
    return nbytes, flops


def configs(args):
    """Workloads 0, 1, 3 and 4 (the parity configurations): median time of one
    gdn_chunk_fwd call over 20 calls (HIP events around each, 5 warm-ups, a 512 MB
    buffer written between calls so that no input stays in the 256 MB Infinity
    Cache), both roofline fractions, and o / S_T of sequence 0, head 0 against the
    float64 oracle."""
    import torch
    import gated_delta_rule_69_amd as gdn
    import oracle
    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    rows = []
    for idx in (0, 1, 3, 4):
        cfg = gdn_inputs.CONFIGS[idx]
        inp = gdn_inputs.config_inputs(idx)
        io = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
        names = [n for n in ("q", "k", "v", "alpha", "beta", "j", "eta") if n in inp]
        t = {n: torch.from_numpy(inp[n]).to(dev).to(io).contiguous() for n in names}
        B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
        o = torch.empty((B, T, H, dv), dtype=io, device=dev)
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        a = gdn.make_args(cfg["variant"], t["q"], t["k"], t["v"], t["alpha"], t.get("beta"),
                          chunk=cfg["chunk"], j=t.get("j"), eta=t.get("eta"), s_final=s_final, o=o)
        ws = torch.empty(gdn.gdn_workspace_bytes(a), dtype=torch.uint8, device=dev)
        for _ in range(5):
            gdn.gdn_chunk_fwd_args(a, ws)
        times = []
        for _ in range(20):
            flush.fill_(1)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            gdn.gdn_chunk_fwd_args(a, ws)
            ev[1].record()
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]) * 1e3)
        us = float(np.median(times))
        sub = {k: (v[0:1, :, 0:1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        sub["B"], sub["H"] = 1, 1
        o_ref, s_ref = oracle.forward(sub)
        o_err = float(np.linalg.norm(o[0, :, 0].float().cpu().numpy() - o_ref[0, :, 0]) /
                      np.linalg.norm(o_ref[0, :, 0]))
        s_err = float(np.linalg.norm(s_final[0, 0].cpu().numpy() - s_ref[0, 0]) / np.linalg.norm(s_ref[0, 0]))
        nb, nf = alg_per_th(cfg)
        units = B * T * H
        nbytes = nb * units + B * H * dk * dv * 4
        peak_tf = MFMA_PEAK_TFLOPS if cfg["dtype"] == "bf16" else MFMA_F32_PEAK_TFLOPS
        gbs = nbytes / (us * 1e-6) / 1e9
        tfs = nf * units / (us * 1e-6) / 1e12
        rows.append(dict(workload=cfg["name"], index=idx, variant=cfg["variant"], dtype=cfg["dtype"],
                         B=B, T=T, H=H, dk=dk, dv=dv, chunk=cfg["chunk"], n_h=cfg["n_h"], us=us,
                         tokens_per_s=B * T / (us * 1e-6),
                         hbm=dict(achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                                  algorithmic=nbytes),
                         mfma=dict(achieved=tfs, peak=peak_tf, unit="TFLOP/s", frac=tfs / peak_tf,
                                   algorithmic=nf * units),
                         parity=dict(o_rel_l2=o_err, S_rel_l2=s_err)))
        log(f"configs: {cfg['name']}: {us:.1f} us, HBM {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%}), "
            f"MFMA {tfs:.1f} TFLOP/s ({tfs / peak_tf:.1%}), parity o {o_err:.2e} S {s_err:.2e}")
        del t, o, s_final, ws, a
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "time per gdn_chunk_fwd call and roofline fractions, workloads 0, 1, 3, 4",
                      "rows": rows, "data": "synthetic", "n_gpus": 1}), flush=True)


# ---- decode: one token per sequence through gdn_recurrent_step --------------------
def decode(args):
    """Time of one gdn_recurrent_step call with T = 1 over B = 512 sequences, H = 16,
    dk = dv = 128 (FG2, bf16 inputs, fp32 state resident in HBM: 512 MB, twice the
    Infinity Cache). The step reads and writes the whole state once: its roofline is
    HBM traffic of 2 * 4 * dk * dv bytes per (sequence, head) plus the token's inputs.
    Parity: sequence 0, head 0 (output and updated state) against the float64 oracle."""
    import torch
    import gated_delta_rule_69_amd as gdn
    import oracle
    dev = torch.device("cuda:0")
    B, H, d = 512, 16, 128
    inp = gdn_inputs.make_inputs("fg2", B, 1, H, d, d, dtype="bf16", seed=30)
    s0 = gdn_inputs.make_state(B, H, d, d, seed=30)
    tens = {k: torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous()
            for k in ("q", "k", "v", "alpha", "beta")}
    state = torch.from_numpy(s0).to(dev)
    o = torch.empty((B, 1, H, d), dtype=torch.bfloat16, device=dev)
    # parity on a fresh copy of the state (the timed calls update it in place)
    gdn.gdn_recurrent_step("fg2", tens["q"], tens["k"], tens["v"], tens["alpha"], tens["beta"],
                           state=state, o=o)
    torch.cuda.synchronize()
    sub = {k: (v[0:1, :, 0:1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    sub["B"], sub["H"] = 1, 1
    o_ref, s_ref = oracle.forward(sub, s0[0:1, 0:1])
    o_err = float(np.linalg.norm(o[0, 0, 0].float().cpu().numpy() - o_ref[0, 0, 0]) /
                  np.linalg.norm(o_ref[0, 0, 0]))
    s_err = float(np.linalg.norm(state[0, 0].cpu().numpy() - s_ref[0, 0]) / np.linalg.norm(s_ref[0, 0]))
    for _ in range(args.warmup):
        gdn.gdn_recurrent_step("fg2", tens["q"], tens["k"], tens["v"], tens["alpha"], tens["beta"],
                               state=state, o=o)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(args.steps):
        gdn.gdn_recurrent_step("fg2", tens["q"], tens["k"], tens["v"], tens["alpha"], tens["beta"],
                               state=state, o=o)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps
    state_bytes = 2 * 4 * d * d * B * H
    io_bytes = B * H * (5 * d + d) * 2
    gbs = (state_bytes + io_bytes) / (us * 1e-6) / 1e9
    copy_gbs = copy_bandwidth_gbs()
    log(f"decode: {us:.1f} us per step, {gbs:.0f} GB/s (device copy {copy_gbs:.0f} GB/s), "
        f"parity o {o_err:.2e} S {s_err:.2e}")
    print(json.dumps({
        "metric": "decode step: gdn_recurrent_step, one token for 512 sequences (H=16, d=128)",
        "us_per_step": us, "tokens_per_s": B / (us * 1e-6),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic": state_bytes + io_bytes,
                     "device_copy_gbs": copy_gbs},
        "parity": {"o_rel_l2": o_err, "S_rel_l2": s_err},
        "data": "synthetic", "n_gpus": 1}), flush=True)


# ---- GDN2 stabilisers: gdn_asym_stabilize on the asymmetric workload ---------------
def stabilize(args):
    """Both stabiliser modes on workload 4 (ASYM, fp32, B=8, H=32, T=2048, dk=64):
    median time of one gdn_asym_stabilize call over 20 calls (512 MB written between
    calls so that nothing stays in the Infinity Cache), HBM fraction with
    (4 dk + 1) elements per token-head (k, j, D and eta in, dk out), the cost beside
    one gdn_chunk_fwd call of the same workload, the time of gdn_chunk_fwd with the
    stabiliser inside the pass, and the first 4096 token-heads against the float64
    oracle."""
    import torch
    import gated_delta_rule_69_amd as gdn
    import oracle
    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cfg = gdn_inputs.CONFIGS[4]
    inp = gdn_inputs.config_inputs(4)
    t = {n: torch.from_numpy(inp[n]).to(dev).contiguous() for n in ("q", "k", "v", "alpha", "j", "eta")}
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    out = torch.empty_like(t["k"])

    def timed(fn):
        for _ in range(5):
            fn()
        times = []
        for _ in range(20):
            flush.fill_(1)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]) * 1e3)
        return float(np.median(times))

    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    a = gdn.make_args("asym", t["q"], t["k"], t["v"], t["alpha"], None, chunk=cfg["chunk"],
                      j=t["j"], eta=t["eta"], s_final=s_final, o=o)
    ws = torch.empty(gdn.gdn_workspace_bytes(a), dtype=torch.uint8, device=dev)
    fwd_us = timed(lambda: gdn.gdn_chunk_fwd_args(a, ws))
    units = B * T * H
    nbytes = (4 * dk + 1) * 4 * units
    n = 4096
    sub = {x: inp[x].reshape(units, -1)[:n].astype(np.float64) for x in ("k", "j", "alpha")}
    eta = inp["eta"].reshape(units)[:n].astype(np.float64)
    rows = []
    for mode in ("clip_decay", "project_j"):
        fa = gdn.make_args("asym", t["q"], t["k"], t["v"], t["alpha"], None, chunk=cfg["chunk"],
                           j=t["j"], eta=t["eta"], s_final=s_final, o=o, stabilize=mode)
        fused_us = timed(lambda: gdn.gdn_chunk_fwd_args(fa, ws))
        us = timed(lambda: gdn.gdn_asym_stabilize(mode, t["k"], t["j"], t["alpha"], t["eta"], out=out))
        fn = oracle.stabilize.clip_decay if mode == "clip_decay" else oracle.stabilize.project_j
        ref = fn(sub["k"], sub["j"], eta, sub["alpha"])
        got = out.reshape(units, dk)[:n].cpu().numpy().astype(np.float64)
        err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        gbs = nbytes / (us * 1e-6) / 1e9
        rows.append(dict(mode=mode, us=us, vs_chunk_fwd=us / fwd_us, fused_chunk_fwd_us=fused_us,
                         hbm=dict(achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                                  frac=gbs / HBM_PEAK_GBS, algorithmic=nbytes),
                         parity=dict(rel_l2=err, rows=n)))
        log(f"stabilize {mode}: {us:.1f} us, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%}), "
            f"{us / fwd_us:.1%} of gdn_chunk_fwd ({fwd_us:.1f} us), parity {err:.2e}; "
            f"inside gdn_chunk_fwd: {fused_us:.1f} us")
    print(json.dumps({"metric": "time per gdn_asym_stabilize call, workload 4 (B=8, H=32, T=2048, dk=64, fp32)",
                      "rows": rows, "chunk_fwd_us": fwd_us, "device_copy_gbs": copy_bandwidth_gbs(),
                      "data": "synthetic", "n_gpus": 1}), flush=True)


# ---- backward: gdn_recurrent_bwd on the 4K prefill workload --------------------------
def bwd_flops_per_step(dk, dv, C=16):
    """Algorithmic flops of the chunkwise backward pass per step (token, or DeltaProduct
    sub-step) and head: the state and state-gradient recursions (W S, A^^T U; A^ D,
    W^T X, (Q+ - P W)^T dO) and the intra-chunk products U, A^ D, dO S^T, dR S^T, U D^T,
    10 dk dv multiply-adds, plus the C x C x d ones of the chunk (Grams, W, U~, Q+ - P W,
    P^T dO, dR, dP, dM and the four per key tile), about 11 C d."""
    return 2 * (10 * dk * dv + 11 * C * max(dk, dv))


def backward_one(index, steps):
    """One gdn_recurrent_bwd workload: time per call (HIP events over `steps` calls
    after 3 warm-ups), HBM fraction of the algorithmic bytes (inputs, d_o and float32
    gradients) and fp32 MFMA fraction of the algorithmic flops, and every gradient of
    sequence 0, head 0 against the float64 oracle (rel-L2)."""
    import torch
    import gated_delta_rule_69_amd as gdn
    import oracle
    dev = torch.device("cuda:0")
    cfg = gdn_inputs.CONFIGS[index]
    var, B, T, H, dk, dv, nh = (cfg[k] for k in ("variant", "B", "T", "H", "dk", "dv", "n_h"))
    io = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    es = 2 if cfg["dtype"] == "bf16" else 4
    inp = gdn_inputs.config_inputs(index)
    t = {n: torch.from_numpy(inp[n]).to(dev).to(io).contiguous()
         for n in ("q", "k", "v", "alpha", "beta", "beta_v", "j", "eta") if inp.get(n) is not None}
    rng = np.random.default_rng(7)
    do_np = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    if cfg["dtype"] == "bf16":
        do_np = gdn_inputs.round_bf16(do_np)
    do = torch.from_numpy(do_np).to(dev).to(io)
    run = lambda: gdn.gdn_recurrent_bwd(var, t["q"], t["k"], t["v"], t["alpha"], t.get("beta"), d_o=do,  # noqa: E731
                                        beta_v=t.get("beta_v"), j=t.get("j"), eta=t.get("eta"))
    got = run()
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        run()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    sub = {k: (v[0:1, :, 0:1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    sub["B"], sub["H"] = 1, 1
    ref = oracle.backward.backward(sub, do_np[0:1, :, 0:1])
    errs = {n: float(np.linalg.norm(got[n][0:1, :, 0:1].cpu().numpy() - r) / np.linalg.norm(r))
            for n, r in ref.items() if n != "ds0"}
    steps_th = B * T * H * nh
    in_bytes = sum(x.numel() * es for x in t.values()) + do.numel() * es
    out_bytes = sum(x.numel() * 4 for n, x in got.items() if n != "ds0" and x is not None)
    nbytes = in_bytes + out_bytes
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = bwd_flops_per_step(dk, dv) * steps_th
    tfs = flops / (ms * 1e-3) / 1e12
    return dict(workload=cfg["name"], ms=ms, tokens_per_s=B * T / (ms * 1e-3),
                roofline={"bound": "mfma", "achieved": tfs, "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": tfs / MFMA_F32_PEAK_TFLOPS, "algorithmic": flops},
                hbm={"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "algorithmic": nbytes},
                parity=errs)


def backward(args):
    """gdn_recurrent_bwd on workload 1 (FG2, bf16, B=1, H=16, T=4096, d=128), or with
    --all on workloads 1, 3 and 4: one JSON line each (see backward_one)."""
    for index in ((1, 3, 4) if args.all else (1,)):
        r = backward_one(index, args.steps)
        log(f"backward {r['workload']}: {r['ms']:.3f} ms per call ({r['tokens_per_s']:.3e} tokens/s), "
            f"{r['roofline']['achieved']:.1f} TFLOP/s fp32 ({r['roofline']['frac']:.1%}), "
            f"{r['hbm']['achieved']:.0f} GB/s ({r['hbm']['frac']:.1%}), parity max rel-L2 {max(r['parity'].values()):.2e}")
        print(json.dumps({"metric": f"gdn_recurrent_bwd time, {r['workload']}", **r,
                          "data": "synthetic", "n_gpus": 1}), flush=True)


def fg2_plus(args):
    """FG2-GDN+ (a value-side beta of its own) on the headline workload's shape (B=2,
    T=32768, H=16, d=128, chunk 64, bf16): prepare and scan times (HIP events around
    each stage, mean over --steps steps after --warmup), the prepare stage's HBM
    fraction on its 6 d bf16 input bytes per token-head, and o / S_T of sequence 0,
    head 0 against the float64 oracle."""
    import torch
    import gated_delta_rule_69_amd as gdn
    import oracle
    dev = torch.device("cuda:0")
    W = gdn_inputs.CONFIGS[2]
    B, T, H, d, C = W["B"], W["T"], W["H"], W["dk"], W["chunk"]
    log("fg2+: generating inputs")
    inp = gdn_inputs.make_inputs("fg2", B, T, H, d, d, dtype="bf16", seed=2, fg2_plus=True)
    t = {n: torch.from_numpy(inp[n]).to(dev).to(torch.bfloat16).contiguous()
         for n in ("q", "k", "v", "alpha", "beta", "beta_v")}
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    s_final = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    a = gdn.make_args("fg2", t["q"], t["k"], t["v"], t["alpha"], t["beta"], chunk=C, beta_v=t["beta_v"],
                      s_final=s_final, o=o)
    ws = torch.empty(gdn.gdn_workspace_bytes(a), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        gdn.gdn_chunk_prepare(a, ws)
        gdn.gdn_chunk_scan(a, ws)
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        gdn.gdn_chunk_prepare(a, ws)
        e[1].record()
        gdn.gdn_chunk_scan(a, ws)
        e[2].record()
        evs.append(e)
    torch.cuda.synchronize()
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    nbytes = B * T * H * 6 * d * 2  # q, k, v, alpha, beta, beta_v
    gbs = nbytes / (prep_ms * 1e-3) / 1e9
    sub = {k: (v[0:1, :, 0:1] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    sub["B"], sub["H"] = 1, 1
    o_ref, s_ref = oracle.forward(sub)
    o_err = oracle.rel_l2(o[0, :, 0].float().cpu().numpy(), o_ref[0, :, 0])
    s_err = oracle.rel_l2(s_final[0, 0].cpu().numpy(), s_ref[0, 0])
    log(f"fg2+: prepare {prep_ms:.3f} ms ({gbs:.0f} GB/s, {gbs / HBM_PEAK_GBS:.1%}), scan {scan_ms:.3f} ms, "
        f"parity o {o_err:.2e} S {s_err:.2e}")
    print(json.dumps({"metric": "FG2-GDN+ chunked prefill at 32K (B=2, H=16, d=128): stage times",
                      "prepare_ms": prep_ms, "scan_ms": scan_ms, "ms_per_step": prep_ms + scan_ms,
                      "tokens_per_s": B * T / ((prep_ms + scan_ms) * 1e-3),
                      "prepare_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": gbs / HBM_PEAK_GBS, "algorithmic": nbytes},
                      "parity": {"o_rel_l2": o_err, "S_rel_l2": s_err}, "data": "synthetic", "n_gpus": 1}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens per sequence for the oracle leg (default: all)")
    ap.add_argument("--write-traffic", metavar="PMC_DIR",
                    help="write the traffic summary from FETCH_SIZE / WRITE_SIZE runs under PMC_DIR")
    ap.add_argument("--profile-driver", action="store_true",
                    help="only run the workload for rocprofv3 counter collection")
    ap.add_argument("--configs", action="store_true",
                    help="workloads 0, 1, 3, 4: time per call, roofline fractions, parity")
    ap.add_argument("--decode", action="store_true",
                    help="one-token decode step (gdn_recurrent_step) over 512 sequences")
    ap.add_argument("--backward", action="store_true",
                    help="backward pass (gdn_recurrent_bwd) on the 4K prefill workload")
    ap.add_argument("--all", action="store_true",
                    help="with --backward: workloads 1, 3 and 4")
    ap.add_argument("--stabilize", action="store_true",
                    help="GDN2 stabilisers (gdn_asym_stabilize) on the asymmetric workload")
    ap.add_argument("--fg2-plus", action="store_true",
                    help="FG2-GDN+ (value-side beta) stage times on the 32K workload's shape")
    ap.add_argument("--sweep", action="store_true",
                    help="the prefill sweep at a fixed 32,768 tokens (2K x 16 .. 32K x 1), FG2 and KDA")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.profile_driver:
        profile_driver(args)
        return
    if args.sweep:
        sweep(args)
        return
    if args.decode:
        decode(args)
        return
    if args.stabilize:
        stabilize(args)
        return
    if args.fg2_plus:
        fg2_plus(args)
        return
    if args.backward:
        backward(args)
        return
    if args.configs:
        configs(args)
        return

    W = WORKLOAD
    B, H, T, d, C = W["B"], W["H"], W["T"], W["dk"], W["chunk"]
    log(f"bench: generating inputs {W['name']} (seed {W['index']})")
    inp = gdn_inputs.config_inputs(W["index"])

    cpu = None
    cpu_res = []
    if not args.no_cpu_baseline:
        log("bench: oracle CPU baseline")
        cpu, cpu_res = cpu_baseline(inp, min(args.cpu_tokens, T) if args.cpu_tokens > 0 else T)
        log(f"bench: cpu {cpu['value']:.1f} tokens/s on {cpu['cores']} cores")

    import torch
    import gated_delta_rule_69_amd as gdn
    dev = torch.device("cuda:0")
    tens = {k: torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous()
            for k in ("q", "k", "v", "alpha", "beta")}
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    s_final = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    a = gdn.make_args("fg2", tens["q"], tens["k"], tens["v"], tens["alpha"], tens["beta"],
                      chunk=C, s_final=s_final, o=o)
    ws = torch.empty(gdn.gdn_workspace_bytes(a), dtype=torch.uint8, device=dev)
    log(f"bench: workspace {ws.numel() / 2**30:.2f} GiB")

    def step(evs=None):
        if evs:
            evs[0].record()
        gdn.gdn_chunk_prepare(a, ws)
        if evs:
            evs[1].record()
        gdn.gdn_chunk_scan(a, ws)
        if evs:
            evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    log(f"bench: {ms_step:.3f} ms/step (prepare {prep_ms:.3f} ms, scan {scan_ms:.3f} ms)")

    units = B * T * H                                   # token-heads per launch
    # per-kernel rooflines (algorithmic work per launch / mean launch time from the
    # HIP events above); `roofline` reports the longer of the two kernels
    prep_bytes = prep_bytes_per_th(d) * units
    prep_gbs = prep_bytes / (prep_ms * 1e-3) / 1e9
    prep_roof = dict(kernel="chunk_prep2_kernel", bound="hbm", achieved=prep_gbs, peak=HBM_PEAK_GBS,
                     unit="GB/s", frac=prep_gbs / HBM_PEAK_GBS, algorithmic=prep_bytes,
                     ms=prep_ms, traffic=read_traffic("chunk_prep2_kernel"))
    scan_flops = scan_flops_per_th(d, C) * units
    scan_tf = scan_flops / (scan_ms * 1e-3) / 1e12
    scan_roof = dict(kernel="chunk_scan_rows_kernel", bound="mfma", achieved=scan_tf,
                     peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s", frac=scan_tf / MFMA_PEAK_TFLOPS,
                     algorithmic=scan_flops, ms=scan_ms, traffic=read_traffic("chunk_scan_rows_kernel"))
    roof = dict(prep_roof if prep_ms >= scan_ms else scan_roof)
    roof["other_kernel"] = scan_roof if prep_ms >= scan_ms else prep_roof
    path_bytes = (prep_bytes_per_th(d) + scan_bytes_per_th(d)) * units + B * H * d * d * 4
    path_gbs = path_bytes / (ms_step * 1e-3) / 1e9
    path = dict(bound="hbm", achieved=path_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=path_gbs / HBM_PEAK_GBS, algorithmic=path_bytes,
                prepare_ms=prep_ms, scan_ms=scan_ms, device_copy_gbs=copy_bandwidth_gbs())

    parity = None
    if cpu_res:
        parity = parity_check(o, s_final, cpu_res, dict(rel_l2=5e-3, max_rel=2e-2))
        log(f"bench: parity vs oracle over {parity['sequences']} sequences x {parity['tokens']} tokens: "
            f"o {parity['o_rel_l2']:.2e} / {parity['o_max_rel']:.2e}, S {parity['S_rel_l2']:.2e} / "
            f"{parity['S_max_rel']:.2e} -> {'pass' if parity['pass'] else 'FAIL'}")

    out = {
        "metric": METRIC,
        "value": B * T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W["name"], "variant": "fg2", "B": B, "T": T, "H": H, "dk": d,
                   "dv": d, "chunk": C, "io_dtype": "bf16", "state_dtype": "f32",
                   "mfma": "fp16 (Gram: bf16 hi/lo split), fp32 accumulate"},
        "roofline": roof,
        "path_roofline": path,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    if parity is not None and not parity["pass"]:
        log("bench: the results are outside the parity tolerance")
        sys.exit(1)


if __name__ == "__main__":
    main()
