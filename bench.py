#!/usr/bin/env python3
"""Benchmark of the MSA training hot path on one MI355X (gfx950).

One step is the whole hot path over one batch of synthetic input:
msa_proxy_select (Index Branch: proxy score, block max-pool, top-k into the
block-index cache) -> msa_fwd -> msa_bwd (Main Branch over the cached blocks).
Inputs are resident in HBM before the timed region.  W warm-up steps, then K
timed steps between two device synchronisations.

Printed: one JSON line.  `value` is tokens/s of the whole step on the main
workload (the 128K configuration: B=1, T=131072, 32 query / 4 KV heads, head
dim 128, 4 proxy heads of dim 64, top-k 32).  Extra fields give the fwd+bwd
rate with cached indices, effective TFLOP/s on the executed sparse FLOPs,
per-phase and per-kernel times (HIP events recorded by the library on the
launch stream), the roofline of the dominant kernel, extra workloads (the 1M
configuration; the 128K step on a fixed window/dilation pattern united with
the proxy top-k; the 128K step through the merged forward/backward call;
decode steps of 16 sequences at 128K cached tokens), and the
CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--also 1m,pattern,merged,decode|''] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
import block_sparse_attention_qk_amd as msa  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "MSA fwd+bwd tokens/s and effective TFLOP/s (% bf16 MFMA peak), 128K & 1M"

# Library timing slot -> kernel symbol prefix and the source file it is built from.
KERNELS = {  # bench name -> (kernel symbol in rocprofv3 output, source files it is compiled from)
    "proxy_pool": ("msa::k_proxy_pool<", ("msa_select.hip",)),
    "topk": ("msa::k_topk<", ("msa_select.hip", "msa_topk.h")),
    "inverse": ("msa::k_inv_scatter", ("msa_inverse.hip",)),
    "fwd_partials": ("msa::k_fwd_kv<", ("msa_fwd.hip",)),
    "fwd_combine": ("msa::k_fwd_combine<", ("msa_fwd.hip",)),
    "bwd_dot": ("msa::k_bwd_dot<", ("msa_bwd.hip",)),
    "bwd_partials": ("msa::k_bwd_kv<", ("msa_bwd.hip",)),
    "dq_combine": ("msa::k_dq_combine<", ("msa_bwd.hip",)),
    "convert": ("msa::k_cvt_bf16", ("msa_bwd.hip",)),
    "dec_pool": ("msa::k_dec_pool<", ("msa_decode.hip",)),
    "dec_topk": ("msa::k_dec_topk<", ("msa_decode.hip", "msa_topk.h")),
    "dec_attn": ("msa::k_dec_attn<", ("msa_decode.hip",)),
    "dec_combine": ("msa::k_dec_combine<", ("msa_decode.hip",)),
}
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "msa_hbm_traffic_*.md")


def kernel_source_hash(name: str) -> str:
    """Hash of what a kernel is compiled from (its sources, the shared headers and
    the build flags): stored HBM counter figures apply only while it matches."""
    import hashlib
    csrc = os.path.join(ROOT, "block_sparse_attention_qk_amd", "csrc")
    h = hashlib.sha256()
    paths = [os.path.join(csrc, f) for f in KERNELS[name][1]]
    paths += [os.path.join(csrc, "msa_common.h"), os.path.join(csrc, "msa_internal.h"),
              os.path.join(ROOT, "block_sparse_attention_qk_amd", "build.py")]
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, name: str):
    """Calibrated HBM bytes per launch (read + write) of one kernel, from the
    committed counter summaries, or None if absent or taken on other code."""
    import glob
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        for line in open(path):
            f = dict(kv.split("=", 1) for kv in line.split()[1:] if "=" in kv) if line.startswith("traffic ") else {}
            if f.get("workload") == workload and f.get("kernel") == name:
                if f.get("source") != kernel_source_hash(name):
                    return None
                return int(f["read_bytes"]) + int(f["write_bytes"])
    return None


def pmc_summary(pmc_dir: str, copy_mib: int, workload: str) -> str:
    """Per-kernel HBM bytes per dispatch from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain device copy of copy_mib MiB in the same run."""
    import csv
    import glob
    vals = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        per = {}
        for f in glob.glob(os.path.join(pmc_dir, ctr, "*_counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == ctr:
                    per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        vals[ctr] = per
    copy_bytes = float(copy_mib << 20)
    factor = {}
    for ctr in vals:
        cands = [max(v) for k, v in vals[ctr].items() if "copyBuffer" in k]
        if not cands:
            raise SystemExit("no copy kernel in the %s run" % ctr)
        factor[ctr] = copy_bytes / max(cands)
    out = ["Copy calibration (%d MiB device copy): FETCH_SIZE x %.3f, WRITE_SIZE x %.3f" % (
        copy_mib, factor["FETCH_SIZE"], factor["WRITE_SIZE"]), "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GiB | write GiB |", "|---|---|---|---|---|---|"]
    lines = []
    for name, (sym, _) in KERNELS.items():
        rd = [v for k, v in vals["FETCH_SIZE"].items() if sym in k]
        wr = [v for k, v in vals["WRITE_SIZE"].items() if sym in k]
        if not rd or not wr:
            continue
        rd = [x for v in rd for x in v]
        wr = [x for v in wr for x in v]
        r_avg, w_avg = sum(rd) / len(rd), sum(wr) / len(wr)
        rb, wb = r_avg * factor["FETCH_SIZE"], w_avg * factor["WRITE_SIZE"]
        out.append("| %s (%s) | %d | %.0f | %.0f | %.3f | %.3f |" % (
            name, sym.split("::")[-1].rstrip("<"), len(rd), r_avg / 1024, w_avg / 1024, rb / 2**30, wb / 2**30))
        lines.append("traffic workload=%s kernel=%s read_bytes=%d write_bytes=%d source=%s" % (
            workload, name, rb, wb, kernel_source_hash(name)))
    return "\n".join(out + ["", "```"] + lines + ["```"])



def gpu_inputs(cfg: synth.Config, seed: int = 0) -> dict:
    """Same recipe as synth (N(0,1) bf16; proxy keys plus a per-block mean of
    variance 0.5) drawn directly on the GPU, for workloads too large to draw
    on the host in reasonable time.  Values differ from synth's CPU draws."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    out = {}
    shapes = {"q": (cfg.B, cfg.T, cfg.H, cfg.d), "dout": (cfg.B, cfg.T, cfg.H, cfg.d),
              "k": (cfg.B, cfg.T, cfg.G, cfg.d), "v": (cfg.B, cfg.T, cfg.G, cfg.d),
              "qp": (cfg.B, cfg.T, cfg.G, cfg.dp), "kp": (cfg.B, cfg.T, cfg.G, cfg.dp)}
    for i, (name, shp) in enumerate(shapes.items()):
        g.manual_seed(0x5EED + 7919 * (i + 1) + seed)
        t = torch.empty(shp, dtype=torch.bfloat16, device=dev)
        flat = t.view(-1)
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            n = min(step, flat.numel() - s)
            flat[s:s + n] = torch.randn(n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        out[name] = t
    g.manual_seed(0x5EED + 7919 * 7 + seed)
    mu = torch.randn((cfg.B, cfg.N, cfg.G, cfg.dp), generator=g, device=dev) * math.sqrt(0.5)
    kp = out["kp"].float().view(cfg.B, cfg.N, synth.BLOCK, cfg.G, cfg.dp) + mu[:, :, None]
    out["kp"] = kp.view(cfg.B, cfg.T, cfg.G, cfg.dp).to(torch.bfloat16).contiguous()
    del kp, mu
    return out


def gpu_decode_inputs(cfg: synth.Config, B: int, seed: int = 0) -> dict:
    """Decode-step inputs drawn on the GPU with the synth recipe: caches kp
    [B,T,G,dp] (plus the per-block proxy-key mean), k, v [B,T,G,d], and the new
    tokens' qp [B,G,dp] and q [B,H,d]."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    shapes = {"k": (B, cfg.T, cfg.G, cfg.d), "v": (B, cfg.T, cfg.G, cfg.d), "kp": (B, cfg.T, cfg.G, cfg.dp),
              "qp": (B, cfg.G, cfg.dp), "q": (B, cfg.H, cfg.d)}
    out = {}
    for i, (name, shp) in enumerate(shapes.items()):
        g.manual_seed(0x5EED + 104729 * (i + 1) + seed)
        t = torch.empty(shp, dtype=torch.bfloat16, device=dev)
        flat = t.view(-1)
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            n = min(step, flat.numel() - s)
            flat[s:s + n] = torch.randn(n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        out[name] = t
    g.manual_seed(0x5EED + 104729 * 6 + seed)
    mu = torch.randn((B, cfg.N, cfg.G, cfg.dp), generator=g, device=dev) * math.sqrt(0.5)
    for b in range(B):
        kb = out["kp"][b].float().view(cfg.N, synth.BLOCK, cfg.G, cfg.dp) + mu[b][:, None]
        out["kp"][b] = kb.view(cfg.T, cfg.G, cfg.dp).to(torch.bfloat16)
    del mu
    return out


PATTERN = (8, 64)  # window blocks, dilation: the fixed-pattern leg (united with the proxy top-k)


def run_workload(cfg: synth.Config, steps: int, warmup: int, host_inputs: bool, pattern=None,
                 merged: bool = False) -> dict:
    """One step = proxy select (+ the fixed window/dilation pattern united with
    it, when `pattern` is given) + forward + backward over the cache (one
    msa_fwd_bwd call when `merged`)."""
    if host_inputs:
        x = {n: t.cuda() for n, t in synth.make_inputs(cfg).items()}
    else:
        x = gpu_inputs(cfg)
    width = msa.pattern_width(cfg.T, pattern[0], pattern[1], cfg.topk) if pattern else cfg.topk
    dims = (cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, width)
    ops = (msa.OP_SELECT, msa.OP_FWD_BWD) if merged else (msa.OP_SELECT, msa.OP_FWD, msa.OP_BWD)
    ws_bytes = max(msa.msa_workspace_bytes(*dims, op) for op in ops)
    ws = msa.Workspace(nbytes=ws_bytes)
    idx = torch.empty((cfg.B, cfg.G, cfg.T, cfg.topk), dtype=torch.int32, device="cuda")
    idx_main = torch.empty((cfg.B, cfg.G, cfg.T, width), dtype=torch.int32, device="cuda") if pattern else idx
    o = torch.empty_like(x["q"])
    lse = torch.empty((cfg.B, cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    def step(ev=None):
        if ev:
            ev[0].record()
        msa.msa_proxy_select(x["qp"], x["kp"], cfg.topk, ws=ws, out=idx)
        if pattern:
            msa.msa_pattern_select(cfg.B, cfg.T, cfg.G, pattern[0], pattern[1], idx_in=idx, width=width,
                                   out=idx_main)
        if ev:
            ev[1].record()
        if merged:
            msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx_main, ws=ws, out=(o, lse, dq, dk, dv))
            if ev:
                ev[2].record()
        else:
            msa.msa_fwd(x["q"], x["k"], x["v"], idx_main, ws=ws, out=(o, lse))
            if ev:
                ev[2].record()
            msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx_main, ws=ws, out=(dq, dk, dv))
        if ev:
            ev[3].record()

    for _ in range(warmup):
        step()
    # pairs actually read by the Main Branch (the pattern's rows vary in length)
    pairs = int((idx_main >= 0).sum().item()) if pattern else cfg.pairs()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    msa.timing_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(steps):
        step(evs[s])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    phase = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) for i in range(3)]
    kern = msa.timing_read()
    msa.timing_enable(False)

    tokens = cfg.B * cfg.T
    ms_step = total_ms / steps
    t_sel, t_fwd, t_bwd = (p / steps for p in phase)
    f_pair = 4 * cfg.d * cfg.R * 128  # forward flop per (token, group, block); backward is 2.5x
    f_fwd, f_bwd, f_proxy = f_pair * pairs, 2.5 * f_pair * pairs, cfg.flops_proxy()
    res = {
        "workload": cfg.name + ("+pattern(window=%d,dilation=%d)" % pattern if pattern else "") +
                    (" merged fwd+bwd (msa_fwd_bwd)" if merged else ""),
        "shape": {"B": cfg.B, "T": cfg.T, "H": cfg.H, "G": cfg.G, "d": cfg.d, "dp": cfg.dp, "topk": cfg.topk,
                  "cache_width": width},
        "ms_per_step": ms_step,
        "wall_ms_per_step": 1e3 * wall / steps,
        "tokens_per_s": tokens / (ms_step / 1e3),
        "phases_ms": {"select": t_sel, "fwd": t_fwd, "bwd": t_bwd} if not merged else {"select": t_sel,
                                                                                          "fwd_bwd": t_fwd + t_bwd},
        "fwd_bwd_tokens_per_s": tokens / ((t_fwd + t_bwd) / 1e3),
        "fwd_bwd_effective_tflops": (f_fwd + f_bwd) / ((t_fwd + t_bwd) / 1e3) / 1e12,
        "select_tflops": f_proxy / (t_sel / 1e3) / 1e12,
        "pairs": pairs,
        "flops": {"fwd": f_fwd, "bwd": f_bwd, "proxy": f_proxy},
        "kernels_ms_per_step": {k: v[0] / steps for k, v in kern.items()},
        "kernel_launches_per_step": {k: v[1] / steps for k, v in kern.items()},
    }
    res["fwd_bwd_frac_of_peak"] = res["fwd_bwd_effective_tflops"] / PEAK_BF16_TFLOPS
    res["roofline"] = roofline(cfg, kern, steps, pairs)
    del x, ws, idx, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return res


DECODE_BATCH = 16  # sequences per decode step, each at the workload's full context


def run_dense_context(steps: int) -> dict:
    """Dense context: the same path with topk = N (every causal block selected,
    i.e. dense causal GQA attention) next to the sparse configuration, at 16K
    and 128K tokens; the sparse/dense ratio of the fwd+bwd time shows how the
    sparse advantage grows with sequence length."""
    out = {"what": "fwd+bwd (cached indices) of the sparse configuration and of the same shapes at topk = N "
                   "(dense causal through the same kernels); flops count every selected 128-key block",
           "runs": []}
    for name in ("16k", "128k"):
        sparse = synth.CONFIGS[name]
        dense = dataclasses.replace(sparse, name=name + "-dense", topk=sparse.N)
        row = {"T": sparse.T}
        for tag, c in (("sparse", sparse), ("dense", dense)):
            r = run_workload(c, steps, 1, host_inputs=False)
            ms = r["phases_ms"]["fwd"] + r["phases_ms"]["bwd"]
            row[tag] = {"topk": c.topk, "pairs": r["pairs"], "fwd_bwd_ms": ms,
                        "fwd_bwd_effective_tflops": r["fwd_bwd_effective_tflops"],
                        "kernels_ms_per_step": {k: v for k, v in r["kernels_ms_per_step"].items() if v}}
        row["dense_over_sparse_time"] = row["dense"]["fwd_bwd_ms"] / row["sparse"]["fwd_bwd_ms"]
        out["runs"].append(row)
        print("bench: dense context %s: sparse %.1f ms, dense %.1f ms" % (
            name, row["sparse"]["fwd_bwd_ms"], row["dense"]["fwd_bwd_ms"]), file=sys.stderr, flush=True)
    return out


def run_decode(cfg: synth.Config, B: int, steps: int, warmup: int) -> dict:
    """One decode step = msa_decode_select + msa_decode_fwd for B sequences whose
    caches hold cfg.T tokens (the new one last)."""
    x = gpu_decode_inputs(cfg, B)
    lens = torch.full((B,), cfg.T, dtype=torch.int32, device="cuda")
    dims = (B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    ws = msa.Workspace(nbytes=max(msa.msa_workspace_bytes(*dims, op)
                                  for op in (msa.OP_DECODE_SELECT, msa.OP_DECODE_FWD)))
    idx = torch.empty((B, cfg.G, cfg.topk), dtype=torch.int32, device="cuda")
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, cfg.H), dtype=torch.float32, device="cuda")

    def step():
        msa.msa_decode_select(x["qp"], x["kp"], lens, cfg.topk, ws=ws, out=idx)
        msa.msa_decode_fwd(x["q"], x["k"], x["v"], lens, idx, ws=ws, out=(o, lse))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    msa.timing_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    kern = {k: v for k, v in msa.timing_read().items() if v[1]}
    msa.timing_enable(False)
    # algorithmic HBM bytes per launch: the causal proxy-key cache rows (pool) and
    # the selected K/V blocks (attention); queries and outputs are noise
    pool_bytes = float(B) * cfg.T * cfg.G * cfg.dp * 2
    attn_bytes = float(B) * cfg.G * min(cfg.topk, cfg.N) * 128 * cfg.d * 2 * 2
    rl = {}
    for name, work in (("dec_pool", pool_bytes), ("dec_attn", attn_bytes)):
        ms, n = kern[name]
        avg_s = ms / n / 1e3
        rl[name] = {"bound": "hbm", "achieved": work / avg_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": work / avg_s / 1e9 / PEAK_HBM_GBS, "traffic": stored_traffic("decode-" + cfg.name, name),
                    "avg_launch_ms": avg_s * 1e3, "work_per_launch": work}
    res = {
        "workload": "%s decode: B=%d sequences at %d cached tokens" % (cfg.name, B, cfg.T),
        "shape": {"B": B, "T": cfg.T, "H": cfg.H, "G": cfg.G, "d": cfg.d, "dp": cfg.dp, "topk": cfg.topk},
        "ms_per_step": ms_step,
        "tokens_per_s": B / (ms_step / 1e3),
        "kernels_ms_per_step": {k: v[0] / steps for k, v in kern.items()},
        "roofline": rl,
    }
    del x, ws, idx, o, lse
    torch.cuda.empty_cache()
    return res


def roofline(cfg: synth.Config, kern: dict, steps: int, pairs: int) -> dict:
    """Roofline entry of the kernel with the largest time: algorithmic work per
    launch divided by its average launch duration."""
    name = max(kern, key=lambda k: kern[k][0])
    ms, launches = kern[name]
    avg_s = ms / max(launches, 1) / 1e3
    per_step_launch = launches / steps
    BG = cfg.B * cfg.G
    f_pair = 4 * cfg.d * cfg.R * 128
    if name == "bwd_partials":
        work, bound, unit = 2.5 * f_pair * pairs / per_step_launch, "mfma", "TFLOP/s"
    elif name == "fwd_partials":
        work, bound, unit = f_pair * pairs / per_step_launch, "mfma", "TFLOP/s"
    elif name == "proxy_pool":
        work, bound, unit = cfg.flops_proxy() / per_step_launch, "mfma", "TFLOP/s"
    elif name in ("fwd_combine", "dq_combine"):
        # read every partial (bf16) once, write the bf16 result (+ lse for fwd)
        work = (pairs * cfg.R * cfg.d * 2 + cfg.B * cfg.T * cfg.H * cfg.d * 2) / per_step_launch
        bound, unit = "hbm", "GB/s"
    else:
        work = float("nan")
        bound, unit = "hbm", "GB/s"
    if unit == "TFLOP/s":
        achieved, peak = work / avg_s / 1e12, PEAK_BF16_TFLOPS
    else:
        achieved, peak = work / avg_s / 1e9, PEAK_HBM_GBS
    return {"kernel": name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": stored_traffic(cfg.name, name), "avg_launch_ms": avg_s * 1e3,
            "work_per_launch": work}


def cpu_baseline(cfg: synth.Config, target_s: float = 15.0) -> dict:
    """The oracle, as it stands, on a uniform sample of query tokens of the same
    workload: Index Branch rows, forward rows and backward dQ rows."""
    import numpy as np
    import oracle

    oracle.build()
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    x = synth.make_inputs(cfg)
    f64 = {n: x[n].double().numpy() for n in x}
    dm = oracle.Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    rng = np.random.default_rng(1)

    def run(n_rows):
        rows = np.sort(rng.choice(cfg.B * cfg.T, size=n_rows, replace=False))
        t0 = time.perf_counter()
        sel = oracle.select(dm, f64["qp"], f64["kp"], rows=rows)                 # [n, G, k]
        idx = np.full((cfg.B, cfg.G, cfg.T, cfg.topk), -1, dtype=np.int32)
        b_, t_ = rows // cfg.T, rows % cfg.T
        idx[b_, :, t_, :] = sel
        oracle.fwd(dm, f64["q"], f64["k"], f64["v"], idx, rows=rows)
        oracle.bwd_rows(dm, f64["q"], f64["k"], f64["v"], f64["dout"], idx, rows=rows)
        return time.perf_counter() - t0

    pilot_rows = 16
    t_pilot = run(pilot_rows)
    n = int(min(4096, max(pilot_rows, pilot_rows * target_s / max(t_pilot, 1e-3))))
    t = run(n)
    # the same kind of sample on one thread, about a third of the time budget
    oracle.set_threads(1)
    n1 = int(max(8, min(n, (n / t) / cores * (target_s / 3))))
    t1 = run(n1)
    oracle.set_threads(cores)
    return {"value": n / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": ("%d query tokens drawn uniformly from the %s workload: Index Branch rows, forward rows and "
                       "backward dQ rows over all heads and groups (the oracle's dK/dV pass is not in the sample); "
                       "%.1f s on %d threads" % (n, cfg.name, t, cores)),
            "single_thread": {"value": n1 / t1, "unit": "tokens/s", "cores": 1,
                              "sample": "%d query tokens of the same kind; %.1f s on 1 thread" % (n1, t1)}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="128k", choices=sorted(synth.CONFIGS))
    ap.add_argument("--also", default="1m,pattern,merged,decode,dense",
                    help="comma list of extra workloads: config names, 'pattern' (the main config with the fixed "
                         "window/dilation pattern united with the proxy top-k), 'merged' (the main config through "
                         "msa_fwd_bwd), 'decode' (decode steps of %d sequences at the main config's full context), "
                         "'dense' (16K and 128K at topk = N beside their sparse configurations); '' for none"
                         % DECODE_BATCH)
    ap.add_argument("--also-steps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference kernel for traffic counters)")
    ap.add_argument("--gpu-inputs", action="store_true",
                    help="draw the main workload's inputs on the GPU (same recipe, different stream; for profiling)")
    ap.add_argument("--decode-only", metavar="CONFIG",
                    help="run only decode steps (%d sequences at CONFIG's full context) and print their record; "
                         "for profiling" % DECODE_BATCH)
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="print calibrated per-kernel HBM bytes from rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR "
                         "(needs --copy-calibration-mib of those runs) and exit; no GPU needed")
    args = ap.parse_args()
    if args.pmc_summary:
        workload = "decode-" + args.decode_only if args.decode_only else args.config
        print(pmc_summary(args.pmc_summary, args.copy_calibration_mib or 1024, workload))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    msa.load()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.decode_only:
        res = run_decode(synth.CONFIGS[args.decode_only], DECODE_BATCH, max(20, 5 * args.steps), 5)
        print(json.dumps(res))
        return 0
    cfg = synth.CONFIGS[args.config]
    print("bench: %s steps=%d warmup=%d" % (cfg, args.steps, args.warmup), file=sys.stderr, flush=True)
    main_res = run_workload(cfg, args.steps, args.warmup, host_inputs=not args.gpu_inputs)
    print("bench: main workload done: %.3f ms/step" % main_res["ms_per_step"], file=sys.stderr, flush=True)
    extra = []
    dense_context = None
    for name in [s for s in args.also.split(",") if s and s != args.config]:
        if name == "pattern":
            print("bench: extra workload %s + pattern %s" % (cfg, PATTERN), file=sys.stderr, flush=True)
            extra.append(run_workload(cfg, args.steps, 2, host_inputs=False, pattern=PATTERN))
            print("bench: pattern done: %.1f ms/step" % extra[-1]["ms_per_step"], file=sys.stderr, flush=True)
            continue
        if name == "merged":
            print("bench: extra workload %s, merged fwd+bwd" % (cfg,), file=sys.stderr, flush=True)
            extra.append(run_workload(cfg, args.steps, 2, host_inputs=False, merged=True))
            print("bench: merged done: %.1f ms/step" % extra[-1]["ms_per_step"], file=sys.stderr, flush=True)
            continue
        if name == "dense":
            print("bench: dense context (topk = N) at 16K and 128K", file=sys.stderr, flush=True)
            dense_context = run_dense_context(args.also_steps)
            continue
        if name == "decode":
            print("bench: decode steps, %d sequences of %s" % (DECODE_BATCH, cfg), file=sys.stderr, flush=True)
            extra.append(run_decode(cfg, DECODE_BATCH, max(20, 5 * args.steps), 5))
            print("bench: decode done: %.3f ms/step" % extra[-1]["ms_per_step"], file=sys.stderr, flush=True)
            continue
        c = synth.CONFIGS[name]
        print("bench: extra workload %s" % (c,), file=sys.stderr, flush=True)
        extra.append(run_workload(c, args.also_steps, 1, host_inputs=False))
        print("bench: %s done: %.1f ms/step" % (name, extra[-1]["ms_per_step"]), file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg)
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d T=%d H=%d G=%d d=%d dp=%d topk=%d; step = proxy select + fwd + bwd" % (
            cfg.name, cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk),
            "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "none (1 GPU)"},
        "roofline": {k: main_res["roofline"][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "roofline_kernel": main_res["roofline"]["kernel"],
        "cpu_baseline": cpu,
        "fwd_bwd_tokens_per_s": main_res["fwd_bwd_tokens_per_s"],
        "fwd_bwd_effective_tflops": main_res["fwd_bwd_effective_tflops"],
        "fwd_bwd_frac_of_bf16_peak": main_res["fwd_bwd_frac_of_peak"],
        "phases_ms": main_res["phases_ms"],
        "kernels_ms_per_step": main_res["kernels_ms_per_step"],
        "workloads": [main_res] + extra,
    }
    if dense_context is not None:
        line["dense_context"] = dense_context
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
