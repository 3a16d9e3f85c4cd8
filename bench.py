#!/usr/bin/env python3
"""Benchmark of the MSA training hot path on one MI355X (gfx950).

One step is the whole hot path over one batch of synthetic input:
msa_proxy_select (Index Branch: proxy score, block max-pool, top-k into the
block-index cache) -> msa_fwd -> msa_bwd (Main Branch over the cached blocks).
Inputs are resident in HBM before the timed region.  W warm-up steps, then K
timed steps between two device synchronisations.

Printed: one JSON line.  `value` is tokens/s of the whole step on the main
workload (the 128K configuration: B=1, T=131072, 32 query / 4 KV heads, head
dim 128, 4 proxy heads of dim 64, top-k 32), from the median of the K
per-step times (HIP events around each step; the mean is reported beside it).
Extra fields give the fwd+bwd rate with cached indices, effective TFLOP/s on
the executed sparse FLOPs, per-phase and per-kernel times (HIP events recorded
by the library on the launch stream), the roofline of the dominant kernel,
extra workloads (the 512K and 1M configurations; the 128K step on a fixed
window/dilation pattern united with the proxy top-k; the 128K step through the
merged forward/backward call; decode steps of 16 sequences at 128K cached
tokens), the dense context (topk = N through the same kernels, forward and
backward ratios), the device memory of separate against merged calls, and the
CPU oracle timed on bounded samples (extrapolated where marked).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--also 512k,1m,pattern,merged,decode,dense,memory|''] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import statistics
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
    "topk": ("msa::k_topk", ("msa_select.hip", "msa_topk.h")),  # k_topk and k_topk_wg
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
    kern = msa.timing_read()
    msa.timing_enable(False)

    # per-step times from the step's own events; the reported figures are medians
    per_step = [e[0].elapsed_time(e[3]) for e in evs]
    per_phase = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(3)]
    tokens = cfg.B * cfg.T
    ms_step = statistics.median(per_step)
    t_sel, t_fwd, t_bwd = (statistics.median(p) for p in per_phase)
    t_fb = statistics.median([a + b for a, b in zip(per_phase[1], per_phase[2])])
    f_pair = 4 * cfg.d * cfg.R * 128  # forward flop per (token, group, block); backward is 2.5x
    f_fwd, f_bwd, f_proxy = f_pair * pairs, 2.5 * f_pair * pairs, cfg.flops_proxy()
    res = {
        "workload": cfg.name + ("+pattern(window=%d,dilation=%d)" % pattern if pattern else "") +
                    (" merged fwd+bwd (msa_fwd_bwd)" if merged else ""),
        "shape": {"B": cfg.B, "T": cfg.T, "H": cfg.H, "G": cfg.G, "d": cfg.d, "dp": cfg.dp, "topk": cfg.topk,
                  "cache_width": width},
        "steps": steps,
        "ms_per_step": ms_step,
        "ms_per_step_mean": total_ms / steps,
        "ms_per_step_min_max": [min(per_step), max(per_step)],
        "wall_ms_per_step": 1e3 * wall / steps,
        "tokens_per_s": tokens / (ms_step / 1e3),
        "phases_ms": {"select": t_sel, "fwd": t_fwd, "bwd": t_bwd} if not merged else {"select": t_sel,
                                                                                          "fwd_bwd": t_fb},
        "fwd_bwd_ms": t_fb,
        "fwd_bwd_tokens_per_s": tokens / (t_fb / 1e3),
        "fwd_bwd_effective_tflops": (f_fwd + f_bwd) / (t_fb / 1e3) / 1e12,
        "select_tflops": f_proxy / (t_sel / 1e3) / 1e12,
        "pairs": pairs,
        "flops": {"fwd": f_fwd, "bwd": f_bwd, "proxy": f_proxy},
        "kernels_ms_per_step": {k: v[0] / steps for k, v in kern.items()},
        "kernel_launches_per_step": {k: v[1] / steps for k, v in kern.items()},
    }
    res["fwd_bwd_frac_of_peak"] = res["fwd_bwd_effective_tflops"] / PEAK_BF16_TFLOPS
    res["roofline"] = roofline(cfg, kern, steps, pairs, res["workload"])
    del x, ws, idx, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return res


DECODE_BATCH = 16  # sequences per decode step, each at the workload's full context

# timed steps (after one warm-up) of the long-context legs
LEG_STEPS = {"512k": 5, "1m": 3}


def memory_footprint(cfg: synth.Config) -> dict:
    """Device memory of the Main Branch calls, separate (msa_fwd, then msa_bwd)
    against merged (msa_fwd_bwd), with cached indices: the activations a
    training step keeps between forward and backward, and the peak allocated
    during the calls (workspace, activations and outputs; the inputs q, k, v,
    dout and idx are resident beforehand and not counted)."""
    x = gpu_inputs(cfg)
    idx = msa.msa_proxy_select(x["qp"], x["kp"], cfg.topk)
    del x["qp"], x["kp"]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    dims = (cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    out = {"workload": cfg.name, "unit": "bytes"}
    for tag in ("separate", "merged"):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        if tag == "separate":
            ws = msa.Workspace(nbytes=msa.msa_workspace_bytes(*dims, msa.OP_FWD))
            o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx, ws=ws)
            ws_f = ws.get(0).numel()
            del ws
            kept = o.numel() * o.element_size() + lse.numel() * lse.element_size()
            ws = msa.Workspace(nbytes=msa.msa_workspace_bytes(*dims, msa.OP_BWD))
            grads = msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, ws=ws)
            ws_b = ws.get(0).numel()
            out[tag] = {"workspace_fwd": ws_f, "workspace_bwd": ws_b, "activations_kept": kept}
        else:
            ws = msa.Workspace(nbytes=msa.msa_workspace_bytes(*dims, msa.OP_FWD_BWD))
            res = msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx, ws=ws)
            out[tag] = {"workspace": ws.get(0).numel(), "activations_kept": 0}
            o, lse, grads = res[0], res[1], res[2:]
        torch.cuda.synchronize()
        out[tag]["peak_during_calls"] = torch.cuda.max_memory_allocated() - base
        del ws, o, lse, grads
    out["activations_kept_note"] = ("between forward and backward the separate calls keep o and lse (idx is kept "
                                    "by both); the merged call recomputes the forward and keeps nothing more")
    del x, idx
    torch.cuda.empty_cache()
    return out



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
            row[tag] = {"topk": c.topk, "pairs": r["pairs"], "fwd_ms": r["phases_ms"]["fwd"],
                        "bwd_ms": r["phases_ms"]["bwd"], "fwd_bwd_ms": r["fwd_bwd_ms"],
                        "fwd_bwd_effective_tflops": r["fwd_bwd_effective_tflops"],
                        "kernels_ms_per_step": {k: v for k, v in r["kernels_ms_per_step"].items() if v}}
        row["dense_over_sparse_time"] = row["dense"]["fwd_bwd_ms"] / row["sparse"]["fwd_bwd_ms"]
        row["dense_over_sparse_fwd"] = row["dense"]["fwd_ms"] / row["sparse"]["fwd_ms"]
        row["dense_over_sparse_bwd"] = row["dense"]["bwd_ms"] / row["sparse"]["bwd_ms"]
        out["runs"].append(row)
        print("bench: dense context %s: sparse %.1f ms, dense %.1f ms (fwd %.1fx, bwd %.1fx)" % (
            name, row["sparse"]["fwd_bwd_ms"], row["dense"]["fwd_bwd_ms"], row["dense_over_sparse_fwd"],
            row["dense_over_sparse_bwd"]), file=sys.stderr, flush=True)
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


def roofline(cfg: synth.Config, kern: dict, steps: int, pairs: int, traffic_key: str = "") -> dict:
    """Roofline entry of the kernel with the largest time: algorithmic work per
    launch divided by its average launch duration.  `traffic_key` names the
    workload whose committed counter summary applies (the plain workload by
    default); legs with other launch patterns pass their own name, for which no
    summary exists, so their traffic is reported as unknown."""
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
            "frac": achieved / peak, "traffic": stored_traffic(traffic_key or cfg.name, name),
            "avg_launch_ms": avg_s * 1e3,
            "work_per_launch": work}


def _cpu_host_rows(cfg: synth.Config, rows):
    """Float64 host inputs for the oracle on the given token rows (B = 1):
    q, dout and qp hold only those rows (the rest stay untouched zero pages),
    k, v and kp are whole.  Drawn with synth's seeded per-chunk generators, so
    the values are the workload's own."""
    import numpy as np
    assert cfg.B == 1
    T = cfg.T
    out = {}
    for name in ("k", "v", "kp"):
        parts = [synth.make_tensor(name, cfg, t0, min(T, t0 + (1 << 17))).double().numpy()
                 for t0 in range(0, T, 1 << 17)]
        out[name] = np.concatenate(parts, axis=1)
    for name in ("q", "dout", "qp"):
        width = (cfg.H, cfg.d) if name != "qp" else (cfg.G, cfg.dp)
        a = np.zeros((1, T) + width, dtype=np.float64)
        for c in np.unique(rows // synth.CHUNK):
            t0, t1 = int(c) * synth.CHUNK, min(T, (int(c) + 1) * synth.CHUNK)
            sel = rows[(rows >= t0) & (rows < t1)]
            a[0, sel] = synth.make_tensor(name, cfg, t0, t1).double().numpy()[0, sel - t0]
        out[name] = a
    return out


def _oracle_rows(cfg, dm, x, rows):
    """Oracle Index Branch, forward and backward dQ on the sampled rows; seconds of each."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    sel = oracle.select(dm, x["qp"], x["kp"], rows=rows)
    t1 = time.perf_counter()
    idx = np.full((cfg.B, cfg.G, cfg.T, cfg.topk), -1, dtype=np.int32)
    idx[rows // cfg.T, :, rows % cfg.T, :] = sel
    oracle.fwd(dm, x["q"], x["k"], x["v"], idx, rows=rows)
    t2 = time.perf_counter()
    oracle.bwd_rows(dm, x["q"], x["k"], x["v"], x["dout"], idx, rows=rows)
    t3 = time.perf_counter()
    return t1 - t0, t2 - t1, t3 - t2


def _dkdv_ratio(cfg: synth.Config) -> float:
    """Cost of the oracle's dK/dV pass relative to its dQ rows on one small
    full problem with the workload's head shape (T = 2048, one group): the
    full backward is the dQ rows plus that pass, which repeats each row's score
    work and scatters into the key rows."""
    import oracle
    c = synth.custom(1, 2048, cfg.R, 1, cfg.d, cfg.dp, min(cfg.topk, 16))
    x = {n: t.double().numpy() for n, t in synth.make_inputs(c, seed_offset=5).items()}
    dm = oracle.Dims(c.B, c.T, c.H, c.G, c.d, c.dp, c.topk)
    idx = oracle.select(dm, x["qp"], x["kp"])
    oracle.bwd_rows(dm, x["q"], x["k"], x["v"], x["dout"], idx)  # warm-up: threads, pages
    oracle.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    t_rows, t_full = [], []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.bwd_rows(dm, x["q"], x["k"], x["v"], x["dout"], idx)
        t1 = time.perf_counter()
        oracle.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
        t2 = time.perf_counter()
        t_rows.append(t1 - t0)
        t_full.append(t2 - t1)
    tr, tf = statistics.median(t_rows), statistics.median(t_full)
    return max(0.0, tf - tr) / tr


def cpu_full(cfg: synth.Config) -> dict:
    """The whole oracle on the whole workload: Index Branch, forward and the
    full backward (dQ rows and the dK/dV pass)."""
    import oracle
    x = {n: t.double().numpy() for n, t in synth.make_inputs(cfg).items()}
    dm = oracle.Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    t0 = time.perf_counter()
    idx = oracle.select(dm, x["qp"], x["kp"])
    t1 = time.perf_counter()
    oracle.fwd(dm, x["q"], x["k"], x["v"], idx)
    oracle.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    t2 = time.perf_counter()
    tokens = cfg.B * cfg.T
    return {"config": cfg.name, "value": tokens / (t2 - t0), "unit": "tokens/s", "seconds": t2 - t0,
            "fwd_bwd_tokens_per_s": tokens / (t2 - t1), "extrapolated": False,
            "sample": "the whole %s workload: select, fwd and the full bwd; %.1f s" % (cfg.name, t2 - t0)}


def cpu_sampled(cfg: synth.Config, n_rows: int, ratio: float, max_chunks: int = 32, seed: int = 1) -> dict:
    """The oracle on a seeded uniform sample of query tokens of the workload
    (rows drawn uniformly inside up to `max_chunks` randomly chosen 4096-token
    chunks), extrapolated to the whole step: the Index Branch by the ratio of
    causal keys scored, the forward and backward by the ratio of (token, group,
    block) pairs, the dK/dV pass as `ratio` times the dQ rows' time."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(seed)
    nchunk = (cfg.T + synth.CHUNK - 1) // synth.CHUNK
    chunks = np.sort(rng.choice(nchunk, size=min(nchunk, max_chunks), replace=False))
    per = max(1, n_rows // len(chunks))
    rows = np.unique(np.concatenate([c * synth.CHUNK + rng.choice(synth.CHUNK, size=per, replace=False)
                                     for c in chunks]))
    x = _cpu_host_rows(cfg, rows)
    dm = oracle.Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    t_sel, t_fwd, t_dq = _oracle_rows(cfg, dm, x, rows)
    keys_all = cfg.B * cfg.G * cfg.T * (cfg.T + 1) / 2.0
    keys_s = cfg.G * float(np.sum(rows + 1))
    pairs_s = cfg.G * float(np.sum(np.minimum(cfg.topk, rows // synth.BLOCK + 1)))
    f_keys, f_pairs = keys_all / keys_s, cfg.pairs() / pairs_s
    t_sel_all = t_sel * f_keys
    t_fb_all = (t_fwd + t_dq * (1.0 + ratio)) * f_pairs
    tokens = cfg.B * cfg.T
    return {"config": cfg.name, "value": tokens / (t_sel_all + t_fb_all), "unit": "tokens/s",
            "fwd_bwd_tokens_per_s": tokens / t_fb_all, "seconds_sampled": t_sel + t_fwd + t_dq,
            "seconds_extrapolated": t_sel_all + t_fb_all, "extrapolated": True,
            "sample": ("%d query tokens from %d of %d chunks of the %s workload; select, fwd and dQ rows timed "
                       "(%.1f s), extrapolated by causal keys scored (x%.0f) and by pairs (x%.0f); the dK/dV "
                       "pass counted as %.2fx the dQ rows" % (len(rows), len(chunks), nchunk, cfg.name,
                                                               t_sel + t_fwd + t_dq, f_keys, f_pairs, ratio))}


def cpu_baseline(cfg: synth.Config, target_s: float = 15.0, others=("tiny", "16k", "512k", "1m")) -> dict:
    """The oracle as it stands, timed on this host's cores: the main workload
    on a sample of about target_s seconds extrapolated to the whole step, a
    single-thread rate on a smaller sample, and one entry per other
    configuration (tiny and 16K whole, 512K and 1M sampled and extrapolated)."""
    import oracle

    oracle.build()
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    ratio = _dkdv_ratio(cfg)
    pilot = cpu_sampled(cfg, 64, ratio)
    n = int(min(4096, max(64, 64 * target_s / max(pilot["seconds_sampled"], 1e-3))))
    main = cpu_sampled(cfg, n, ratio, seed=2)
    oracle.set_threads(1)
    n1 = int(max(16, min(n, n / main["seconds_sampled"] / cores * (target_s / 3))))
    single = cpu_sampled(cfg, n1, ratio, seed=3)
    oracle.set_threads(cores)
    per_config = []
    for name in others:
        c = synth.CONFIGS[name]
        print("bench: cpu baseline %s" % name, file=sys.stderr, flush=True)
        if c.T <= 16384:
            per_config.append(cpu_full(c))
        else:
            per_config.append(cpu_sampled(c, 32 if c.topk > 128 else 64, _dkdv_ratio(c), max_chunks=8, seed=4))
    return {"value": main["value"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": main["sample"] + "; %d threads" % cores, "extrapolated": True,
            "fwd_bwd_tokens_per_s": main["fwd_bwd_tokens_per_s"],
            "single_thread": {"value": single["value"], "unit": "tokens/s", "cores": 1,
                              "sample": single["sample"] + "; 1 thread"},
            "per_config": per_config}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="128k", choices=sorted(synth.CONFIGS))
    ap.add_argument("--also", default="512k,1m,pattern,merged,decode,dense,memory",
                    help="comma list of extra workloads: config names, 'pattern' (the main config with the fixed "
                         "window/dilation pattern united with the proxy top-k), 'merged' (the main config through "
                         "msa_fwd_bwd), 'decode' (decode steps of %d sequences at the main config's full context), "
                         "'dense' (16K and 128K at topk = N beside their sparse configurations), 'memory' (device "
                         "memory of separate against merged calls at 128K and 1M); '' for none" % DECODE_BATCH)
    ap.add_argument("--also-steps", type=int, default=0,
                    help="timed steps of the config legs (0: 5 at 512K, 3 at 1M) and of the dense context (0: 2)")
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
    memory = None
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
            dense_context = run_dense_context(args.also_steps or 2)
            continue
        if name == "memory":
            print("bench: device memory, separate against merged calls", file=sys.stderr, flush=True)
            memory = [memory_footprint(synth.CONFIGS[c]) for c in ("128k", "1m")]
            continue
        if name == "decode":
            print("bench: decode steps, %d sequences of %s" % (DECODE_BATCH, cfg), file=sys.stderr, flush=True)
            extra.append(run_decode(cfg, DECODE_BATCH, max(20, 5 * args.steps), 5))
            print("bench: decode done: %.3f ms/step" % extra[-1]["ms_per_step"], file=sys.stderr, flush=True)
            continue
        c = synth.CONFIGS[name]
        print("bench: extra workload %s" % (c,), file=sys.stderr, flush=True)
        extra.append(run_workload(c, args.also_steps or LEG_STEPS.get(name, 3), 1, host_inputs=False))
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
    if memory is not None:
        line["memory"] = memory
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
