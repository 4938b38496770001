#!/usr/bin/env python3
"""Throughput of one routed-expert MoE layer on one MI355X.

A step is one whole layer over one prompt, through the C ABI
(moe_layer_prefill): fp32 router logits, top-k routing, the per-slot route
map, gate/up + SwiGLU and down projections on bf16 MFMA, and the fixed-order
combine into the fp32 accumulator. Inputs and weights are resident in HBM
before timing starts; data is synthetic (seeded, the shapes of the models on
the pages; no trained weights).

Prints one JSON line: routed tokens/s (T / layer time), the % of the bf16
MFMA peak the layer reaches on its algorithmic FLOPs, a roofline entry for
the dominant kernel (the gate/up projection), and the CPU oracle's throughput
on a bounded sample of the same workload (all host cores and one core).

    python bench.py [--steps K] [--warmup W] [--workload olmoe_t4096]

Order of the run:
  1. warm-up: W layers, continued until --warmup-min-s seconds have passed,
     so that the timed steps run at steady clocks (the GPU's clocks ramp over
     the first few tens of back-to-back layers); the first 20 warm-up layers
     are timed one by one and reported, which shows the ramp;
  2. the timed region: K layers between two events, nothing else recorded;
  3. a second pass of K layers with one event between consecutive layers:
     median, p10, p90, first and last step;
  4. a third pass of K layers with every gate/up launch bracketed by HIP
     events on its stream: the roofline's kernel time;
  5. a per-kernel breakdown pass (every launch bracketed);
  6. the CPU oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer + % bf16 MFMA peak at T=4096 (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

WORKLOAD_TEXT = {
    "olmoe_t4096": "OLMoE-shaped MoE layer: T=4096 tokens, d=2048, E=64 experts, top-8 renormalised, "
                   "SwiGLU f=1024, bf16 weights/activations, fp32 router and accumulator",
    "olmoe_t1024": "OLMoE-shaped MoE layer: T=1024 tokens, d=2048, E=64 experts, top-8 renormalised, "
                   "SwiGLU f=1024, bf16",
    "dsv2lite_t4096": "DeepSeek-V2-Lite-shaped MoE layer: T=4096, d=2048, 64 routed experts top-6 "
                      "(not renormalised) + 2 shared, SwiGLU f=1408, bf16",
    "mixtral_t4096": "Mixtral-8x7B-shaped MoE layer: T=4096, d=4096, E=8, top-2 renormalised, SwiGLU "
                     "f=14336, bf16",
    "mixtral_t1024": "Mixtral-8x7B-shaped MoE layer: T=1024, d=4096, E=8, top-2, f=14336, bf16",
    "mixtral_t256": "Mixtral-8x7B-shaped MoE layer: T=256, d=4096, E=8, top-2, f=14336, bf16",
    "tiny_fp32": "tiny fp32 MoE layer: T=64, d=128, E=8, top-2, f=256",
}
for _t in (256, 512, 1024, 2048, 4096):
    WORKLOAD_TEXT[f"virt_olmoe_t{_t}"] = (
        f"OLMoE-shaped MoE layer with experts paged from pinned host memory: T={_t}, d=2048, E=64, "
        "top-8 with a Zipf(1.1) popularity bias, f=1024, bf16; P=16 arena slots in 2 banks of G=8")
for _t in (256, 1024, 4096):
    WORKLOAD_TEXT[f"mixtral_stack_t{_t}"] = (
        f"32 Mixtral-8x7B-shaped MoE layers with independent weights, all resident (90.2 GB): T={_t}, "
        "d=4096, E=8, top-2 renormalised, SwiGLU f=14336, bf16; only the MoE sublayers are timed")
for _n in list(WORKLOAD_TEXT):
    if _n in ("tiny_fp32", "virt_olmoe_t512", "virt_olmoe_t2048"):   # no quantised-weight variant
        continue
    _act = WORKLOAD_TEXT[_n].replace("bf16 weights/activations", "bf16").replace(", bf16", ", bf16 activations")
    WORKLOAD_TEXT[_n + "_fp8w"] = (_act
                                   + "; expert weights stored as fp8 e4m3 codes with one fp32 scale per row "
                                   "(weight-only quantisation, decoded to bf16 MFMA operands)")
    WORKLOAD_TEXT[_n + "_fp4w"] = (_act
                                   + "; expert weights stored as MXFP4 (E2M1 codes, one E8M0 scale per 32 "
                                   "weights of a row; weight-only quantisation, decoded to bf16 MFMA operands)")
PCIE_GEN5_X16_GBS = 64.0   # one direction, before protocol overhead
MALL_BYTES = 256 << 20     # MI355X Infinity Cache


def working_set_bytes(cfg) -> int:
    """Bytes one layer touches: expert weights, X, Y, and the intermediate H
    and per-route rows Yr."""
    esz = 4 if cfg.dtype == "f32" else 2
    R = cfg.T * cfg.kp
    return (cfg.n_exp * expert_slice_bytes(cfg) + cfg.T * cfg.d * (esz + 4) + R * cfg.f * esz + R * cfg.d * 4)


def cold_cache_steps(torch, layer, Y, K, scratch_bytes=512 << 20) -> dict:
    """Layer time with caches cold: before each layer a 512 MB scratch buffer
    is written (twice the 256 MB Infinity Cache), then the layer alone is
    timed between two events. For working sets that fit in the cache."""
    import numpy as np
    scratch = torch.empty(scratch_bytes // 4, dtype=torch.float32, device="cuda")
    times = []
    for i in range(K + 2):
        scratch.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        layer.forward(Y)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(a.elapsed_time(b))
    del scratch
    return {"median_ms": round(float(np.median(times)), 4), "p10_ms": round(float(np.percentile(times, 10)), 4),
            "p90_ms": round(float(np.percentile(times, 90)), 4), "steps": K,
            "method": "512 MB scratch write before each layer, layer timed alone"}


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("expert_gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "routed_expert_ffn_top_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, launch_flops: float):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != gemm_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_per_kernel(path: str, counter: str) -> dict:
    """Average of one counter per dispatch, by kernel name, from a
    rocprofv3 --pmc counter_collection.csv."""
    import csv
    tot, n = {}, {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
            n[k] = n.get(k, 0) + 1
    return {k: (tot[k] / n[k], n[k]) for k in tot}


def summarize_pmc(fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, out, command) -> None:
    """HBM bytes per gate/up launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain 1 GiB
    device copy (bench.py --copy-calibration)."""
    def pick(d, key):
        hits = {k: v for k, v in d.items() if key(k)}
        if not hits:
            raise SystemExit(f"no matching kernel in {list(d)[:5]}")
        return max(hits.items(), key=lambda kv: kv[1][0])
    is_gu = lambda k: "k_gemm_mfma_lds<" in k and ", true, false, false>" in k   # gate/up, bf16 weights
    is_copy = lambda k: "elementwise" in k.lower() and "Mul" in k
    gf_name, (gf, gfn) = pick(_pmc_per_kernel(fetch_csv, "FETCH_SIZE"), is_gu)
    gw_name, (gw, gwn) = pick(_pmc_per_kernel(write_csv, "WRITE_SIZE"), is_gu)
    cf_name, (cf, _) = pick(_pmc_per_kernel(calib_fetch_csv, "FETCH_SIZE"), is_copy)
    cw_name, (cw, _) = pick(_pmc_per_kernel(calib_write_csv, "WRITE_SIZE"), is_copy)
    copy_bytes = float(1 << 30)
    kf, kw = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    fetch_b, write_b = gf * 1024.0 * kf, gw * 1024.0 * kw
    with open(out, "w") as fh:
        fh.write(f"# HBM traffic of the gate/up projection kernel, OLMoE-shaped layer T=4096\n")
        fh.write(f"# command: {command}\n")
        fh.write(f"# kernel: {gf_name[:120]}\n")
        fh.write(f"# calibration kernel: {cf_name[:100]} (reads 1 GiB, writes 1 GiB)\n")
        fh.write(f"kernel_source_hash: {gemm_source_hash()}\n")
        fh.write(f"dispatches_fetch: {gfn}\ndispatches_write: {gwn}\n")
        fh.write(f"fetch_kib_per_dispatch_raw: {gf:.1f}\nwrite_kib_per_dispatch_raw: {gw:.1f}\n")
        fh.write(f"copy_fetch_kib_raw: {cf:.1f}\ncopy_write_kib_raw: {cw:.1f}\n")
        fh.write(f"fetch_scale: {kf:.4f}\nwrite_scale: {kw:.4f}\n")
        fh.write(f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}\nhbm_write_bytes_per_launch: {write_b:.0f}\n")
        fh.write(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}\n")
    print(open(out).read())


def _stats_avg_us(stats_csv) -> dict:
    """Average duration (us) per kernel name from a rocprofv3 kernel_stats.csv."""
    import csv
    out = {}
    for r in csv.DictReader(open(stats_csv)):
        out[r.get("Name") or r.get("KernelName") or "?"] = float(r.get("AverageNs", 0)) / 1e3
    return out


# The layer's kernels, by a test on the full kernel name.
LAYER_KERNELS = (
    ("router", lambda k: "k_router_logits<" in k),
    ("top-k", lambda k: "k_topk<" in k),
    ("route count", lambda k: "k_route_count" in k),
    ("route place", lambda k: "k_route_place" in k),
    ("gate/up", lambda k: "k_gemm_mfma_lds<" in k and ", true, false, false>" in k),
    ("down", lambda k: "k_gemm_mfma_lds<" in k and ", false, false, false>" in k),
    ("combine", lambda k: "k_combine<" in k),
)


def layer_algorithmic(cfg) -> dict:
    """Algorithmic HBM bytes and MFMA FLOPs per launch of each layer kernel
    (bf16 activations and weights; the method's own traffic: each input read
    once, each output written once)."""
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
    kp = k + cfg.n_shared
    ne = E + cfg.n_shared   # expert slices read: the routed experts and the shared ones
    R = T * kp
    return {
        "router": (T * d * 2 + E * d * 4 + T * E * 4, 2.0 * T * E * d),
        "top-k": (T * E * 4 + T * kp * 8, 0.0),
        "route count": (R * 4, 0.0),
        "route place": (R * 4 + R * 12, 0.0),
        "gate/up": (ne * 2 * f * d * 2 + R * d * 2 + R * f * 2, 4.0 * R * d * f),
        "down": (ne * d * f * 2 + R * f * 2 + R * d * 4, 2.0 * R * d * f),
        "combine": (R * d * 4 + 2 * T * d * 4, 0.0),
    }


def summarize_kernels(fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, mfma_csv, stats_csv, out,
                      command, workload) -> None:
    """Per layer kernel: trace-average duration, HBM bytes (FETCH_SIZE and
    WRITE_SIZE scaled by the 1 GiB copy calibration) and GB/s, algorithmic
    bytes, MFMA busy % (MfmaUtil) and MFMA FLOPs counted by the hardware
    (MfmaFlopsBF16 + MfmaFlopsF32) against the algorithmic FLOPs."""
    from routed_expert_ffn_top_amd.inputs import CONFIGS
    cfg = CONFIGS[workload]
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    is_copy = lambda k: "elementwise" in k.lower() and "Mul" in k
    cf = max(v for k, v in _pmc_per_kernel(calib_fetch_csv, "FETCH_SIZE").items() if is_copy(k))[0]
    cw = max(v for k, v in _pmc_per_kernel(calib_write_csv, "WRITE_SIZE").items() if is_copy(k))[0]
    kf, kw = float(1 << 30) / (cf * 1024.0), float(1 << 30) / (cw * 1024.0)
    util = _pmc_per_kernel(mfma_csv, "MfmaUtil")
    fl16 = _pmc_per_kernel(mfma_csv, "MfmaFlopsBF16")
    fl32 = _pmc_per_kernel(mfma_csv, "MfmaFlopsF32")
    dur = _stats_avg_us(stats_csv)
    alg = layer_algorithmic(cfg)

    def one(d, test):
        hits = [v[0] for k, v in d.items() if test(k)]
        return max(hits) if hits else float("nan")

    with open(out, "w") as fh:
        fh.write(f"# Layer kernels: HBM traffic, bandwidth and MFMA use ({workload}: T={cfg.T}, d={cfg.d}, "
                 f"E={cfg.E}, k={cfg.k}, f={cfg.f})\n\n")
        fh.write(f"Commands: {command}\n\n")
        fh.write(f"HBM bytes = FETCH_SIZE x {kf:.3f} + WRITE_SIZE x {kw:.3f} (KiB per dispatch; the factors make a "
                 "plain 1 GiB device copy read and write 1 GiB). Duration: trace average of the timed run. "
                 "MFMA busy: MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs). MFMA FLOPs: "
                 "(SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F32) x 512, all rows of every tile included.\n\n")
        fh.write("| kernel | avg us | HBM MB | HBM GB/s | algorithmic MB | HBM / algorithmic | MFMA busy % | "
                 "MFMA GFLOP counted | algorithmic GFLOP |\n|---|---|---|---|---|---|---|---|---|\n")
        for name, test in LAYER_KERNELS:
            us = one({k: (v, 1) for k, v in dur.items()}, test)
            hb = one(fetch, test) * 1024.0 * kf + one(write, test) * 1024.0 * kw
            ab, af = alg[name]
            u = one(util, test)
            fc = one(fl16, test) + one(fl32, test)
            fh.write(f"| {name} | {us:.1f} | {hb / 1e6:.1f} | {hb / (us * 1e-6) / 1e9:.0f} | {ab / 1e6:.1f} | "
                     f"{hb / ab:.2f} | {u:.1f} | {fc / 1e9:.1f} | {af / 1e9:.1f} |\n")
    print(open(out).read())


def summarize_stats(stats_csv, out, command) -> None:
    """Markdown table of a rocprofv3 --stats kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    with open(out, "w") as fh:
        fh.write("# rocprofv3 kernel statistics\n\n")
        fh.write(f"Command: `{command}`\n\n")
        fh.write("| kernel | calls | avg us | min us | max us | total % |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = r.get("Name") or r.get("KernelName") or "?"
            short = name.replace("void ", "").replace("(anonymous namespace)::", "")
            short = short[:short.rfind("(")] if short.endswith(")") and "(" in short else short
            short = short[:90]
            avg = float(r.get("AverageNs", 0)) / 1e3
            mn = float(r.get("MinNs", 0)) / 1e3
            mx = float(r.get("MaxNs", 0)) / 1e3
            fh.write(f"| `{short}` | {r.get('Calls')} | {avg:.1f} | {mn:.1f} | {mx:.1f} | "
                     f"{float(r.get('Percentage', 0)):.2f} |\n")
    print(open(out).read())


def torch_matmul_ceiling(torch, n=8192, reps=10) -> float:
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        a @ b
    e.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (s.elapsed_time(e) / 1e3) / 1e12


def torch_bmm_expert_shape(torch, cfg, reps=10) -> dict:
    """The vendor library (torch.bmm on hipBLASLt) on the dense batched
    equivalent of the two projections: every expert gets exactly the mean
    number of rows, with no gather, no scatter and no SwiGLU."""
    m = cfg.T * cfg.kp // cfg.n_exp
    out = {}
    for name, n, k in (("gate_up", 2 * cfg.f, cfg.d), ("down", cfg.d, cfg.f)):
        a = torch.randn((cfg.n_exp, m, k), device="cuda", dtype=torch.bfloat16)
        b = (torch.randn((cfg.n_exp, k, n), device="cuda", dtype=torch.bfloat16) * 0.02).contiguous()
        for _ in range(3):
            torch.bmm(a, b)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            torch.bmm(a, b)
        e.record()
        torch.cuda.synchronize()
        out[f"torch_bmm_{name}_{cfg.n_exp}x{m}x{n}x{k}_tflops"] = round(
            2.0 * cfg.n_exp * m * n * k * reps / (s.elapsed_time(e) / 1e3) / 1e12, 1)
        del a, b
    return out


def expert_slice_bytes(cfg) -> int:
    """Bytes of one expert's gate/up and down slices (fp8: codes plus the
    fp32 row scales; MXFP4: half a byte a weight plus a scale byte per 32)."""
    if cfg.fp4_weights:
        return 3 * cfg.d * cfg.f // 2 + 3 * cfg.d * cfg.f // 32
    if cfg.fp8_weights:
        return 3 * cfg.d * cfg.f + (2 * cfg.f + cfg.d) * 4
    return 3 * cfg.d * cfg.f * (4 if cfg.dtype == "f32" else 2)


def cpu_baseline(inp, cfg, target_s=12.0, one_core_s=6.0) -> dict:
    """The CPU oracle (as it stands) on the same workload, on all host cores
    (OpenMP over tokens) and on one core: router, top-k and route map for the
    tokens of the leg, then the expert FFN on a token sample sized to about
    the leg's target seconds, extrapolated to the whole layer."""
    import numpy as np
    from oracle import oracle as oracle_mod

    orc = oracle_mod.get()
    f32 = lambda t: t.detach().float().cpu().numpy()
    X, Wr = f32(inp.X), f32(inp.Wr)
    bias = None if inp.bias is None else f32(inp.bias)
    scales = None
    if cfg.fp8_weights:   # the oracle decodes the e4m3 codes itself and applies the row scales
        dec = lambda q: orc.fp8e4m3_decode(q.cpu().numpy())
        Wg, Wu, Wd = dec(inp.Wg), dec(inp.Wu), dec(inp.Wd)
        scales = (f32(inp.Sg), f32(inp.Su), f32(inp.Sd))
    elif cfg.fp4_weights:   # the oracle decodes the MXFP4 codes and block scales to fp32 weights
        dec = lambda q, s: orc.mxfp4_decode(q.cpu().numpy(), s.cpu().numpy())
        Wg, Wu, Wd = dec(inp.Wg, inp.Sg), dec(inp.Wu, inp.Su), dec(inp.Wd, inp.Sd)
    else:
        Wg, Wu, Wd = f32(inp.Wg), f32(inp.Wu), f32(inp.Wd)
    all_threads = orc.threads()

    def leg(threads, budget_s, route_tokens):
        orc.set_threads(threads)
        rt = np.arange(route_tokens)
        t0 = time.perf_counter()
        L = orc.router_logits(X[rt], Wr, bias)
        idx, alpha = orc.topk(L, cfg.k, cfg.n_shared, cfg.renorm)
        orc.route_map(idx, np.arange(cfg.n_exp, dtype=np.int32), cfg.n_exp)
        t_route = (time.perf_counter() - t0) * cfg.T / route_tokens
        idx_all, alpha_all = np.zeros((cfg.T, cfg.kp), np.int32), np.zeros((cfg.T, cfg.kp))
        idx_all[rt], alpha_all[rt] = idx, alpha
        probe = min(route_tokens, max(threads, 4))
        t1 = time.perf_counter()
        orc.expert_ffn(X, idx_all, alpha_all, Wg, Wu, Wd, None, tokens=np.arange(probe), scales=scales)
        per_tok = (time.perf_counter() - t1) / probe
        n = int(min(route_tokens, max(probe, budget_s / max(per_tok, 1e-9))))
        rng = np.random.default_rng(5)
        toks = np.sort(rng.choice(route_tokens, size=n, replace=False))
        t2 = time.perf_counter()
        orc.expert_ffn(X, idx_all, alpha_all, Wg, Wu, Wd, None, tokens=toks, scales=scales)
        t_ffn = time.perf_counter() - t2
        t_layer = t_route + t_ffn * cfg.T / n
        return cfg.T / t_layer, t_route, n, t_ffn

    v, t_route, n, t_ffn = leg(all_threads, target_s, cfg.T)
    v1, t_route1, n1, t_ffn1 = leg(1, one_core_s, min(cfg.T, 256))
    orc.set_threads(all_threads)
    return {"value": round(v, 3), "unit": "tokens/s", "cores": all_threads,
            "kind": "oracle",
            "sample": (f"{all_threads} threads: router, top-k and route map for all {cfg.T} tokens "
                       f"({t_route:.2f} s); expert FFN "
                       + (f"for all {n} tokens ({t_ffn:.2f} s): the whole layer" if n == cfg.T else
                          f"for {n} sampled tokens ({t_ffn:.2f} s), extrapolated to T={cfg.T}")),
            "one_core": {"value": round(v1, 3), "unit": "tokens/s", "cores": 1,
                         "sample": (f"router, top-k and route map for {min(cfg.T, 256)} tokens and the expert FFN "
                                    f"for {n1} of them ({t_ffn1:.2f} s), extrapolated to T={cfg.T}")}}


def run_paged(args, cfg):
    """The expert-virtualised layer: experts live in pinned host memory and
    stream into P arena slots (groups of G experts into 2 banks) on a copy
    stream while the compute stream runs each loaded group; the first banks
    fill before routing is known. Reports the layer throughput, the
    host-to-device rate, the experts and groups left out for having no routes,
    the bubble rate 1 - max(T_io, T_exec) / T_total (T_io: busy time of the
    copies, T_exec: busy time of the compute kernels, T_total: the layer's
    wall time on the compute stream), and the max-plus model's prediction of
    T_total from the measured service times."""
    import numpy as np
    import torch

    from routed_expert_ffn_top_amd import binding as B
    from routed_expert_ffn_top_amd.inputs import make_inputs
    from routed_expert_ffn_top_amd.layer import MoELayer
    from routed_expert_ffn_top_amd.pipeline_model import predict, schedule

    if getattr(args, "group_size", None):
        cfg = cfg.with_(G=args.group_size)
    inp = make_inputs(cfg, device="cuda", residual=False)
    layer = MoELayer(inp, paged=True)
    Y = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    for _ in range(args.warmup):
        layer.forward(Y, compute=compute, copy=copy)
    torch.cuda.synchronize()
    counts = np.bincount(layer.routes["topk_idx"].cpu().numpy().ravel(), minlength=cfg.n_exp)
    G, nb = cfg.G, cfg.P // cfg.G
    ng = (cfg.n_exp + G - 1) // G
    routed = [int(counts[g * G:(g + 1) * G].sum()) for g in range(ng)]
    loads = schedule(routed, nb, prefetch=True)
    experts_copied = sum((G if ld["early"] else int((counts[ld["group"] * G:(ld["group"] + 1) * G] > 0).sum()))
                         for ld in loads)
    n_exec = sum(1 for r in routed if r > 0)
    expert_bytes = expert_slice_bytes(cfg)
    K = args.steps
    kernels = ["router", "topk", "route_count", "route_place", "gate_up", "down", "combine"]
    cap = K * (n_exec + len(loads) + 2)
    for nme in kernels + ["h2d"]:
        B.moe_profile_begin(nme, cap)
    t_total = []
    for _ in range(K):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(compute)
        layer.forward(Y, compute=compute, copy=copy)
        b.record(compute)
        b.synchronize()
        t_total.append(a.elapsed_time(b))
    torch.cuda.synchronize()
    rec = {nme: B.moe_profile_end(nme, cap) for nme in kernels + ["h2d"]}
    T_total = sum(t_total) / K
    T_io = sum(rec["h2d"]) / K
    T_exec = sum(sum(rec[n]) for n in kernels) / K
    # per-step service times, averaged over the steps: loads in loading order,
    # executions (route count + place + gate/up + down) in group order
    nl = len(loads)
    L = [float(np.mean(rec["h2d"][i::nl])) for i in range(nl)]
    cnt = np.array(rec["route_count"]).reshape(K, n_exec + 1)
    X = [float(np.mean(cnt[:, 1 + k]) + np.mean(rec["route_place"][k::n_exec]) +
               np.mean(rec["gate_up"][k::n_exec]) + np.mean(rec["down"][k::n_exec])) for k in range(n_exec)]
    T_ne = float(np.mean(rec["router"]) + np.mean(rec["topk"]) + np.mean(cnt[:, 0]))
    T_tail = float(np.mean(rec["combine"]))
    model = predict(routed, L, X, B=nb, q=1, T_ne=T_ne, T_route=T_ne, T_tail=T_tail, prefetch=True)
    h2d_bytes = experts_copied * expert_bytes
    gbs = h2d_bytes / (T_io / 1e3) / 1e9 if T_io > 0 else None
    out = {
        "metric": "routed tokens/s per MoE layer, experts paged from host memory (1 GPU)",
        "value": round(cfg.T / (T_total / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(T_total, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, Zipf(1.1) logit bias)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "k": cfg.k, "f": cfg.f, "slots": cfg.P, "G": G, "banks": nb},
        "paging": {
            "experts_with_routes": int((counts > 0).sum()),
            "zero_route_experts": int(cfg.n_exp - (counts > 0).sum()),
            "groups_loaded": len(loads),
            "groups_executed": n_exec,
            "groups_skipped": ng - n_exec,
            "experts_copied": experts_copied,
            "h2d_bytes_per_step": h2d_bytes,
            "t_io_ms": round(T_io, 4),
            "t_exec_ms": round(T_exec, 4),
            "t_total_ms": round(T_total, 4),
            "bubble_rate": round(1.0 - max(T_io, T_exec) / T_total, 4),
            "maxplus_t_pipe_ms": round(model["t_pipe"], 4),
            "maxplus_error": round(model["t_pipe"] / T_total - 1.0, 4),
            "kernel_ms_per_step": {n: round(sum(v) / K, 4) for n, v in rec.items() if n != "h2d"},
        },
        "roofline": {
            "kernel": "host-to-device expert copies (pinned host memory to the arena)",
            "bound": "host-link",
            "achieved": round(gbs, 2) if gbs else None,
            "peak": PCIE_GEN5_X16_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PCIE_GEN5_X16_GBS, 4) if gbs else None,
            "traffic": h2d_bytes,
        },
    }
    profile = {"routed": routed, "group_size": [min(G, cfg.n_exp - g * G) for g in range(ng)],
               "routed_experts": [int((counts[g * G:(g + 1) * G] > 0).sum()) for g in range(ng)],
               "l_expert": T_io / experts_copied, "X": X, "T_ne": T_ne, "T_tail": T_tail}
    layer.close()
    return out, profile


def bench_paged(args, cfg) -> int:
    out, _ = run_paged(args, cfg)
    print(json.dumps(out), flush=True)
    return 0


def bench_configure(args, cfg, sizes=(1, 2, 4, 8, 16)) -> int:
    """The configuration step of the pages (section 3.4) on this GPU: one
    profiled run of the paged layer per group size g (with B = P/g banks),
    then the max-plus model evaluates every feasible bank count per g under
    the arena's slot budget P and picks (G*, B*). Prints the measured layer
    time of each profiled run next to its prediction, and the choice."""
    from routed_expert_ffn_top_amd.pipeline_model import configure, predict_from_profile

    profiles, measured = {}, {}
    for g in sizes:
        if cfg.P % g:
            continue
        args.group_size = g
        out, prof = run_paged(args, cfg)
        profiles[g] = prof
        measured[g] = out["paging"]["t_total_ms"]
        print(f"profiled G={g}: {measured[g]:.3f} ms", file=sys.stderr, flush=True)
    res = configure(profiles, cfg.P)
    rows = [{"G": g, "B": cfg.P // g, "measured_ms": round(measured[g], 4),
             "predicted_ms": round(predict_from_profile(profiles[g], cfg.P // g)["t_pipe"], 4)}
            for g in sorted(profiles)]
    print(json.dumps({
        "metric": "paged layer configuration (max-plus model over profiled group sizes)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": cfg.T, "slots": cfg.P},
        "profiled_runs": rows,
        "chosen": {"G": res["G"], "B": res["B"], "predicted_ms": round(res["t_pipe"], 4),
                   "measured_ms_at_G": round(measured[res["G"]], 4)},
        "predicted_ms_by_G_B": {f"{g}x{b}": round(t, 4) for (g, b), t in sorted(res["table"].items())},
    }), flush=True)
    return 0


def bench_fused(args, cfg) -> int:
    """The fused expert tile (MOE_FFN_FUSED: gate/up, SwiGLU and down in one
    kernel, H kept in LDS) against the two projection kernels on the same
    layer: each path runs router, route build, expert FFN and combine as
    separate calls; per-kernel HIP events and whole-step times over K steps
    after a time-based warm-up."""
    import numpy as np
    import torch

    from routed_expert_ffn_top_amd import binding as B
    from routed_expert_ffn_top_amd.inputs import make_inputs
    from routed_expert_ffn_top_amd.layer import MoELayer

    inp = make_inputs(cfg, device="cuda", residual=False)
    layer = MoELayer(inp)
    s = layer.shape
    Y = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")

    def step(fused):
        B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
        B.moe_route_build(s, 0, s.T, L, layer.phi, 0, layer.routes, layer.ws)
        fl = B.MOE_FFN_EXPERTS | B.MOE_FFN_FINALIZE | (B.MOE_FFN_FUSED if fused else 0)
        B.moe_expert_ffn(s, layer.X, Y, layer.routes, layer.arena, layer.phi, fl, layer.ws)

    K = args.steps
    res = {}
    for fused in (False, True):
        w0 = time.perf_counter()
        n = 0
        while n < args.warmup or time.perf_counter() - w0 < args.warmup_min_s:
            step(fused)
            n += 1
            if n % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            step(fused)
        b.record()
        torch.cuda.synchronize()
        names = ["fused"] if fused else ["gate_up", "down"]
        for nme in names + ["combine"]:
            B.moe_profile_begin(nme, K)
        for _ in range(K):
            step(fused)
        torch.cuda.synchronize()
        kern = {nme: round(float(np.mean(B.moe_profile_end(nme, K))), 4) for nme in names + ["combine"]}
        res["fused" if fused else "split"] = {"step_ms": round(a.elapsed_time(b) / K, 4), "kernel_ms": kern}
    R = cfg.T * cfg.kp
    flops = 6.0 * R * cfg.d * cfg.f
    sp = res["split"]["kernel_ms"]
    ffn_split = sp["gate_up"] + sp["down"]
    ffn_fused = res["fused"]["kernel_ms"]["fused"]
    out = {
        "metric": "expert FFN time: fused expert tile vs the two projection kernels (1 GPU)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "f": cfg.f},
        "steps": K,
        "split": res["split"],
        "fused": res["fused"],
        "expert_ffn_ms": {"split": round(ffn_split, 4), "fused": round(ffn_fused, 4)},
        "expert_ffn_tflops": {"split": round(flops / (ffn_split / 1e3) / 1e12, 1),
                              "fused": round(flops / (ffn_fused / 1e3) / 1e12, 1)},
        "fused_over_split": round(ffn_fused / ffn_split, 3),
    }
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


def bench_rows_curve(args, cfg, counts=(1, 8, 16, 32, 64, 128, 256, 384, 512, 768, 1024, 2048, 4096, 8192)) -> int:
    """Expert-projection time against the number of routes one expert
    receives (the pages' characterisation of expert latency by route count):
    every token of a T-token prompt is routed to the same expert (top-1), so
    one slot holds T records, and the gate/up and down kernels are timed on
    it with HIP events. One line per route count."""
    import numpy as np
    import torch

    from routed_expert_ffn_top_amd import binding as B
    from routed_expert_ffn_top_amd.inputs import make_inputs
    from routed_expert_ffn_top_amd.layer import MoELayer

    base = cfg.with_(T=max(counts), k=1)
    inp = make_inputs(base, device="cuda", residual=False)
    layer = MoELayer(inp)
    K = args.steps
    rows = []
    for R in counts:
        s = B.make_shape(R, cfg.d, cfg.f, cfg.E, 1, cfg.n_shared, P=layer.shape.P, dtype=cfg.dtype,
                         renorm=cfg.renorm)
        routes, ws = B.alloc_routes(s), B.alloc_workspace(s)
        L = torch.zeros((R, cfg.E), dtype=torch.float32, device="cuda")
        L[:, 0] = 1.0   # every token picks expert 0
        X = layer.X[:R]
        B.moe_route_build(s, 0, R, L, layer.phi, 0, routes, ws)
        for _ in range(max(args.warmup, 20)):
            B.moe_expert_ffn(s, X, None, routes, layer.arena, layer.phi, B.MOE_FFN_EXPERTS, ws)
        torch.cuda.synchronize()
        for nme in ("gate_up", "down"):
            B.moe_profile_begin(nme, K)
        for _ in range(K):
            B.moe_expert_ffn(s, X, None, routes, layer.arena, layer.phi, B.MOE_FFN_EXPERTS, ws)
        torch.cuda.synchronize()
        gu = float(np.mean(B.moe_profile_end("gate_up", K)))
        dn = float(np.mean(B.moe_profile_end("down", K)))
        us = (gu + dn) * 1e3
        fl = 6.0 * R * cfg.d * cfg.f
        rows.append({"routes": R, "gate_up_us": round(gu * 1e3, 2), "down_us": round(dn * 1e3, 2),
                     "expert_us": round(us, 2), "us_per_route": round(us / R, 4),
                     "tflops": round(fl / (us * 1e-6) / 1e12, 1),
                     "weight_gbs": round(3 * cfg.d * cfg.f * 2 / (us * 1e-6) / 1e9, 1)})
        print(json.dumps({"routes": R, **rows[-1]}), file=sys.stderr, flush=True)
        del routes, ws
    print(json.dumps({"metric": "expert projection time against the routes of one expert (1 GPU)",
                      "config": {"workload": f"one expert of the {cfg.name} layer (d={cfg.d}, f={cfg.f}), bf16",
                                 "steps": K},
                      "curve": rows}), flush=True)
    layer.close()
    return 0


def bench_ep_share(args, cfg, n: int) -> int:
    """One GPU's share of the layer under n-way expert parallelism, run on
    this GPU at its real shape. The whole prompt is routed (router, top-k) as
    on every GPU; the route map and the expert FFN then see a placement map
    that holds only this share's routed experts (E/n consecutive ids) and
    leaves the rest absent, so the kernels work on exactly the records the
    share owns. Shared experts, replicated on every GPU, are run token
    parallel: each GPU runs them for its own T/n tokens (a second route build
    over that token range with a map that holds only the shared experts).
    The exchange of rows between GPUs and the combine of the returned rows
    are not run. Each share is timed in turn; the slowest bounds the layer."""
    import numpy as np
    import torch

    from routed_expert_ffn_top_amd import binding as B
    from routed_expert_ffn_top_amd.inputs import make_inputs
    from routed_expert_ffn_top_amd.layer import MoELayer

    if cfg.E % n or cfg.T % n:
        raise SystemExit(f"--ep-share {n}: {cfg.E} experts or {cfg.T} tokens do not split evenly")
    inp = make_inputs(cfg, device="cuda", residual=False)
    layer = MoELayer(inp)
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    K = args.steps
    per, tpg = cfg.E // n, cfg.T // n
    ws2 = B.alloc_workspace(s) if cfg.n_shared else None
    routes2 = B.alloc_routes(s) if cfg.n_shared else None

    def tiles_of(counts):
        return int(sum(-(-int(c) // 256) for c in counts)) * (-(-2 * cfg.f // 256))

    shares = []
    for r in range(n):
        phi = [slot if r * per <= e < (r + 1) * per else -1 for e, slot in enumerate(layer.phi)]
        B.moe_route_build(s, 0, s.T, L, phi, 0, layer.routes, layer.ws)
        calls = [(phi, layer.routes, layer.ws)]
        if cfg.n_shared:
            phi_s = [slot if e >= cfg.E else -1 for e, slot in enumerate(layer.phi)]
            B.moe_route_build(s, r * tpg, tpg, L, phi_s, 0, routes2, ws2)
            calls.append((phi_s, routes2, ws2))

        def ffn():
            for ph, rt, w in calls:
                B.moe_expert_ffn(s, layer.X, None, rt, layer.arena, ph, B.MOE_FFN_EXPERTS, w)

        w0, m = time.perf_counter(), 0
        while m < args.warmup or time.perf_counter() - w0 < args.warmup_min_s:
            ffn()
            m += 1
            if m % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        for nme in ("gate_up", "down"):
            B.moe_profile_begin(nme, K * len(calls))
        for _ in range(K):
            ffn()
        torch.cuda.synchronize()
        gu = float(np.sum(B.moe_profile_end("gate_up", K * len(calls)))) / K
        dn = float(np.sum(B.moe_profile_end("down", K * len(calls)))) / K
        R = sum(int(rt["slot_count"].cpu().numpy().sum()) for _, rt, _ in calls)
        fl = 6.0 * R * cfg.d * cfg.f
        shares.append({"share": r, "routes": R, "gate_up_tiles": sum(tiles_of(rt["slot_count"].cpu().numpy())
                                                                     for _, rt, _ in calls),
                       "gate_up_ms": round(gu, 4), "down_ms": round(dn, 4), "expert_ffn_ms": round(gu + dn, 4),
                       "tflops": round(fl / ((gu + dn) * 1e-3) / 1e12, 1)})
        print(json.dumps(shares[-1]), file=sys.stderr, flush=True)
    worst = max(shares, key=lambda x: x["expert_ffn_ms"])
    out = {"metric": f"expert FFN of one GPU's share under {n}-way expert parallelism, run on 1 GPU",
           "config": {"workload": WORKLOAD_TEXT[args.workload], "experts_per_share": per,
                      "shared_experts": f"{cfg.n_shared}, run for each share's {tpg} tokens" if cfg.n_shared else 0,
                      "steps": K},
           "shares": shares,
           "slowest_share": worst["share"],
           "slowest_share_ms": worst["expert_ffn_ms"],
           "slowest_share_tflops": worst["tflops"],
           "routes_total": sum(x["routes"] for x in shares),
           "not_run": "the all-to-all exchange of X rows and Yr rows, the combine"}
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


def bench_stack(args, cfg, n_layers: int = 32) -> int:
    """A stack of n_layers MoE layers with independent weights (each layer's
    own seeded X, router and experts), all resident in HBM; one step runs the
    layers back to back on one stream. Reports the stack time and the
    per-layer average."""
    import torch

    from routed_expert_ffn_top_amd.inputs import make_inputs
    from routed_expert_ffn_top_amd.layer import MoELayer

    layers, outs = [], []
    for l in range(n_layers):
        inp = make_inputs(cfg, layer=l, device="cuda", residual=False)
        layers.append(MoELayer(inp))
        outs.append(torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda"))
        del inp
        torch.cuda.empty_cache()
        print(f"built layer {l + 1}/{n_layers}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for lay, Y in zip(layers, outs):
            lay.forward(Y)
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        for lay, Y in zip(layers, outs):
            lay.forward(Y)
    b.record()
    torch.cuda.synchronize()
    stack_ms = a.elapsed_time(b) / K
    R = cfg.T * cfg.kp
    flops = 6.0 * R * cfg.d * cfg.f * n_layers
    out = {
        "metric": f"routed tokens/s through {n_layers} MoE layers (1 GPU)",
        "value": round(cfg.T / (stack_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(stack_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights per layer)",
        "config": {"workload": WORKLOAD_TEXT[f"mixtral_stack_t{cfg.T}"], "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "k": cfg.k, "f": cfg.f, "layers": n_layers},
        "per_layer_ms": round(stack_ms / n_layers, 4),
        "stack_ms": round(stack_ms, 3),
        "pct_bf16_peak": round(100.0 * flops / (stack_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "resident_expert_gb": round(n_layers * cfg.n_exp * expert_slice_bytes(cfg) / 1e9, 1),
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-min-s", type=float, default=1.0,
                    help="keep warming up until this many seconds have passed (steady clocks)")
    ap.add_argument("--rows-curve", action="store_true",
                    help="time one expert's projections against the number of routes it receives")
    ap.add_argument("--fused", action="store_true",
                    help="time the fused expert tile against the two projection kernels")
    ap.add_argument("--ep-share", type=int, default=0, metavar="N",
                    help="time each GPU's share of the expert FFN under N-way expert parallelism, on this GPU")
    ap.add_argument("--cold", action="store_true",
                    help="also time layers with a 512 MB scratch write before each (cold caches)")
    ap.add_argument("--workload", default="olmoe_t4096", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--group-size", type=int, default=None, help="paged workloads: experts per group")
    ap.add_argument("--configure", action="store_true",
                    help="paged workloads: profile every group size and pick (G, B) with the max-plus model")
    ap.add_argument("--no-context", action="store_true", help="skip the torch.matmul ceiling")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "OUT_MD"))
    ap.add_argument("--summarize-pmc", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV", "CALIB_WRITE_CSV", "OUT"))
    ap.add_argument("--summarize-kernels", nargs=7,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV", "CALIB_WRITE_CSV", "MFMA_CSV",
                             "STATS_CSV", "OUT"))
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats, args.command)
        return 0
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.command)
        return 0
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels, args.command, args.workload)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU (one MI355X); "
                                   f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported"}))
        return 2

    import numpy as np
    import torch

    from routed_expert_ffn_top_amd import binding as B
    from routed_expert_ffn_top_amd.inputs import CONFIGS, make_inputs
    from routed_expert_ffn_top_amd.layer import MoELayer

    torch.cuda.set_device(0)
    if args.copy_calibration:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))
        return 0

    B.load()
    if args.workload.startswith("virt_"):
        if args.configure:
            return bench_configure(args, CONFIGS[args.workload])
        return bench_paged(args, CONFIGS[args.workload])
    if args.workload.startswith("mixtral_stack_"):
        return bench_stack(args, CONFIGS[args.workload.replace("mixtral_stack_", "mixtral_")])
    if args.fused:
        return bench_fused(args, CONFIGS[args.workload])
    if args.rows_curve:
        return bench_rows_curve(args, CONFIGS[args.workload])
    if args.ep_share:
        return bench_ep_share(args, CONFIGS[args.workload], args.ep_share)
    cfg = CONFIGS[args.workload]
    inp = make_inputs(cfg, device="cuda", residual=False)
    layer = MoELayer(inp)
    Y = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # 1. warm-up: W steps, and at least warmup_min_s seconds; the first 20
    # steps are timed one by one (the clock ramp)
    ramp = [ev() for _ in range(21)]
    w_steps, w0 = 0, time.perf_counter()
    while w_steps < args.warmup or time.perf_counter() - w0 < args.warmup_min_s:
        if w_steps < 21:
            ramp[w_steps].record()
        layer.forward(Y)
        w_steps += 1
        if w_steps == 20:
            ramp[20].record()
        if w_steps % 20 == 0:
            torch.cuda.synchronize()   # ties the wall-clock minimum to GPU time
    if w_steps < 20:
        ramp[w_steps].record()   # the end of the last of fewer than 20 warm-up steps
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - w0
    ramp_ms = [ramp[i].elapsed_time(ramp[i + 1]) for i in range(min(w_steps, 20))]

    # 2. the timed region: K whole layers between two events
    K = args.steps
    start, stop = ev(), ev()
    w1 = time.perf_counter()
    start.record()
    for _ in range(K):
        layer.forward(Y)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w1
    ms = start.elapsed_time(stop) / K

    # 3. per-step times: a second pass, one event between consecutive layers
    marks = [ev() for _ in range(K + 1)]
    marks[0].record()
    for i in range(K):
        layer.forward(Y)
        marks[i + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(K)])

    # 4. gate/up launch times: a third pass, each launch bracketed on its stream
    B.moe_profile_begin("gate_up", K)
    for _ in range(K):
        layer.forward(Y)
    torch.cuda.synchronize()
    gate_up_ms = B.moe_profile_end("gate_up", K)

    # 5. per-kernel breakdown: every kernel bracketed
    names = ["router", "topk", "route_count", "route_place", "gate_up", "down", "combine"]
    reps = min(K, 10)
    for nme in names:
        B.moe_profile_begin(nme, reps)
    for _ in range(reps):
        layer.forward(Y)
    torch.cuda.synchronize()
    breakdown = {}
    for nme in names:
        d = B.moe_profile_end(nme, reps)
        breakdown[nme] = round(sum(d) / len(d), 4) if d else None

    cold = None
    if args.cold or working_set_bytes(cfg) < MALL_BYTES:
        cold = cold_cache_steps(torch, layer, Y, K)

    R = cfg.T * cfg.kp
    flops_layer = 6.0 * R * cfg.d * cfg.f
    gate_up_flops = 4.0 * R * cfg.d * cfg.f
    down_flops = 2.0 * R * cfg.d * cfg.f
    gu_avg = sum(gate_up_ms) / len(gate_up_ms)
    achieved = gate_up_flops / (gu_avg / 1e3) / 1e12
    traffic = read_traffic(args.workload, gate_up_flops)
    tokens_s = cfg.T / (ms / 1e3)
    ffn_ms = (breakdown["gate_up"] or 0) + (breakdown["down"] or 0)

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; random-init, no checkpoint)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "k": cfg.k, "n_shared": cfg.n_shared, "f": cfg.f, "slots": layer.shape.P,
                   "router": "fp32 logits computed in the step", "parallelism": "single GPU"},
        "routes_per_s": round(R / (ms / 1e3), 1),
        "pct_bf16_peak_layer": round(100.0 * flops_layer / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "expert_ffn_tflops": round(flops_layer / (ffn_ms / 1e3) / 1e12, 1) if ffn_ms else None,
        "pct_bf16_peak_expert_ffn": round(100.0 * flops_layer / (ffn_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2)
        if ffn_ms else None,
        "kernel_ms": breakdown,
        "down_tflops": round(down_flops / (breakdown["down"] / 1e3) / 1e12, 1) if breakdown["down"] else None,
        "wall_s_timed": round(wall, 4),
        "warmup_steps_run": w_steps,
        "warmup_s": round(warm_s, 3),
        "clock_ramp_ms": {"first_warmup_step": round(ramp_ms[0], 4) if ramp_ms else None,
                          "warmup_steps_1_to_20_mean": round(float(np.mean(ramp_ms)), 4) if ramp_ms else None,
                          "timed_mean": round(ms, 4)},
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4),
                    "first": round(float(step_ms[0]), 4), "last": round(float(step_ms[-1]), 4),
                    "pass": f"second pass of {K} layers, one event between consecutive layers"},
        "roofline": {
            "kernel": "gate_up (gathered X rows x packed gate/up slice, bf16 MFMA, SwiGLU epilogue)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "launch_ms_avg": round(gu_avg, 4),
            "launch_timing": f"third pass of {K} layers after the timed region, each gate/up launch "
                             "bracketed by HIP events on its own stream",
            "flops_per_launch": gate_up_flops,
        },
    }
    if cold is not None:
        out["cold_cache"] = cold
    if not args.no_context:
        out["context"] = {"torch_matmul_bf16_8192_tflops": round(torch_matmul_ceiling(torch), 1),
                          **torch_bmm_expert_shape(torch, cfg)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
