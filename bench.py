#!/usr/bin/env python3
"""Benchmark of the DeepSeekMoE feed-forward layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_bf16] [--no-extra]

A step is one training-step pass of the whole layer over one batch of synthetic
input already resident in HBM: route -> permute -> [FP8 quantization of u] ->
routed grouped FFN -> shared FFN -> combine -> bias update. The headline
workload is the decode-shaped layer at the DeepSeek-V3 shape (T=128 tokens,
H=7168, 256 routed experts top-8 + 1 shared, I=2048, bf16), the configuration
the tokens/s metric is quoted on; the other workloads are reported under
"extra" with their tokens/s and MFMA / HBM fractions.

Prints ONE JSON line (rank 0). Per-kernel durations come from HIP events that
the library records on its stream inside the timed region
(moe_grouped_ffn_profiled); the "roofline" object is for the dominant kernel,
the routed gate/up GEMM. "cpu_baseline" times the float64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at H7168/256e/top-8 (prefill %MFMA peak, decode %HBM)"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def binding_roof(flops, nbytes, ms, dtype="bf16"):
    """The binding roof of a piece of work: the larger of its MFMA-time floor (flops at the dtype's
    dense peak) and its HBM-time floor (algorithmic bytes at 8 TB/s), and the fraction of it that
    `ms` reaches."""
    t_mfma = flops / (PEAK_TFLOPS[dtype] * 1e12) * 1e3
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
    roof = max(t_mfma, t_hbm)
    return {"binding_roof": "mfma" if t_mfma > t_hbm else "hbm", "roof_ms": roof,
            "frac_of_binding_roof": roof / ms if ms > 0 else None}


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (a comment edit leaves the counters valid)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("ffn.hip", "kloop.h", "common.h", "fp8.h", "lds.h", "tiles.h"):
        with open(os.path.join(ROOT, "sparse_moe_transformer_02_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != _kernel_source_hash():
        return None
    return ent["hbm_bytes_per_launch"]


def _work(cfg, counts):
    """Algorithmic FLOPs and HBM bytes of one layer forward, and of the routed gate/up GEMM."""
    import numpy as np
    T, H, I, K, N_r = cfg.T, cfg.H, cfg.I, cfg.K, cfg.N_r
    wbytes = 1 if cfg.dtype == "fp8" else (4 if cfg.dtype == "f32" else 2)
    abytes = 4 if cfg.dtype == "f32" else 2
    n_sel = int(np.count_nonzero(counts))
    flops = 2 * 3 * H * I * (T * K + T) + 2 * T * H * N_r
    expert_w = 3 * I * H * wbytes
    scales = (3 * (I // 128) * (H // 128) * 4) if cfg.dtype == "fp8" else 0
    layer_bytes = (n_sel + 1) * (expert_w + scales) + N_r * H * 4 + 2 * T * H * abytes
    # gate/up GEMM over the shared and the selected routed experts: W_g and W_u of each, the
    # token rows once, and h written once per (token, expert) row (FP8: E4M3 codes and one fp32
    # scale per 1x128 tile)
    hbytes = {"fp8": 1 + 4 / 128, "f32": 4}.get(cfg.dtype, 2)
    gemm1_bytes = (n_sel + 1) * (2 * I * H * wbytes + (2 * scales // 3)) \
        + T * H * (1 if cfg.dtype == "fp8" else abytes) + T * (K + 1) * I * hbytes
    gemm1_flops = 2 * 2 * H * I * T * (K + 1)
    return {"flops": flops, "bytes": layer_bytes, "n_selected": n_sel, "gemm1_bytes": gemm1_bytes,
            "gemm1_flops": gemm1_flops}


def run_workload(name, steps, warmup, measure_kernels=True, cfg=None):
    import numpy as np
    import torch
    import workloads as W
    from sparse_moe_transformer_02_amd.layer import MoeLayer

    cfg = cfg or W.config(name)
    inp = W.make_inputs(cfg, device="cuda")
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma)
    u = inp["u"]
    for _ in range(warmup):
        layer.step(u)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in ev:                       # torch creates the HIP event on first record(); the library
        for x in e:                    # records these handles itself, so create them up front
            x.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        if measure_kernels:
            layer.step(u, ffn_events=ev[i], marks=marks[i])
        else:
            layer.step(u)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = start.elapsed_time(end) / steps
    out = {"cfg": cfg, "ms": ms, "wall_ms": wall_ms}
    if measure_kernels:
        out["gemm1_ms"] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        out["gemm2_ms"] = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
        if cfg.dtype == "fp8":
            out["h_quant_ms"] = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        names = ["route", "permute", "quant_u", "expert_ffn", "combine"]
        stage = {}
        for j, n in enumerate(names):
            stage[n] = float(np.mean([m[j].elapsed_time(m[j + 1]) for m in marks]))
        out["stage_ms"] = stage
    counts = layer.last["counts"].cpu().numpy()
    out["work"] = _work(cfg, counts)
    out["max_over_mean_load"] = float(counts.max() / (cfg.T * cfg.K / cfg.N_r))
    out["layer"], out["inp"] = layer, inp
    return out


def imbalance_trajectory(steps=100, warmup=2):
    """The load-imbalance workload as configured: `steps` forward + bias-update steps at T = 16384
    with experts 0-7 hot, a fresh u every step (drawn on the GPU before the step's timed span) and
    the bias carried from step to step from zero. Each step is timed with HIP events around
    layer.step(); its per-expert counts are copied aside after the step (outside the span), so the
    max/mean load of every step is reported. Warm-up runs forwards only (no bias update)."""
    import numpy as np
    import torch
    import workloads as W
    from sparse_moe_transformer_02_amd.layer import MoeLayer

    cfg = W.config("imbalance_bf16")
    inp = W.make_inputs(cfg, device="cuda")
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma)
    for _ in range(warmup):
        layer.forward(inp["u"])
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    span = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in ev:
        for x in e:
            x.record()
    counts = torch.empty((steps, cfg.N_r), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for i in range(steps):
        u = W.make_tokens(cfg, i, device="cuda")
        span[i][0].record()
        layer.step(u, ffn_events=ev[i], marks=marks[i])
        span[i][1].record()
        counts[i].copy_(layer.last["counts"])
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in span])
    c = counts.cpu().numpy()
    mean_load = cfg.T * cfg.K / cfg.N_r
    res = {"cfg": cfg, "ms": float(ms.mean()), "wall_ms": float(ms.mean()),
           "gemm1_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
           "gemm2_ms": float(np.mean([e[2].elapsed_time(e[3]) for e in ev])),
           "stage_ms": {n: float(np.mean([m[j].elapsed_time(m[j + 1]) for m in marks]))
                        for j, n in enumerate(["route", "permute", "quant_u", "expert_ffn", "combine"])},
           "work": _work(cfg, c[-1]), "max_over_mean_load": float(c[0].max() / mean_load)}
    s = _summary(res)
    s.update({"steps": steps, "fresh_u_per_step": True, "ms_per_step_median": float(np.median(ms)),
              "ms_per_step_min": float(ms.min()), "ms_per_step_max": float(ms.max()),
              "ms_first_step": float(ms[0]), "ms_last_step": float(ms[-1]),
              "max_over_mean_load": [float(x) for x in c.max(axis=1) / mean_load],
              "hot_bias_after": float(layer.bias[: cfg.hot_experts].mean().item())})
    del layer, inp, counts
    torch.cuda.empty_cache()
    return s


def t_sweep(Ts=(1024, 2048, 4096, 8192, 16384, 32768)):
    """The bf16 layer at the prefill shape (uniform routing) over token counts: ms per step,
    fractions of the bf16 MFMA and HBM peaks, and the fraction of the binding roof (the larger of
    the MFMA-time and HBM-time floors of the layer's algorithmic work). The binding roof moves
    from HBM to the MFMAs where the arithmetic intensity reaches the ridge, near T = 8.9k."""
    import torch
    import workloads as W
    out = {}
    for T in Ts:
        cfg = W.config("prefill_bf16").scaled(name=f"prefill_bf16_T{T}", T=T)
        r = run_workload(cfg.name, max(3, min(10, 40960 // T)), 2, cfg=cfg)
        s = _summary(r)
        w = r["work"]
        t_mfma = w["flops"] / (PEAK_TFLOPS["bf16"] * 1e12) * 1e3
        t_hbm = w["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
        out[f"T={T}"] = {"ms_per_step": s["ms_per_step"], "tokens_per_s": s["tokens_per_s"],
                         "gemm1_ms": s["gemm1_ms"], "gemm2_ms": s["gemm2_ms"],
                         "frac_mfma_peak": s["frac_mfma_peak"], "frac_hbm_peak": s["frac_hbm_peak"],
                         "binding_roof": "mfma" if t_mfma > t_hbm else "hbm",
                         "frac_of_binding_roof": max(t_mfma, t_hbm) / s["ms_per_step"]}
        del r
        torch.cuda.empty_cache()
    return out


def graph_timing(name="decode_bf16", steps=20, warmup=5):
    """The same layer training step captured once in a HIP graph (torch.cuda.graph) and replayed:
    the kernels are the same; the replay drops the per-launch host work and gaps."""
    import torch
    import workloads as W
    from sparse_moe_transformer_02_amd.layer import MoeLayer
    cfg = W.config(name)
    inp = W.make_inputs(cfg, device="cuda")
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma)
    u = inp["u"]
    layer.step(u)                        # per-T buffers are allocated outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step(u)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    w = _work(cfg, layer.last["counts"].cpu().numpy())
    del graph, layer, inp
    torch.cuda.empty_cache()
    return {"workload": name, "steps": steps, "ms_per_step": ms, "tokens_per_s": cfg.T / ms * 1e3,
            **binding_roof(w["flops"], w["bytes"], ms, "fp8" if cfg.dtype == "fp8" else "bf16")}


def ep_shard_timing(reps=10, n_experts=32, rows_per_expert=1024):
    """The grouped FFN alone on one GPU's share of an expert-parallel layer: 32 of the 256 experts
    (an 8-GPU node) with ~1024 rows each (4096 tokens per GPU, top-8), H = 7168, I = 2048, bf16, the
    received rows contiguous. No routing or exchange (those need several GPUs); the rows are seeded
    random, the group sizes drawn around the mean."""
    import numpy as np
    import torch
    import sparse_moe_transformer_02_amd as moe
    H, I, G = 7168, 2048, n_experts
    g = torch.Generator(device="cuda").manual_seed(8)
    counts = np.random.default_rng(8).poisson(rows_per_expert, G)
    rows = int(counts.sum())
    X = torch.randn((rows, H), generator=g, device="cuda").bfloat16()
    Wg = (torch.randn((G, I, H), generator=g, device="cuda") / H ** 0.5).bfloat16()
    Wu = (torch.randn((G, I, H), generator=g, device="cuda") / H ** 0.5).bfloat16()
    Wd = (torch.randn((G, H, I), generator=g, device="cuda") / I ** 0.5).bfloat16()
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda")
    Y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_grouped_ffn_workspace_size(G, rows, H, I, moe.BF16), dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for x in ev:                       # create the HIP events (the library records these handles)
        x.record()
    torch.cuda.synchronize()
    g1 = g2 = 0.0
    for it in range(reps + 2):
        moe.moe_grouped_ffn(off, rows, X, Wg, Wu, Wd, Y=Y, workspace=ws, events=ev)
        torch.cuda.synchronize()
        if it >= 2:
            g1 += ev[0].elapsed_time(ev[1]) / reps
            g2 += ev[2].elapsed_time(ev[3]) / reps
    ms = g1 + g2
    flops = 2 * 3 * H * I * rows
    wbytes = 3 * G * H * I * 2 + 2 * rows * H * 2 + 2 * rows * I * 2
    t_mfma = flops / (PEAK_TFLOPS["bf16"] * 1e12) * 1e3
    t_hbm = wbytes / (PEAK_HBM_GBS * 1e9) * 1e3
    out = {"experts": G, "rows": rows, "H": H, "I": I, "dtype": "bf16", "gemm1_ms": g1, "gemm2_ms": g2,
           "ffn_ms": ms, "tflops": flops / ms / 1e9, "frac_mfma_peak": t_mfma / ms,
           "binding_roof": "mfma" if t_mfma > t_hbm else "hbm", "frac_of_binding_roof": max(t_mfma, t_hbm) / ms}
    del X, Wg, Wu, Wd, Y, ws
    torch.cuda.empty_cache()
    return out


def ceilings_timing(reps=10):
    """Measured ceilings beside the published peaks: the HBM rates of PyTorch's own kernels on large
    buffers (a sum reads every byte once; a device copy reads and writes every byte), hipBLASLt's bf16
    GEMM rate (torch.matmul run as a library, a sanity ceiling only) at the shared expert's gate/up
    and down shapes of the prefill and imbalanced workloads, and the compute-unit count and engine
    clock that rocminfo reports for the device."""
    import subprocess
    import torch

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")          # 4 GiB
    out["torch_sum_read_gbs"] = x.numel() * 4 / timed(lambda: x.sum()) / 1e6
    del x
    src = torch.ones(1 << 31, dtype=torch.uint8, device="cuda")          # 2 GiB
    dst = torch.empty_like(src)
    out["torch_copy_read_plus_write_gbs"] = 2 * src.numel() / timed(lambda: dst.copy_(src)) / 1e6
    del src, dst
    torch.cuda.empty_cache()
    g = torch.Generator(device="cuda").manual_seed(11)
    gemms = {}
    for label, (M, K, N) in {"gate_up_T4096": (4096, 7168, 4096), "gate_up_T16384": (16384, 7168, 4096),
                             "down_T16384": (16384, 2048, 7168)}.items():
        a = torch.randn((M, K), generator=g, device="cuda").bfloat16()
        b = torch.randn((K, N), generator=g, device="cuda").bfloat16().contiguous()
        ms = timed(lambda: torch.matmul(a, b))
        tf = 2 * M * N * K / ms / 1e9
        gemms[label] = {"M": M, "K": K, "N": N, "ms": ms, "tflops": tf, "frac_bf16_peak": tf / PEAK_TFLOPS["bf16"]}
        del a, b
    out["hipblaslt_bf16_gemm"] = gemms
    torch.cuda.empty_cache()
    # this library's grouped GEMMs on the same plain shapes: one group of M contiguous rows (the
    # shared expert of the prefill and imbalanced workloads), gate/up = M x 7168 x 4096 and down =
    # M x 2048 x 7168, timed by the library's own events around each launch
    import numpy as np
    import sparse_moe_transformer_02_amd as moe
    H, I = 7168, 2048
    Wg = (torch.randn((1, I, H), generator=g, device="cuda") / H ** 0.5).bfloat16()
    Wu = (torch.randn((1, I, H), generator=g, device="cuda") / H ** 0.5).bfloat16()
    Wd = (torch.randn((1, H, I), generator=g, device="cuda") / I ** 0.5).bfloat16()
    own = {}
    for M in (4096, 16384):
        X = torch.randn((M, H), generator=g, device="cuda").bfloat16()
        Y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        off = torch.tensor([0, M], dtype=torch.int32, device="cuda")
        ws = torch.empty(moe.moe_grouped_ffn_workspace_size(1, M, H, I, moe.BF16), dtype=torch.uint8, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for x in ev:
            x.record()
        torch.cuda.synchronize()
        g1 = g2 = 0.0
        for it in range(reps + 2):
            moe.moe_grouped_ffn(off, M, X, Wg, Wu, Wd, Y=Y, workspace=ws, events=ev)
            torch.cuda.synchronize()
            if it >= 2:
                g1 += ev[0].elapsed_time(ev[1]) / reps
                g2 += ev[2].elapsed_time(ev[3]) / reps
        f1, f2 = 2 * M * 2 * I * H, 2 * M * H * I
        own[f"gate_up_T{M}"] = {"M": M, "K": H, "N": 2 * I, "ms": g1, "tflops": f1 / g1 / 1e9,
                                "frac_bf16_peak": f1 / g1 / 1e9 / PEAK_TFLOPS["bf16"]}
        own[f"down_T{M}"] = {"M": M, "K": I, "N": H, "ms": g2, "tflops": f2 / g2 / 1e9,
                             "frac_bf16_peak": f2 / g2 / 1e9 / PEAK_TFLOPS["bf16"]}
        del X, Y, ws
    out["library_grouped_gemm_one_group"] = own
    del Wg, Wu, Wd
    torch.cuda.empty_cache()
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": getattr(props, "gcnArchName", props.name), "compute_units": props.multi_processor_count}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        for block in txt.split("Agent ")[1:]:
            if "gfx950" not in block:
                continue
            for line in block.splitlines():
                key, _, val = line.strip().partition(":")
                if key == "Compute Unit":
                    out["device"]["rocminfo_compute_units"] = int(val.split()[0])
                elif key == "Max Clock Freq. (MHz)":
                    out["device"]["rocminfo_max_clock_mhz"] = int(val.split()[0])
            break
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    return out


def route_timing(reps=20):
    """Router alone (affinity GEMM + selection) at three token counts: plain Top-K and the
    group-limited variant (8 groups of 32 experts, at most 4 per token)."""
    import torch
    import workloads as W
    import sparse_moe_transformer_02_amd as moe
    out = {}
    for name in ("decode_bf16", "prefill_bf16", "imbalance_bf16"):
        cfg = W.config(name)
        inp = W.make_inputs(cfg, device="cuda", with_weights=False)
        u, E, b = inp["u"], inp["centroids"], inp["bias"]
        T = u.shape[0]
        idx = torch.empty((T, cfg.K), dtype=torch.int32, device="cuda")
        gate = torch.empty((T, cfg.K), dtype=torch.float32, device="cuda")
        ws = torch.empty(moe.moe_route_workspace_size(T, cfg.H, cfg.N_r), dtype=torch.uint8, device="cuda")
        calls = {"topk": lambda: moe.moe_route(u, E, b, cfg.K, logit_offset=inp["logit_offset"], topk_idx=idx,
                                               topk_gate=gate, workspace=ws),
                 "group_limited_8x4": lambda: moe.moe_route_group_limited(
                     u, E, b, cfg.K, 8, 4, logit_offset=inp["logit_offset"], topk_idx=idx, topk_gate=gate,
                     workspace=ws)}
        row = {}
        for k, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            for _ in range(reps):
                fn()
            s1.record()
            torch.cuda.synchronize()
            row[k + "_ms"] = s0.elapsed_time(s1) / reps
        # sequence-wise balance loss (4096-token sequences) on this batch's affinities and selection
        aff = torch.empty((T, cfg.N_r), dtype=torch.float32, device="cuda")
        moe.moe_route(u, E, b, cfg.K, logit_offset=inp["logit_offset"], affinity_out=aff, topk_idx=idx,
                      topk_gate=gate, workspace=ws)
        loss = torch.empty((T + 4095) // 4096, dtype=torch.float32, device="cuda")
        moe.moe_seq_balance_loss(aff, idx, 4096, loss=loss)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            moe.moe_seq_balance_loss(aff, idx, 4096, loss=loss)
        s1.record()
        torch.cuda.synchronize()
        row["seq_balance_loss_ms"] = s0.elapsed_time(s1) / reps
        row["seq_balance_loss"] = float(loss.mean().item())
        # plain Top-K routing: the logits GEMM as issued (three bf16 parts of the fp32 centroids,
        # 3 x 2 T H N_r flops at the bf16 peak) against reading u and the fp32 centroids once and
        # writing the selection (K indices and gates per token)
        r = binding_roof(3 * 2 * T * cfg.H * cfg.N_r, T * cfg.H * 2 + cfg.N_r * cfg.H * 4 + T * cfg.K * 8,
                         row["topk_ms"])
        row["topk_binding_roof"], row["topk_frac_of_binding_roof"] = r["binding_roof"], r["frac_of_binding_roof"]
        out[f"T={T}"] = row
        del inp, u, E, b, ws
        torch.cuda.empty_cache()
    return out


def payload_timing(reps=20, n_ranks=8):
    """FP8 dispatch payload at the FP8 workload's shape (T=8192, H=7168, 256 experts top-8) for
    8 destination ranks: pack (send plan + gathered 1x128 quantization) and unpack (to bf16)."""
    import torch
    import workloads as W
    import sparse_moe_transformer_02_amd as moe
    cfg = W.config("fp8")
    inp = W.make_inputs(cfg, device="cuda", with_weights=False)
    u = inp["u"]
    idx, _ = moe.moe_route(u, inp["centroids"], inp["bias"], cfg.K)
    p = moe.moe_pack_fp8_payload(u, idx, cfg.N_r, n_ranks)
    n = int(p["offsets"][-1].item())
    out = torch.empty((n, cfg.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_pack_fp8_payload_workspace_size(cfg.T, cfg.K, n_ranks), dtype=torch.uint8,
                     device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    pack_ms = timed(lambda: moe.moe_pack_fp8_payload(u, idx, cfg.N_r, n_ranks, workspace=ws))
    unpack_ms = timed(lambda: moe.moe_unpack_fp8_payload(p["codes"][:n], p["scales"][:n], out=out))
    row_bytes = cfg.H + cfg.H // 128 * 4
    pack_bytes = cfg.T * cfg.H * 2 + n * row_bytes          # read u once, write the payload
    unpack_bytes = n * row_bytes + n * cfg.H * 2
    return {"T": cfg.T, "n_ranks": n_ranks, "rows_sent": n, "rows_per_token": n / cfg.T,
            "payload_bytes": n * row_bytes, "bf16_rows_bytes": n * cfg.H * 2,
            "pack_ms": pack_ms, "pack_gbs": pack_bytes / pack_ms / 1e6,
            "unpack_ms": unpack_ms, "unpack_gbs": unpack_bytes / unpack_ms / 1e6,
            "binding_roof": "hbm",
            "pack_frac_of_binding_roof": binding_roof(0, pack_bytes, pack_ms)["frac_of_binding_roof"],
            "unpack_frac_of_binding_roof": binding_roof(0, unpack_bytes, unpack_ms)["frac_of_binding_roof"]}


def backward_timing(names=("decode_bf16", "prefill_bf16", "fp8_decode", "fp8"), reps=3):
    """Layer backward (combine, grouped FFN, gate/router/input backward) after a forward, per
    workload (the FP8 workloads run the FP8 backward: every GEMM operand E4M3, z / v recomputed).
    Two bf16 training forms: the forward keeps the experts' gate/up pre-activations and the
    backward uses them ("saved"), or the backward recomputes them ("recompute"). For each: ms per
    backward, the grouped FFN's row GEMMs (z/v recompute when done, dh, dx) and weight-gradient
    GEMMs from the library's HIP events, and their algorithmic work; plus the forward's ms with and
    without keeping the pre-activations."""
    import numpy as np
    import torch
    import workloads as W
    from sparse_moe_transformer_02_amd.layer import MoeLayer

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {}
    for name in names:
        cfg = W.config(name)
        inp = W.make_inputs(cfg, device="cuda")
        layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                         inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                         logit_offset=inp["logit_offset"], gamma=cfg.gamma)
        g = torch.Generator(device="cuda").manual_seed(cfg.seed)
        dout = torch.randn((cfg.T, cfg.H), generator=g, device="cuda").bfloat16()
        rec = {}
        forms = (("saved", True), ("recompute", False)) if cfg.dtype == "bf16" else (("recompute", False),)
        for form, keep in forms:
            fwd_ms = timed(lambda i=0: layer.forward(inp["u"], keep_preact=keep), reps)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
            for e in ev:                       # torch only reads events it has seen recorded once;
                for x in e:                    # the library re-records them on the stream
                    x.record()
            ms = timed(lambda i=None: layer.backward(dout, ffn_events=None if i is None else ev[i]), reps)
            rec[form] = (fwd_ms, ms, float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
                         float(np.mean([e[2].elapsed_time(e[3]) for e in ev])))
        counts = layer.last["counts"].cpu().numpy()
        rows = cfg.T * (cfg.K + 1)
        n_sel = int(np.count_nonzero(counts)) + 1
        HI = cfg.H * cfg.I
        fwd_ms, ms, rows_ms, wgrad_ms = rec[forms[0][0]]
        fp8 = cfg.dtype == "fp8"
        # row GEMMs: dh 2HI, dx 4HI per row (bf16 "saved": z, v kept by the forward; fp8: plus the
        # z, v recompute, 4HI per row)
        rows_flops = (10 if fp8 else 6) * HI * rows
        wgrad_flops = 6 * HI * rows            # dW_d 2HI, dW_g + dW_u 4HI per row
        # weight gradients: write fp32 dW of every expert, read the rows of dY, h, dz, dv and x once
        # (E4M3 codes + a scale per 128 in fp8, bf16 otherwise)
        op_bytes = 1 + 4 / 128 if fp8 else 2
        wgrad_bytes = (cfg.N_r + 1) * 3 * HI * 4 + rows * (2 * cfg.H + 3 * cfg.I) * op_bytes
        # weights read by the row GEMMs: W_g, W_u (dx) and W_d (dh) once each; fp8 also W_g, W_u for z, v
        rows_bytes = n_sel * (5 if fp8 else 3) * HI * (1 if fp8 else 2)
        out[name] = {"dtype": cfg.dtype, "ms": ms, "forward_ms": rec["recompute"][0],
                     "rows_gemm_ms": rows_ms, "wgrad_gemm_ms": wgrad_ms,
                     "rows_gemm_tflops": rows_flops / rows_ms / 1e9, "wgrad_gemm_tflops": wgrad_flops / wgrad_ms / 1e9,
                     "rows_gemm_weight_gbs": rows_bytes / rows_ms / 1e6,
                     "wgrad_gemm_gbs": wgrad_bytes / wgrad_ms / 1e6,
                     "tokens_per_s": cfg.T / (ms * 1e-3),
                     # the whole backward against the sum of its GEMMs' work (the element-wise
                     # steps around them are small beside it)
                     **binding_roof(rows_flops + wgrad_flops, rows_bytes + wgrad_bytes, ms,
                                    "fp8" if fp8 else "bf16"),
                     "rows_gemm_frac_of_binding_roof": binding_roof(rows_flops, rows_bytes, rows_ms,
                                                                    "fp8" if fp8 else "bf16")["frac_of_binding_roof"],
                     "wgrad_gemm_frac_of_binding_roof": binding_roof(wgrad_flops, wgrad_bytes, wgrad_ms,
                                                                     "fp8" if fp8 else "bf16")["frac_of_binding_roof"]}
        if not fp8:
            out[name]["forward_keeping_preact_ms"] = fwd_ms
            out[name]["recompute"] = {"ms": rec["recompute"][1], "rows_gemm_ms": rec["recompute"][2],
                                      "wgrad_gemm_ms": rec["recompute"][3]}
        del layer, inp, dout
        torch.cuda.empty_cache()
    return out


def cpu_baseline(res, budget_s=15.0):
    """The float64 oracle, as it stands, on a bounded sample of the same workload on host cores."""
    import numpy as np
    import oracle
    from workloads import bf16_bits

    cfg, inp = res["cfg"], res["inp"]
    host = lambda t: bf16_bits(t) if t.dtype.is_floating_point and t.dtype.itemsize == 2 else t.cpu().numpy()
    u = host(inp["u"])
    E = host(inp["centroids"])
    b = host(inp["bias"])
    cores = min(16, os.cpu_count() or 1)
    # sample: every token's routing + dispatch, and the layer output for S tokens
    rng = np.random.default_rng(0)
    route = oracle.route(u, E, b, cfg.K)
    S = 4
    while True:
        toks = np.sort(rng.choice(cfg.T, size=min(S, cfg.T), replace=False))
        experts = np.unique(route["idx"][toks])
        weights = {int(e): tuple(host(w[e]) for w in (inp["w_gate"], inp["w_up"], inp["w_down"])) for e in experts}
        shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
        t0 = time.perf_counter()
        oracle.layer_forward(u, E, b, cfg.K, weights, shared, fp8=cfg.dtype == "fp8", tokens=toks,
                             workers=cores)
        dt = time.perf_counter() - t0
        if dt * 2 > budget_s or S >= cfg.T:
            break
        S = min(cfg.T, S * 2)
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cfg.name}: routing + dispatch of all {cfg.T} tokens and the float64 layer output of "
                      f"{len(toks)} seeded tokens ({len(experts)} experts + shared) in {dt:.1f} s; "
                      f"tokens/s = sampled tokens / time (per-token-linear extrapolation)"}


def cpu_baseline_fp8_error(res, n_seeded=8, n_outlier=8):
    """Part of the CPU-oracle leg: the FP8 layer's error against the unquantized float64 layer
    (information only; the parity gate is against the FP8-emulating oracle, in the tests).

    One more forward of the FP8 layer on the workload's u; the oracle (without FP8 emulation)
    evaluates n_seeded seeded tokens and the n_outlier tokens holding the largest activation
    magnitudes, on the GPU's own fp32 affinities (so both sides select the same experts)."""
    import numpy as np
    import torch
    import oracle
    from workloads import bf16_bits

    cfg, inp, layer = res["cfg"], res["inp"], res["layer"]
    host = lambda t: bf16_bits(t) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()
    f64 = lambda t: (bf16_bits(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    u = inp["u"]
    bias = host(layer.bias).copy()
    out = layer.forward(u)
    torch.cuda.synchronize()
    aff = host(layer.last["affinity"])
    peak = np.abs(f64(u)).max(axis=1)
    rng = np.random.default_rng(cfg.seed)
    toks = np.unique(np.concatenate([rng.choice(cfg.T, n_seeded, replace=False),
                                     np.argsort(-peak, kind="stable")[:n_outlier]]))
    t0 = time.perf_counter()
    routed = {int(e): tuple(host(w[e]) for w in (inp["w_gate"], inp["w_up"], inp["w_down"]))
              for e in np.unique(host(layer.last["idx"])[toks])}
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    ref = oracle.layer_forward(host(u), None, bias, cfg.K, routed, shared, affinity_in=aff, tokens=toks,
                               workers=min(16, os.cpu_count() or 1))
    gpu = f64(out)[toks]
    return {"frob_rel_err_vs_unquantized_layer": float(np.linalg.norm(gpu - ref["out"]) / np.linalg.norm(ref["out"])),
            "sampled_tokens": int(len(toks)), "sample": f"{n_seeded} seeded tokens + the {n_outlier} tokens with the "
            f"largest activation magnitudes; float64 oracle without FP8 emulation ({time.perf_counter() - t0:.1f} s)"}


def _summary(res):
    cfg, w = res["cfg"], res["work"]
    s = res["ms"] * 1e-3
    pk = PEAK_TFLOPS["fp8" if cfg.dtype == "fp8" else ("f32" if cfg.dtype == "f32" else "bf16")]
    # the binding roof: the larger of the layer's MFMA-time and HBM-time floors at the peaks
    t_mfma = w["flops"] / (pk * 1e12)
    t_hbm = w["bytes"] / (PEAK_HBM_GBS * 1e9)
    d = {"tokens_per_s": cfg.T / s, "ms_per_step": res["ms"],
         "layer_tflops": w["flops"] / s / 1e12, "frac_mfma_peak": w["flops"] / s / 1e12 / pk,
         "layer_hbm_gbs": w["bytes"] / s / 1e9, "frac_hbm_peak": w["bytes"] / s / 1e9 / PEAK_HBM_GBS,
         "binding_roof": "mfma" if t_mfma > t_hbm else "hbm", "roof_ms": max(t_mfma, t_hbm) * 1e3,
         "frac_of_binding_roof": max(t_mfma, t_hbm) / s,
         "experts_selected": w["n_selected"], "max_over_mean_load": res["max_over_mean_load"]}
    for k in ("gemm1_ms", "gemm2_ms", "h_quant_ms", "stage_ms"):
        if k in res:
            d[k] = res[k]
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the layer backward of --workload (--steps backward passes)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer is built and measured on a single MI355X "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 5}))
        return

    if args.backward_only:
        print(json.dumps({"backward": backward_timing((args.workload,), reps=args.steps)}))
        return

    res = run_workload(args.workload, args.steps, args.warmup)
    cfg, w = res["cfg"], res["work"]
    value = cfg.T / (res["ms"] * 1e-3)
    bound = "hbm" if cfg.T * cfg.K / cfg.N_r < 64 else "mfma"
    if bound == "hbm":
        achieved = w["gemm1_bytes"] / (res["gemm1_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        pk = PEAK_TFLOPS["fp8" if cfg.dtype == "fp8" else "bf16"]
        achieved = w["gemm1_flops"] / (res["gemm1_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": pk, "unit": "TFLOP/s", "frac": achieved / pk}
    roof["kernel"] = "ffn1 (gate/up GEMM + SwiGLU over the shared and routed experts)"
    roof["kernel_ms"] = res["gemm1_ms"]
    roof["algorithmic_bytes"] = w["gemm1_bytes"]
    roof["traffic"] = _traffic(args.workload, "ffn1")
    main_summary = _summary(res)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(res)
    del res
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        # the graph replay first, under the same conditions as the eager steps above (after the
        # heavy workloads below the same replay measured up to 3 % slower)
        extra["decode_bf16_graph"] = graph_timing()
        for name in ("prefill_bf16", "fp8", "fp8_decode"):
            if name == args.workload:
                continue
            r = run_workload(name, max(3, args.steps // 2), 2)
            extra[name] = _summary(r)
            if name == "fp8" and not args.no_cpu_baseline:
                extra[name]["vs_unquantized"] = cpu_baseline_fp8_error(r)
            del r
            torch.cuda.empty_cache()
        extra["imbalance_bf16"] = imbalance_trajectory()
        extra["prefill_t_sweep"] = t_sweep()
        extra["ep_shard_bf16"] = ep_shard_timing()
        extra["router"] = route_timing()
        extra["fp8_payload"] = payload_timing()
        extra["backward"] = backward_timing()
        extra["ceilings"] = ceilings_timing()

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_summary["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3"}[cfg.dtype], "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} N_r={cfg.N_r} top-{cfg.K} +{cfg.N_s} shared "
                               f"I={cfg.I} {cfg.dtype}, training step (forward + bias update)",
                   "T": cfg.T, "H": cfg.H, "N_r": cfg.N_r, "K": cfg.K, "I": cfg.I, "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": main_summary,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
