"""Benchmark of the Beam MoE block forward pass on one MI355X.

    python bench.py [--workload decode|prefill|skew|fp8_decode|fp8_prefill|mxfp4_decode|mxfp4_prefill|
                     spec_verify|dense_decode|dense_prefill] [--steps K] [--warmup W] [--block]

A step is one beam_moe_forward call (router, selection, permutation, gate/up
GEMM + SwiGLU, down GEMM, combine) over one batch of seeded synthetic inputs
already resident in HBM; with --block, one beam_moe_block_forward call (the
same plus RMSNorm before, and RMSNorm + the constant-scale residual mix fused
into the combine); for the dense_* workloads, one beam_dense_mlp_forward call.
The timed region is bracketed by device synchronisation; per-kernel durations
come from HIP events that the library records on its own stream between
stages (the *_timed entry points).

Prints one JSON line: tokens/s (value), the whole layer's HBM GB/s and expert
TFLOP/s with their fractions of MI355X's peaks, a roofline entry for the
dominant kernel (gate/up), every stage kernel against its own roofline
(stages), and the CPU oracle timed on a bounded sample of the same workload
on this machine's host cores.

The metric has two halves: HBM GB/s at decode and MFMA TFLOP/s at prefill.
The default run (the decode workload, T = 64) therefore also measures the
balanced prefill workload (T = 8192) on the same expert weights and puts it
in the same line as "prefill" (ms, tokens/s, MFMA TFLOP/s and fraction,
stage rooflines, its own CPU-oracle sample, and for scale the vendor GEMM
library's sustained bf16 rate on large square products on the same GPU);
--no-prefill leaves it out.
--steps / --warmup set the headline workload's counts; the prefill part
uses its own defaults.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + HBM GB/s (decode) / MFMA TFLOP/s (prefill) vs peak, 1 GPU"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
STAGES = ["router_logits", "router_select", "permute", "gateup", "down", "combine"]
BLOCK_STAGES = ["pre_norm", "router_logits", "router_select", "permute", "gateup", "down", "combine_norm_mix"]
BLOCK_STEP, BLOCK_EPS = 23, 1e-6
DEFAULTS = {"decode": (200, 20), "fp8_decode": (200, 20), "prefill": (30, 5), "skew": (40, 5), "fp8_prefill": (60, 5),
            "mxfp4_decode": (200, 20), "mxfp4_prefill": (60, 5), "spec_verify": (200, 20), "dense_decode": (200, 20),
            "dense_prefill": (30, 5)}
DENSE_STAGES = ["setup", "gateup", "down"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"stream": ("experts.hip", "common.h"), "tiled": ("experts_tiled.hip", "common.h"),
                  "wide": ("experts_wide.hip", "common.h")}
KERNEL_NAMES = {"stream": "gateup_stream_kernel", "tiled": "tiled_kernel<gateup>", "wide": "wide_kernel<gateup>"}


def kernel_source_hash(kind):
    """Hash of the sources of the gate/up kernel family ("stream", "tiled" or "wide")."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, "sparse_moe_layer_top_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel, kind, order):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken on this kernel source
    with the weights in this byte order."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != kernel_source_hash(kind) or d.get("weight_order", "rows") != order:
        return None
    return d.get("bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x_bits, wr, b, seconds_target=20.0, block=False):
    """The oracle as it stands, on a bounded token sample of the same workload (host cores)."""
    import oracle
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    n = 2 if w.T >= 2 else 1
    if w.n_experts == 1:                     # dense MLP: generate its three matrices once (not timed)
        mats = [gen.expert_matrix(w, 0, k, 0) for k in ("gate", "up", "down")]
        total_t, total_tok = 0.0, 0
        for start in range(0, w.T, n):
            t0 = time.perf_counter()
            oracle.dense_mlp(x_bits[start:start + n], *mats, weight=w.weight)
            total_t += time.perf_counter() - t0
            total_tok += min(n, w.T - start)
            if total_t > seconds_target * 0.5:
                break
        return {"value": total_tok / total_t, "unit": "tokens/s", "cores": int(threads), "cpu": cpu_model(),
                "kind": "oracle",
                "sample": f"{total_tok} tokens of the {w.name} batch (T={w.T}), dense MLP per token, "
                          f"{total_t:.1f} s of oracle time, weight generation excluded"}
    spec = oracle.LayerSpec.of(w)
    src = gen.ExpertSource(w, 0)
    total_t, total_tok = 0.0, 0
    start = 0
    while start < w.T and (total_t < seconds_target or total_tok == 0):
        sel = slice(start, min(start + n, w.T))
        xs = oracle.rms_norm_bits(x_bits[sel], gen.norm_gains(w, 0)[0], BLOCK_EPS) if block else x_bits[sel]
        ids, _ = oracle.route(spec, xs, wr, b)
        src.prefetch(np.unique(ids))        # input generation: not timed
        t0 = time.perf_counter()
        if block:
            gpre, gpost = gen.norm_gains(w, 0)
            oracle.block_forward(spec, x_bits[sel], gpre, gpost, BLOCK_EPS, BLOCK_STEP, wr, b, src.get)
        else:
            oracle.forward(spec, x_bits[sel], wr, b, src.get)
        total_t += time.perf_counter() - t0
        total_tok += sel.stop - sel.start
        src.drop()
        start = sel.stop
        if total_t > seconds_target * 0.5:
            break
    return {"value": total_tok / total_t, "unit": "tokens/s", "cores": int(threads), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{total_tok} tokens of the {w.name} batch (T={w.T}), "
                      f"{'whole sublayer' if block else 'full layer'} per token, "
                      f"{total_t:.1f} s of oracle time, weight generation excluded"}


def gateup_kind(w, packed=True):
    """Which gate/up kernel family the library runs for this workload (mirrors its schedule choice):
    LDS-tiled from 32 rows per expert (the dense path streams up to 1024 tokens); the
    one-workgroup-per-CU kernel for MoE layers at 32..64 rows per expert (any weight type), and from
    192 rows per expert (bf16; above 64 with the weights in fragment order) wherever the LDS-tiled
    one would run, dense included."""
    dense = w.n_experts == 1
    TK, H, I = w.T * w.top_k, w.hidden, w.inter
    tiled = (TK / w.n_experts >= 32 and H % 256 == 0 and I % 128 == 0 and not (dense and w.T <= 1024)
             and w.weight != "mxfp4")
    wk = 128 if w.weight == "mxfp4" else 64      # k per window
    wide_ok = (TK >= 32 * w.n_experts and w.T * H * 2 < 2 ** 31 and H * I * 2 < 2 ** 31
               and H % (4 * wk) == 0 and I % (4 * wk) == 0)
    wide = wide_ok and ((not dense and TK <= 64 * w.n_experts and H % 512 == 0 and I % 256 == 0)
                        or (w.weight == "bf16" and TK >= (64 if packed else 192) * w.n_experts and tiled))
    return "wide" if wide else ("tiled" if tiled else "stream")


def measure(w, W, x_bits, wr, b, steps, warmup, block=False, stage_events=True, seed=0, layout=1):
    """Time `steps` forward passes of workload w on resident inputs (expert weights W in row order,
    layout 0, or fragment order, layout 1); returns the workload's figures."""
    import torch
    import sparse_moe_layer_top_amd as bm
    from synth import gen

    dev = torch.device("cuda:0")
    wtype = {"bf16": bm.W_BF16, "fp8": bm.W_FP8_E4M3, "mxfp4": bm.W_MXFP4}[w.weight]
    cfg = bm.Config(w.hidden, w.inter, w.n_experts, w.n_groups, w.topk_groups, w.top_k, w.alpha, wtype, layout)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    wr_t = torch.from_numpy(wr).to(dev)
    b_t = torch.from_numpy(b).to(dev)
    out = torch.empty(w.T, w.hidden, dtype=torch.bfloat16, device=dev)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device=dev)
    wts = torch.empty(w.T, w.top_k, dtype=torch.float32, device=dev)
    dense = w.n_experts == 1
    if not dense:
        ws = torch.empty(bm.beam_moe_workspace_bytes(cfg, w.T), dtype=torch.uint8, device=dev)
    stages = BLOCK_STAGES if block else (DENSE_STAGES if dense else STAGES)
    if dense:
        dcfg = bm.DenseConfig(w.hidden, w.inter, wtype, layout)
        Wd = {k: v[0] for k, v in W.items()}
        ws = torch.empty(max(1, bm.beam_dense_workspace_bytes(dcfg, w.T)), dtype=torch.uint8, device=dev)
    if block:
        gpre, gpost = (torch.from_numpy(g).to(dev) for g in gen.norm_gains(w, seed))
        stream_out = torch.empty_like(x)
        ws = torch.empty(bm.beam_moe_workspace_bytes(cfg, w.T, bm.OP_BLOCK), dtype=torch.uint8, device=dev)

    def step(events=None):
        if dense:
            bm.beam_dense_mlp_forward(dcfg, x, Wd["gate"], Wd["up"], Wd["down"], Wd.get("s_gate"), Wd.get("s_up"),
                                      Wd.get("s_down"), out=out, workspace=ws, stage_events=events)
        elif block:
            bm.beam_moe_block_forward(cfg, BLOCK_STEP, BLOCK_EPS, x, gpre, gpost, wr_t, b_t, W["gate"], W["up"],
                                      W["down"], W.get("s_gate"), W.get("s_up"), W.get("s_down"),
                                      stream_out=stream_out, topk_ids_out=ids, topk_w_out=wts, workspace=ws,
                                      stage_events=events)
        else:
            bm.beam_moe_forward(cfg, x, wr_t, b_t, W["gate"], W["up"], W["down"], W.get("s_gate"), W.get("s_up"),
                                W.get("s_down"), out=out, topk_ids_out=ids, topk_w_out=wts, workspace=ws,
                                stage_events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    nev = len(stages) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for row in evs:              # record once so each event exists before the library records it
        for e in row:
            e.record()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: timing {steps} steps")
    start.record()
    for i in range(steps):
        step(evs[i] if stage_events else None)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    stage_ms = {name: (float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
                       if stage_events else float("nan"))
                for j, name in enumerate(stages)}

    # routing statistics and algorithmic work of this batch
    ids_h = np.zeros((w.T, 1), np.int32) if dense else ids.cpu().numpy()
    load = np.bincount(ids_h.ravel(), minlength=w.n_experts)
    D = int((load > 0).sum())
    TK = w.T * w.top_k
    H, I = w.hidden, w.inter

    def mat_bytes(rows, cols):
        """Bytes of one [rows, cols] weight matrix with its scales."""
        return {"bf16": 2 * rows * cols, "fp8": rows * cols + 4 * rows,
                "mxfp4": rows * cols // 2 + rows * cols // 32}[w.weight]

    gu_bytes = D * 2 * mat_bytes(I, H) + w.T * H * 2 + TK * I * 2
    layer_bytes = D * (2 * mat_bytes(I, H) + mat_bytes(H, I)) + 2 * w.T * H * 2
    if not dense:
        layer_bytes += H * w.n_experts * 4 + w.n_experts * 4          # router weights and bias
    layer_flops = 6.0 * TK * H * I
    gu_flops = 4.0 * TK * H * I
    sec = ms / 1e3
    hbm_gbps = layer_bytes / sec / 1e9
    tflops = layer_flops / sec / 1e12
    kind = gateup_kind(w, packed=bool(layout))
    res = {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / sec, 1),
           "hbm_GBps": round(hbm_gbps, 1), "hbm_frac": round(hbm_gbps / PEAK_HBM_GBPS, 4),
           "expert_TFLOPs": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
           "layer_bytes": layer_bytes, "layer_flops": layer_flops,
           "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
           "routing": None if dense else {"touched_experts": D, "max_load": int(load.max()),
                                          "mean_load": TK / w.n_experts, "zero_load_experts": int((load == 0).sum())}}
    if not stage_events:
        return res
    # each step's own span (its first stage event to its last): spread over the timed steps
    per_step = np.array([evs[i][0].elapsed_time(evs[i][nev - 1]) for i in range(steps)])
    res["step_ms"] = {"median": round(float(np.median(per_step)), 4), "min": round(float(per_step.min()), 4),
                      "max": round(float(per_step.max()), 4)}
    t_gu = stage_ms["gateup"] / 1e3
    # the dominant kernel's roofline: the resource whose floor (work / peak) is the larger one binds
    gbps = gu_bytes / t_gu / 1e9
    tfs = gu_flops / t_gu / 1e12
    if gu_bytes / (PEAK_HBM_GBPS * 1e9) >= gu_flops / (PEAK_BF16_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfs, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfs / PEAK_BF16_TFLOPS, 4)}
    roof["traffic"] = load_traffic(w.name, "gateup", kind, "fragments" if layout else "rows")
    roof["kernel"] = KERNEL_NAMES[kind]
    roof["algorithmic_bytes_per_launch"] = gu_bytes
    roof["algorithmic_flops_per_launch"] = gu_flops
    roof["hbm_GBps"] = round(gbps, 1)
    roof["hbm_frac"] = round(gbps / PEAK_HBM_GBPS, 4)
    roof["mfma_TFLOPs"] = round(tfs, 1)
    roof["mfma_frac"] = round(tfs / PEAK_BF16_TFLOPS, 4)

    # every stage against its own roofline: algorithmic bytes (weights of the touched experts, activations
    # in and out) and FLOPs of the step, over the stage's live event time; the bound is the larger floor
    mfma_mult = {"router_logits": 3.0}     # W_router runs as three exact bf16 planes on the MFMAs
    work = {
        "pre_norm": (2 * w.T * H * 2 + H * 4, 0.0),
        "router_logits": (w.T * H * 2 + H * w.n_experts * 4, 2.0 * w.T * H * w.n_experts),
        "router_select": (w.T * w.n_experts * 4 + TK * 8, 0.0),
        "permute": (TK * 4 + (w.n_experts + 1) * 4 + 2 * TK * 4, 0.0),
        "setup": (w.T * 4, 0.0),
        "gateup": (gu_bytes, gu_flops),
        "down": (D * mat_bytes(H, I) + TK * I * 2 + TK * H * 2, 2.0 * TK * H * I),
        "combine": (TK * H * 2 + w.T * H * 2 + TK * 8, 0.0),
        "combine_norm_mix": (TK * H * 2 + 2 * w.T * H * 2 + H * 4 + TK * 8, 0.0),
    }
    stages_roof = {}
    for name in stages:
        t = stage_ms[name] / 1e3
        if not t > 0:
            continue
        nbytes, nflops = work[name]
        mflops = nflops * mfma_mult.get(name, 1.0)
        hbm_floor = nbytes / (PEAK_HBM_GBPS * 1e9)
        mfma_floor = mflops / (PEAK_BF16_TFLOPS * 1e12)
        ent = {"ms": round(stage_ms[name], 4), "bytes": nbytes, "GBps": round(nbytes / t / 1e9, 1),
               "hbm_frac": round(hbm_floor / t, 4)}
        if nflops:
            ent.update(flops=nflops, TFLOPs=round(nflops / t / 1e12, 2), mfma_frac=round(mfma_floor / t, 4))
        ent["bound"] = "mfma" if mfma_floor > hbm_floor else "hbm"
        ent["frac"] = round(max(hbm_floor, mfma_floor) / t, 4)
        stages_roof[name] = ent
    res["roofline"] = roof
    res["stages"] = stages_roof
    if block:
        # the two norm kernels: rows read and written (plus the combine's y reads for the fused one)
        norm_bytes = 2 * w.T * H * 2 + H * 4
        cnm_bytes = TK * H * 2 + 2 * w.T * H * 2 + H * 4 + TK * 8
        res["block"] = {"step": BLOCK_STEP, "eps": BLOCK_EPS,
                        "pre_norm_GBps": round(norm_bytes / (stage_ms["pre_norm"] / 1e3) / 1e9, 1),
                        "combine_norm_mix_GBps": round(cnm_bytes / (stage_ms["combine_norm_mix"] / 1e3) / 1e9, 1),
                        "pre_norm_bytes": norm_bytes, "combine_norm_mix_bytes": cnm_bytes}
    return res


def describe(w, block=False):
    H, I = w.hidden, w.inter
    return ((f"{w.name}: T={w.T}, dense SwiGLU MLP, hidden {H}, inter {I}" if w.n_experts == 1 else
             f"{w.name}: T={w.T}, hidden {H}, {w.n_experts} SwiGLU experts of inter {I}, "
             f"{w.n_groups} groups, top-{w.topk_groups} groups, top-{w.top_k}, x{w.alpha}")
            + (f"; whole sublayer: RMSNorm before and after, residual mix at step {BLOCK_STEP}" if block else ""))


GEMM_CEILING_SHAPES = [(8192, 8192, 8192), (16384, 16384, 16384), (8192, 5120, 40960)]


def gemm_ceiling(torch, dev, shapes=GEMM_CEILING_SHAPES, reps=20, warmup=5):
    """Dense bf16 rate of the vendor GEMM library on large products [M, K] x [K, N] (plain 2-D matmul of
    contiguous operands), timed with events on the current stream: the rate the chip sustains on
    MFMA-bound work, for scale against the datasheet peak."""
    out = {"gemm_ceiling": [], "peak_TFLOPs": PEAK_BF16_TFLOPS}
    for (M, K, N) in shapes:
        g = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        b = torch.randn(K, N, device=dev, generator=g).to(torch.bfloat16)
        c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        for _ in range(warmup):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        tf = 2.0 * M * K * N / (ms * 1e-3) / 1e12
        out["gemm_ceiling"].append({"M": M, "K": K, "N": N, "ms": round(ms, 4), "TFLOPs": round(tf, 1),
                                    "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        log(f"[bench] matmul {M}x{K}x{N}: {ms:.3f} ms, {tf:.0f} TFLOP/s")
        del a, b, c
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode", choices=sorted(DEFAULTS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the decode workload, leave out the balanced prefill part of the line")
    ap.add_argument("--block", action="store_true",
                    help="time the whole sublayer: pre-norm, the MoE block, post-norm and the residual mix "
                         "(beam_moe_block_forward, step 23 = layer 10's MoE sublayer)")
    ap.add_argument("--no-stage-events", action="store_true",
                    help="time the steps without the per-stage events (no roofline entry)")
    ap.add_argument("--weight-order", default="fragments", choices=["fragments", "rows"],
                    help="byte order of the expert weights (and MXFP4 scales) in HBM: fragment order "
                         "(written once by beam_moe_pack_weights / beam_moe_pack_scales before timing; the "
                         "default) or row order")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the layer, run 5 plain device copies of MIB MiB (a known-size "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="instead of the layer, time the vendor GEMM library (torch.matmul, bf16, contiguous "
                         "operands) on large products (two square, one the dense prefill gate/up shape): the dense "
                         "bf16 rate this GPU sustains, for scale against the 2.5 PFLOP/s datasheet peak")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer's multi-GPU "
              "sharding is not built here", file=sys.stderr)
        sys.exit(2)
    steps, warmup = DEFAULTS[args.workload]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup

    import torch
    import sparse_moe_layer_top_amd  # noqa: F401  (fails loudly if the library is not built)
    from synth import gen

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        c = torch.empty_like(a)
        for _ in range(5):
            c.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return
    if args.gemm_ceiling:
        print(json.dumps(gemm_ceiling(torch, dev)), flush=True)
        return
    w = gen.workload(args.workload)
    if w.n_experts == 1 and args.block:
        print("--block applies to the MoE workloads", file=sys.stderr)
        sys.exit(2)
    log(f"[bench] {w.name}: T={w.T} H={w.hidden} I={w.inter} E={w.n_experts} weights={w.weight}")
    x_bits, wr, b = gen.router_inputs(w, args.seed)
    t0 = time.time()
    W = gen.device_expert_weights(w, args.seed, dev, log=log)
    log(f"[bench] expert weights on device in {time.time() - t0:.1f} s")
    layout = 1 if args.weight_order == "fragments" else 0
    if layout:
        import sparse_moe_layer_top_amd as bm
        for k in ("gate", "up", "down"):       # one matrix stack at a time: one extra copy at most
            W[k] = bm.beam_moe_pack_weights(W[k])
            if w.weight == "mxfp4":
                W["s_" + k] = bm.beam_moe_pack_scales(W["s_" + k])
            torch.cuda.synchronize()
        log("[bench] expert weights packed into fragment order")
    m = measure(w, W, x_bits, wr, b, steps, warmup, block=args.block, stage_events=not args.no_stage_events,
                seed=args.seed, layout=layout)

    res = {
        "metric": METRIC, "value": m["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 MFMA",
                                       "mxfp4": "mxfp4 (e2m1 + e8m0) weights, bf16 MFMA"}[w.weight],
        "data": "synthetic (seeded, random-init weights of the real layer shape)",
        "config": {"workload": describe(w, args.block), "T": w.T, "weights": w.weight, "bias": w.bias,
                   "weight_order": args.weight_order},
    }
    res.update({k: v for k, v in m.items() if k not in ("ms_per_step", "tokens_per_s")})
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(w, x_bits, wr, b, block=args.block)

    # the prefill half of the metric: balanced prefill on the same expert weights (MFMA TFLOP/s vs peak)
    if args.workload == "decode" and not args.block and not args.no_prefill:
        wp = gen.workload("prefill")
        assert wp.weights_id == w.weights_id and wp.weight == w.weight
        psteps, pwarm = DEFAULTS["prefill"]
        px, pwr, pb = gen.router_inputs(wp, args.seed)
        pm = measure(wp, W, px, pwr, pb, psteps, pwarm, stage_events=not args.no_stage_events, seed=args.seed,
                     layout=layout)
        pref = {"workload": describe(wp), "T": wp.T, "bias": wp.bias, "steps": psteps, "warmup": pwarm,
                "target": {"ms_per_step": 4.10, "mfma_frac": 0.5}}
        pref.update(pm)
        # for scale: the vendor library's sustained rate on large square products on this same GPU
        ceil = gemm_ceiling(torch, dev, shapes=GEMM_CEILING_SHAPES[:2])
        best = max(g["TFLOPs"] for g in ceil["gemm_ceiling"])
        ceil["best_TFLOPs"] = best
        ceil["layer_expert_TFLOPs_over_best"] = round(pm["expert_TFLOPs"] / best, 4)
        gu = pm.get("stages", {}).get("gateup", {}).get("TFLOPs")
        ceil["gateup_TFLOPs_over_best"] = round(gu / best, 4) if gu else None
        pref["vendor_gemm_ceiling"] = ceil
        if not args.no_cpu_baseline:
            log("[bench] CPU oracle baseline (prefill)")
            pref["cpu_baseline"] = cpu_baseline(wp, px, pwr, pb)
        res["prefill"] = pref
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
