#!/usr/bin/env python3
"""Benchmark of the MoE FFN forward on one MI355X.

Workload (default): the Zipf-skewed layer, T=16384 tokens, H=4096, I=2048, E=128
experts, top-8, bf16, router logits N(0,1) plus a per-expert bias ln(rank^-1.2)
(seed 0).  A step is one moe_forward call: route, permutation tables, row gather,
GEMM1 + SwiGLU, GEMM2, combine, with every input already resident in HBM.

Timing: W untimed warm-up steps, then K moe_forward steps bracketed by device
synchronisation and HIP events on the library's stream (ms_per_step, value).  Then K
single forwards, each after a 512 MB write that flushes the caches (median:
cold_cache_ms_per_step).  Then one forward captured in a HIP graph and replayed K times
(median graph_ms_per_step), and K times after a flush each (graph_cold_ms_per_step: the
FlashInfer MegaMoE Performance section's method, one MoE call per graph, cold cache
before each call).  The
per-stage durations come from K further steps through moe_forward_timed (same
kernels plus a HIP event at every stage boundary), measured live in the same run.
On bf16 data the forward folds the row gather into GEMM1; the permute kernel's own
HBM rate comes from K calls of moe_permute_timed on the same routing.

Prints one JSON line.  The CPU baseline is the fp64 oracle (test infrastructure)
timed on a bounded, stratified sample of the same workload on the host cores (one
token routed to every non-empty expert plus evenly spaced tokens, at least 2048),
with the full layer's time extrapolated from that rate and labelled so.  With the
default workload the line also carries `per_config`: the same measurements (fewer
steps, no standalone permute) for the tiny and mid layers, the W4A8 decode layer at
1, 16 and 256 tokens with NVFP4 and MXFP4 weights (HBM roofline of the expert FFN),
and the ep_share layer.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s + TFLOP/s (% MFMA peak), permute/combine % HBM, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(roles, workload, T, seed):
    """HBM bytes per forward of the kernels in roles (each launched once per forward), summed from
    the committed counter summary, if every record was taken on the current source of its kernel
    and on this workload, token count and seed (None otherwise)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        recs = json.load(fh)
    total = 0
    for role in roles:
        rec = next((r for r in recs if r.get("role") == role and r.get("workload") == workload
                    and r.get("T") == T and r.get("seed") == seed), None)
        if rec is None or rec.get("source_sha") != source_hash(rec["source_files"]):
            return None
        total += rec["bytes_per_launch"]
    return total


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s, min_tokens=2048):
    """The fp64 oracle on the host cores: a stratified sample of at least min_tokens tokens (all of
    them if T is smaller) that holds one token routed to every non-empty expert, the rest evenly
    spaced; the rate is extrapolated to the whole layer and labelled so."""
    import oracle
    cfg = inp["cfg"]
    cores = oracle.max_threads()
    idx, _ = oracle.route(inp["logits"], cfg.k, inp.get("slot_drop"))   # cheap: T x E
    live = np.unique(idx[idx >= 0])
    strata = np.unique([int(np.argmax((idx == e).any(axis=1))) for e in live]).astype(np.int32)
    probe = np.linspace(0, cfg.T - 1, 2 * cores).astype(np.int32)  # two tokens per thread
    t0 = time.perf_counter()
    oracle.moe_forward(inp, probe)
    per_tok = (time.perf_counter() - t0) / probe.size
    n = int(min(cfg.T, max(min_tokens, budget_s / max(per_tok, 1e-9))))
    spread = np.linspace(0, cfg.T - 1, max(n - strata.size, 1)).astype(np.int32)
    tokens = np.union1d(strata, spread).astype(np.int32)
    hit = np.unique(idx[tokens][idx[tokens] >= 0]).size
    log(f"cpu baseline: oracle on {tokens.size} tokens ({hit} of {live.size} non-empty experts) with {cores} "
        f"threads (~{tokens.size * per_tok:.0f} s)")
    t0 = time.perf_counter()
    oracle.moe_forward(inp, tokens)
    dt = time.perf_counter() - t0
    rate = tokens.size / dt
    return {"value": round(rate, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{tokens.size} tokens of the {cfg.name} workload (T={cfg.T}), all k slots each, fp64: one "
                      f"token routed to each of the {live.size} non-empty experts plus evenly spaced tokens; "
                      f"{hit} experts hit; {dt:.1f} s",
            "experts_hit": int(hit), "experts_nonempty": int(live.size),
            "full_layer_s_extrapolated": round(cfg.T / rate, 1)}


def dense_gemm_reference(args):
    """hipBLASLt (through torch.matmul) on dense GEMMs of the grouped GEMMs' sizes: M = T*k rows,
    GEMM1 [M, H] x [2I, H]^T and GEMM2 [M, I] x [H, I]^T, bf16, both operands K-contiguous."""
    import torch
    from moe_synth import CONFIGS

    cfg = CONFIGS[args.workload]
    M = cfg.T * cfg.k
    dev = torch.device("cuda:0")
    out = {"dense_gemm_reference": f"torch.matmul bf16 (hipBLASLt), {args.workload} sizes", "results": []}
    for name, N, K in (("gemm1", 2 * cfg.I, cfg.H), ("gemm2", cfg.H, cfg.I)):
        a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        b = torch.randn(N, K, device=dev, dtype=torch.bfloat16)
        for _ in range(args.warmup):
            c = a @ b.t()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            c = a @ b.t()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out["results"].append({"gemm": name, "M": M, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(tf, 1),
                               "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        del a, b, c
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="skewed")
    ap.add_argument("--tokens", type=int, default=None, help="token count override (e.g. the W4A8 sweep points)")
    ap.add_argument("--w4-layout", choices=("tiled", "rows"), default="tiled",
                    help="W4A8 weight storage: tiled (prepared once by moe_w4a8_tile_weights) or row-major")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-launch", action="store_true",
                    help="W4A8 workloads: the whole forward in one launch (MOE_FLAG_SINGLE_LAUNCH)")
    ap.add_argument("--scatter-y", action="store_true",
                    help="GEMM2 stores its rows in slot order and the combine reads them so (MOE_FLAG_SCATTER_Y)")
    ap.add_argument("--configs", choices=("all", "none"), default="all",
                    help="with the default workload, also report every other configuration (fewer steps each)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference kernel for HBM byte counters)")
    ap.add_argument("--dense-gemm-reference", action="store_true",
                    help="only time the vendor library's dense bf16 GEMMs (torch.matmul, hipBLASLt) with the grouped "
                         "GEMMs' total rows and shapes, as a reference point for the MFMA fraction on this device")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4, "copy_calibration_bytes_written": b.numel() * 4}))
        return

    if args.dense_gemm_reference:
        dense_gemm_reference(args)
        return

    from moe_synth import CONFIGS

    cfg = CONFIGS[args.workload]
    if args.tokens is not None:
        cfg = cfg.with_tokens(args.tokens)
    result, inp = measure(cfg, args, detail=True)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    del inp
    if args.configs == "all" and args.workload == "skewed" and args.tokens is None:
        result["per_config"] = per_config(args)
    print(json.dumps(result), flush=True)


# The other configurations of the workload set, reported beside the headline line (fewer steps
# each; every record from the same run): the mid layer, the W4A8 decode layer at 1, 16 and 256
# tokens with NVFP4 and MXFP4 weights, and one GPU's share of an expert-parallel layer.
PER_CONFIG = [("tiny", None), ("mid", None), ("w4a8", 1), ("w4a8", 16), ("w4a8", 256), ("w4a8_mx", 1),
              ("w4a8_mx", 16), ("w4a8_mx", 256), ("ep_share", None)]
# also measured as one launch (MOE_FLAG_SINGLE_LAUNCH)
PER_CONFIG_SINGLE = [("w4a8", 1), ("w4a8_mx", 1), ("w4a8_mx", 16)]


def per_config(args):
    from moe_synth import CONFIGS

    from moe_synth import generate

    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = min(args.steps, 10), min(args.warmup, 3)
    out = []
    base = {}  # one draw per W4A8 workload: the first T tokens of it are the T-token draw
    for name, T, single in [(n, t, False) for n, t in PER_CONFIG] + [(n, t, True) for n, t in PER_CONFIG_SINGLE]:
        sub.single_launch = single
        cfg = CONFIGS[name] if T is None else CONFIGS[name].with_tokens(T)
        inp = None
        if T is not None:
            if name not in base:
                t0 = time.perf_counter()
                base = {name: generate(CONFIGS[name], seed=args.seed)}
                log(f"generated {name} (seed {args.seed}) in {time.perf_counter() - t0:.1f} s")
            b = base[name]
            inp = dict(b, cfg=cfg, logits=b["logits"][:T], x=b["x"][:T], x_scale=b["x_scale"][:T])
        r, _ = measure(cfg, sub, detail=False, inp=inp)
        keep = ("value", "unit", "ms_per_step", "dtype", "config", "tflops_forward", "tflops_gemms", "mfma_frac_gemms",
                "combine_hbm_frac", "stage_ms", "cold_cache_ms_per_step", "graph_ms_per_step",
                "graph_cold_ms_per_step", "roofline", "steps", "warmup")
        rec = {k: r[k] for k in keep}
        if single:
            rec["single_launch"] = True
        out.append(rec)
    return out


def measure(cfg, args, detail, inp=None):
    """One workload: inputs resident on the GPU, then the timed moe_forward steps, cold-cache and
    graph medians, the stage breakdown and the dominant kernel's roofline.  detail adds the
    standalone permute measurement."""
    import torch

    import token_permute_grouped_amd as tpg
    from moe_synth import generate

    if inp is None:
        t0 = time.perf_counter()
        inp = generate(cfg, seed=args.seed)
        log(f"generated {cfg.name} T={cfg.T} (seed {args.seed}) in {time.perf_counter() - t0:.1f} s")

    dev = torch.device("cuda:0")

    def dt(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    w4 = cfg.prec != "bf16"
    mx = cfg.prec == "w4a8_mx"
    flags = (tpg.MOE_FLAG_SINGLE_LAUNCH if getattr(args, "single_launch", False) else
             tpg.MOE_FLAG_SCATTER_Y if getattr(args, "scatter_y", False) else 0)
    p = tpg.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, tpg.PRECISIONS[cfg.prec], cfg.glu_interleave,
                         cfg.swiglu_clamp, flags)
    d = {k: dt(inp.get(k)) for k in ("logits", "slot_drop", "x", "x_scale", "w1", "w1_bscale", "w1_gscale", "w2",
                                      "w2_bscale", "w2_gscale")}
    layout = tpg.MOE_W4_LAYOUT_ROWS
    if w4 and args.w4_layout == "tiled":
        # the weights prepared once, as a deployment would at load time (moe_w4a8_tile_weights)
        for m, (n, kk) in (("w1", (2 * cfg.I, cfg.H)), ("w2", (cfg.H, cfg.I))):
            ct, st = torch.empty_like(d[m]), torch.empty_like(d[m + "_bscale"])
            tpg.moe_w4a8_tile_weights(d[m], d[m + "_bscale"], ct, st, cfg.E, n, kk, p.prec)
            d[m], d[m + "_bscale"] = ct, st
        layout = tpg.MOE_W4_LAYOUT_TILED
    wts = tpg.make_weights(d["w1"], d["w2"], d["w1_bscale"], d["w1_gscale"], d["w2_bscale"], d["w2_gscale"], layout)
    ws = torch.empty(tpg.moe_workspace_bytes(p), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident on {torch.cuda.get_device_name(0)}; workspace {ws.numel() / 2**30:.2f} GiB")

    def step(events=None):
        if events is None:
            tpg.moe_forward(d["logits"], d["slot_drop"], d["x"], d["x_scale"], wts, p, out, ws)
        else:
            tpg.moe_forward_timed(d["logits"], d["slot_drop"], d["x"], d["x_scale"], wts, p, out, ws, events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warm-up done ({args.warmup} steps)")

    # timed region: K plain moe_forward calls, HIP events on the library's stream around them
    hip = HipEvents()
    e0, e1 = hip.create(), hip.create()
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    hip.record(e0, stream)
    for _ in range(args.steps):
        step()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    step_ms = hip.ms(e0, e1) / args.steps
    hip.destroy(e0)
    hip.destroy(e1)
    log(f"timed {args.steps} steps: {step_ms:.4f} ms/step (events), {wall_ms:.4f} ms/step (wall)")

    # cold caches: before each of K single forwards, overwrite a 512 MB buffer (evicts the L2s
    # and the 256 MB last-level cache), then time the forward alone between HIP events; median
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        c0, c1 = hip.create(), hip.create()
        hip.record(c0, stream)
        step()
        hip.record(c1, stream)
        torch.cuda.synchronize()
        cold.append(hip.ms(c0, c1))
        hip.destroy(c0)
        hip.destroy(c1)
    cold_ms = float(np.median(cold))
    log(f"cold caches: median {cold_ms:.4f} ms per forward over {args.steps}")

    # one forward per HIP graph: captured once (torch's graph capture on its own stream; the
    # library enqueues on torch's current stream, allocates nothing and records no memset),
    # replayed K times warm and K times each after the 512 MB flush
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph_runs = {False: [], True: []}
    for flushed in (False, True):
        for i in range(args.steps):
            if flushed:
                flush.fill_(i & 0xFF)
            c0, c1 = hip.create(), hip.create()
            hip.record(c0, stream)
            graph.replay()
            hip.record(c1, stream)
            torch.cuda.synchronize()
            graph_runs[flushed].append(hip.ms(c0, c1))
            hip.destroy(c0)
            hip.destroy(c1)
    del graph, flush
    graph_ms, graph_cold_ms = float(np.median(graph_runs[False])), float(np.median(graph_runs[True]))
    log(f"graph replay: median {graph_ms:.4f} ms warm, {graph_cold_ms:.4f} ms with the caches flushed")

    # stage breakdown: K more steps through moe_forward_timed (same kernels plus a HIP event at
    # every stage boundary; each event adds a few microseconds, visible only at small T)
    evs = [[hip.create() for _ in range(tpg.MOE_N_STAGE_EVENTS)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = {}
    for s_, name in enumerate(tpg.STAGES):
        stage_ms[name] = float(np.mean([hip.ms(evs[i][s_], evs[i][s_ + 1]) for i in range(args.steps)]))
    for row in evs:
        for e in row:
            hip.destroy(e)

    permute_tables_ms = permute_gather_ms = permute_gather_after_fwd_ms = float("nan")
    if detail:
        # the permute (tables + row gather) on its own, on the forward's routing: the gather kernel's
        # HBM rate (the bf16 forward runs no separate gather)
        S = cfg.T * cfg.k
        idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
        tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
        tpg.moe_route_topk(d["logits"], d["slot_drop"], p, idx, tw)
        offs = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
        rsrc = torch.empty(S, dtype=torch.int32, device=dev)
        srow = torch.empty(S, dtype=torch.int32, device=dev)
        x_perm = torch.empty((S, cfg.H), dtype=torch.uint8 if w4 else torch.int16, device=dev)
        x_perm_scale = torch.empty((S, cfg.H // 128), dtype=torch.float32, device=dev) if w4 else None
        pws = torch.empty(max(1, tpg.moe_call_workspace_bytes(p, tpg.MOE_WS_PERMUTE)), dtype=torch.uint8, device=dev)
        def permute_run(after_forward):
            pev = [[hip.create() for _ in range(tpg.MOE_N_PERMUTE_EVENTS)] for _ in range(args.steps + 2)]
            for i in range(args.steps + 2):  # the first two are warm-up
                if after_forward:
                    step()
                tpg.moe_permute_timed(d["x"], d["x_scale"], idx, p, offs, rsrc, srow, x_perm, x_perm_scale, pws, pev[i])
            torch.cuda.synchronize()
            tab = float(np.mean([hip.ms(pev[i][0], pev[i][1]) for i in range(2, args.steps + 2)]))
            gat = float(np.mean([hip.ms(pev[i][1], pev[i][2]) for i in range(2, args.steps + 2)]))
            for row in pev:
                for e in row:
                    hip.destroy(e)
            return tab, gat

        # back to back: each call also pays the write-back of the previous call's x_perm from the
        # last-level cache (the steady state of a loop of permutes)
        permute_tables_ms, permute_gather_ms = permute_run(False)
        # right after a forward, as the permute would run inside a layer's pipeline
        _, permute_gather_after_fwd_ms = permute_run(True)
        del x_perm, x_perm_scale, pws

    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    R = T * k - (int(inp["slot_drop"].sum()) if inp.get("slot_drop") is not None else 0)
    act_b = 1 if w4 else 2
    gemm1_flops = 4.0 * R * H * I
    gemm2_flops = 2.0 * R * H * I
    gather_bytes = T * H * act_b + R * H * act_b + 4 * T * k
    combine_bytes = R * H * 2 + T * H * 2 + 8 * T * k
    s = 1e-3
    gemm_ms = stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]
    tflops = lambda f, ms: f / (ms * s) / 1e12  # noqa: E731
    gbs = lambda b, ms: b / (ms * s) / 1e9  # noqa: E731

    if not w4:
        g1 = tflops(gemm1_flops, stage_ms["gemm1_swiglu"])
        roofline = {
            "kernel": "grouped_gemm_bf16_kernel<true> (GEMM1 + SwiGLU)",
            "bound": "mfma", "achieved": round(g1, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(g1 / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(["gemm1_swiglu"], cfg.name, T, args.seed),
            "algorithmic_per_launch": f"4*R*H*I = {gemm1_flops:.4g} flop (R={R} rows)",
        }
    else:
        # the W4A8 expert FFN streams the packed weights of every expert that has a row:
        # W1 codes 2I*H/2 + scales 2I*H/16 (MXFP4: /32), W2 codes H*I/2 + scales H*I/16 (/32) per expert,
        # plus activations in (R*H fp8 + scales), h round trip and y out; the weights dominate
        ids = np.argsort(-inp["logits"], axis=1, kind="stable")[:, :k]
        if inp.get("slot_drop") is not None:
            ids = np.where(inp["slot_drop"] == 1, -1, ids)
        n_exp = len(np.unique(ids[ids >= 0]))
        sb = 32 if mx else 16  # K values per weight block scale
        w_bytes = n_exp * (2 * I * H // 2 + 2 * I * H // sb + H * I // 2 + H * I // sb)
        act_bytes = R * H + R * (H // 128) * 4 + R * I * (4 + 4 + 1) + R * (I // 128) * 4 + R * H * 2
        ffn_bytes = w_bytes + act_bytes
        a = gbs(ffn_bytes, stage_ms["gemm1_swiglu"])
        roofline = {
            "kernel": "grouped W4A8 FFN (grouped_gemm_w4a8_kernel<true>, requant_fp8_kernel, "
                      "grouped_gemm_w4a8_kernel<false>)",
            "bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4),
            # the counters were taken on the default launches (not the single-launch kernel, nor
            # GEMM2 storing in slot order)
            "traffic": (None if flags else
                        measured_traffic(["gemm1_swiglu", "requant", "gemm2"], cfg.name, T, args.seed)),
            "algorithmic_per_launch": f"{ffn_bytes} bytes ({n_exp} experts' packed weights {w_bytes} B "
                                      f"+ activations {act_bytes} B)",
        }
    result = {
        "metric": METRIC,
        "value": round(T / (step_ms * s), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8xmxfp4" if mx else "fp8xfp4") if w4 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} H={H} I={I} E={cfg.E} top-{k}"
                               + (f", Zipf s={cfg.zipf_s} expert bias" if cfg.zipf_s else "")
                               + (f", interleave {cfg.glu_interleave}" if cfg.glu_interleave else "")
                               + (f", {cfg.drop_p:.0%} slots dropped" if cfg.drop_p else ""),
                   "T": T, "H": H, "I": I, "E": cfg.E, "k": k, "rows": R, "seed": args.seed},
        "tflops_forward": round(tflops(gemm1_flops + gemm2_flops, step_ms), 2),
        # W4A8 runs both GEMMs (and the h re-quantisation) inside the gemm1_swiglu stage
        "tflops_gemms": round(tflops(gemm1_flops + gemm2_flops, gemm_ms), 2),
        "mfma_frac_gemms": None if w4 else round(tflops(gemm1_flops + gemm2_flops, gemm_ms) / PEAK_BF16_TFLOPS, 4),
        "gemm2_tflops": None if w4 else round(tflops(gemm2_flops, stage_ms["gemm2"]), 2),
        # permute_kernel measured on its own (moe_permute_timed); the bf16 forward folds it into GEMM1
        "gather_ms": round(permute_gather_ms, 4),
        "gather_gbs": round(gbs(gather_bytes, permute_gather_ms), 1),
        "gather_hbm_frac": round(gbs(gather_bytes, permute_gather_ms) / PEAK_HBM_GBS, 4),
        "gather_after_forward_ms": round(permute_gather_after_fwd_ms, 4),
        "gather_after_forward_hbm_frac": round(gbs(gather_bytes, permute_gather_after_fwd_ms) / PEAK_HBM_GBS, 4),
        "gather_in_forward": ("folded into GEMM1 (x read through row_src)" if T * H * act_b < 2 ** 31
                              else "separate kernel"),
        "permute_tables_ms": round(permute_tables_ms, 4),
        "combine_gbs": round(gbs(combine_bytes, stage_ms["combine"]), 1),
        "combine_hbm_frac": round(gbs(combine_bytes, stage_ms["combine"]) / PEAK_HBM_GBS, 4),
        "stage_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
        "wall_ms_per_step": round(wall_ms, 4),
        "cold_cache_ms_per_step": round(cold_ms, 4),  # median, caches flushed before each forward
        "graph_ms_per_step": round(graph_ms, 4),  # median replay of one captured forward
        "graph_cold_ms_per_step": round(graph_cold_ms, 4),  # the same, caches flushed before each
        "weight_layout": (args.w4_layout if w4 else "rows"),
        # order of GEMM2's y rows: expert-major, or slot order (MOE_FLAG_SCATTER_Y)
        "y_order": "slot" if flags == tpg.MOE_FLAG_SCATTER_Y else "expert",
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not detail:
        for k_ in [k_ for k_ in result if k_.startswith("gather") or k_ == "permute_tables_ms"]:
            del result[k_]
    del d, wts, ws, out
    torch.cuda.empty_cache()
    return result, inp




if __name__ == "__main__":
    main()
