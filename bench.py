#!/usr/bin/env python3
"""Benchmark of the routed MoE SwiGLU FFN forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--mode auto]

One step = one whole forward pass (route -> GEMM1 + SwiGLU -> GEMM2 +
routing weight -> combine) over one batch of seeded synthetic inputs that are
resident in HBM before timing starts. W untimed steps, then K timed steps
bracketed by torch.cuda.synchronize(); rank 0 (the only rank) prints one JSON
line on stdout. The headline workload is the decode shape (T=64 tokens,
E=32 experts, top-8, D=6144, H=2048, bf16): one GPU's share of an 8-way
expert-parallel deployment, bound by streaming the expert weights from HBM.

The same line carries a "configs" object with the prefill-shaped workloads,
each timed the same way on inputs of its own: the mid prefill (T=4096,
D=2048, H=768, E=128, top-8) in the split and the fused pipeline, the large
prefill (T=131072, same dims, Zipf-skewed routing) and the MX-fp8 workload
(T=16384, D=4096, H=1536, E=64, top-6), each with its roofline fraction and a
CPU-oracle sample (--no-extra leaves them out).

Per-kernel durations come from HIP events that the library records on the
pass's own stream at its stage boundaries (moe_ffn_forward_events) during
the timed steps: every --event-every-th timed step (default 8, starting with
the first) carries the five events and the others run bare, because each
event record adds a gap to the stream. The dominant kernel's roofline
fraction uses its algorithmic bytes (weights of the experts hit +
activations in and out) or flops (6*P*D*H split 4:2 over the two GEMMs) per
launch, over the instrumented steps.

The CPU baseline is the oracle (oracle/, plain C, OpenMP), built for the
host with -O3 -march=native, timed on a bounded sample of the same workload
on all the host's cores (and, for the headline, on one core).
--cpu-plan runs the fuller CPU timing plan instead of the GPU bench: every
workload, median of 3 runs on the three smaller ones, one-thread runs of the
tiny and decode workloads.

After the timed steps, the same pass is captured once in a HIP graph and
replayed K times between one pair of events (`graph_replay_ms`: the mean
replay); this is reported beside `value`, which stays the eager rate
(--no-graph skips it).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE FFN fwd TFLOP/s + routed tokens/s; % of MFMA peak (prefill), % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0
# MXFP4 weights meet MX-fp8 activations in the scaled MFMA, which then runs at the fp8 rate.
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 5000.0}
STAGES = {"split": ["route", "gemm1_swiglu", "gemm2_weight", "combine"],
          "fused": ["route", "acc_fill", "fused_ffn", "acc_to_bf16"]}
# (workload id, mode) of the prefill-shaped workloads timed beside the headline
EXTRA = [(3, "split"), (3, "fused"), (4, "split"), (5, "split")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload id (1..5); 2 = decode")
    ap.add_argument("--mode", default="auto", choices=["auto", "split", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the headline's CPU-baseline sample")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the prefill-shaped workloads timed beside the headline")
    ap.add_argument("--extra-steps", type=int, default=20, help="timed steps of each extra workload")
    ap.add_argument("--cpu-plan", action="store_true",
                    help="time the CPU oracle on every workload (no GPU) and print one JSON line")
    ap.add_argument("--crossover", default="", metavar="T1,T2,...",
                    help="time both pipelines of the --config workload's dims at these token counts "
                         "(graph replays and stage events) and print one JSON line instead of the bench")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count T (crossover sweeps)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (PMC calibration)")
    ap.add_argument("--event-every", type=int, default=8, metavar="N",
                    help="record the stage events on every N-th timed step (1 = all)")
    ap.add_argument("--shared-ffn", type=int, default=0, metavar="HS",
                    help="add one shared expert of intermediate size HS on every token "
                         "(moe_ffn_forward_shared; bf16 only)")
    ap.add_argument("--mxfp4", action="store_true",
                    help="MXFP4 expert weights (e2m1 codes, e8m0 scale per 32; moe_ffn_mxfp4_quantize) "
                         "with MX-fp8 x and activations, on the chosen workload's dims")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing that follows the timed eager steps")
    ap.add_argument("--logits", action="store_true",
                    help="start each step from router logits (moe_ffn_forward_logits): the router's "
                         "softmax/top-k runs inside the timed pass, fused with the route step")
    return ap.parse_args(argv)


def hit_experts(ids: np.ndarray, E: int) -> int:
    flat = ids.reshape(-1)
    return int(np.unique(flat[(flat >= 0) & (flat < E)]).size)


def kernel_work(cfg, mode, hit, dtype):
    """Algorithmic bytes and flops per launch of each stage's kernel."""
    T, D, H, P = cfg.T, cfg.D, cfg.H, cfg.P
    e = 2 if dtype == "bf16" else 1                      # bytes per element of x and act
    we = {"bf16": 2, "mxfp8": 1, "mxfp4": 0.5}[dtype]    # bytes per weight element
    sc = 0.0 if dtype == "bf16" else 1.0 / 32            # e8m0 bytes per element
    w1 = hit * 2 * H * D * (we + sc)
    w2 = hit * D * H * (we + sc)
    x = T * D * (e + sc)
    act = P * H * (e + sc)
    if mode == "split":
        return {
            "route": (P * 4 * 3 + cfg.E * 8, 0.0),
            "gemm1_swiglu": (w1 + x + act, 4.0 * P * D * H),
            "gemm2_weight": (w2 + act + P * D * 2, 2.0 * P * D * H),
            "combine": (P * D * 2 + T * D * 2, 0.0),
        }
    return {
        "route": (P * 4 * 3 + cfg.E * 8, 0.0),
        "acc_fill": (T * D * 4, 0.0),
        "fused_ffn": (w1 + w2 + x + T * D * 4, 6.0 * P * D * H),
        "acc_to_bf16": (T * D * 6, 0.0),
    }


KERNEL_FILES = {"dma_kmajor_kernel": "gemm_skinny.hip",
                "dma_skinny_kernel": "gemm_skinny.hip",
                "mx_fused_kernel": "mx.hip", "fused_dma_kernel": "gemm_fused.hip",
                "mx_kmajor_kernel": "gemm_skinny.hip",
                "big_gemm_kernel": "gemm_big.hip",
                "mx_gemm1_kernel": "mx.hip", "mx_gemm2_kernel": "mx.hip", "fused_bf16_kernel": "gemm_bf16.hip",
                "gemm1_swiglu_kernel": "gemm_bf16.hip", "gemm2_weight_kernel": "gemm_bf16.hip",
                "combine_kernel": "gemm_bf16.hip"}


def _code_only(text: str) -> str:
    """C/C++ source with comments and blank space removed (string literals in
    these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(symbol: str) -> str:
    """Digest of the code (comments and spacing aside) of the source file
    defining `symbol` plus the shared headers it includes (common.h, and
    dma_ring.h for the DMA-ring kernels): a change to any of them
    invalidates counters stored for that kernel."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "grouped_gemm_amd", "csrc")
    kf = KERNEL_FILES.get(symbol, "")
    ring = "dma_ring.h" if kf in ("gemm_skinny.hip", "gemm_fused.hip") else ""
    for f in ("common.h", ring, kf):
        path = os.path.join(d, f)
        if f and os.path.isfile(path):
            h.update(f.encode())
            h.update(_code_only(open(path, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def kernel_symbol(cfg, mode, stage):
    """The HIP kernel a stage runs for this workload (the GEMM stages ask the
    library's own dispatch, moe_ffn_gemm_kernel)."""
    if mode == "fused" and stage == "route":
        return "route kernels (their extra blocks clear the accumulator)"
    if mode == "fused" and stage == "acc_fill":
        return "none (the route kernels clear the accumulator)"
    if mode == "fused" and stage == "acc_to_bf16":
        if kernel_symbol(cfg, mode, "fused_ffn") == "fused_dma_kernel":
            return "none (fused_dma_kernel converts each completed token row)"
        return "f32_to_bf16_kernel"
    if stage == "route":
        if cfg.P <= 256 and cfg.E <= 64:
            return "route_wave_kernel"
        return "route_small_kernel" if cfg.P <= 16384 and cfg.E <= 1024 else "route_* (4 kernels)"
    if stage == "combine":
        return "combine_kernel"
    # the library reports the kernel its dispatch picks for this shape
    import grouped_gemm_amd as g
    name = g.moe_ffn_gemm_kernel(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, cfg.dtype, mode,
                                 2 if stage == "gemm2_weight" else 1)
    return name.split("<")[0] if name else "unknown"


def measured_traffic(stage: str, symbol: str, workload: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current source of the kernel and the same workload; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.isfile(path):
        return None
    rec = json.load(open(path)).get(f"{workload}::{stage}")
    if not rec or rec.get("source_sha") != source_digest(symbol):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------- the CPU oracle, timed ----------------

def _oracle_forward(cfg, host, dtype, tok):
    import oracle
    if dtype == "bf16":
        oracle.forward_bf16(host["x"], host["w1"], host["w2"], host["topk_ids"], host["topk_weights"],
                            tokens=tok, shared=host.get("shared"))
    elif dtype == "mxfp4":
        oracle.forward_mx4(*host["xq"], *host["w1q"], *host["w2q"], host["topk_ids"], host["topk_weights"],
                           tokens=tok)
    else:
        oracle.forward_mx(*host["xq"], *host["w1q"], *host["w2q"], host["topk_ids"], host["topk_weights"],
                          tokens=tok)


def cpu_baseline(cfg, host, dtype, target_s, threads=None, repeats=1, max_tokens=None):
    """The oracle (native build) on the first n tokens of the workload, n grown
    until one run takes about target_s / 4 or more; then `repeats` runs of
    those n tokens (median reported) on `threads` threads (default: all)."""
    import oracle
    oracle.use_native_build()
    all_threads = oracle.num_threads()
    oracle.set_num_threads(threads or all_threads)
    used = oracle.num_threads()
    cap = min(cfg.T, max_tokens or cfg.T)
    n = min(cap, 2)
    try:
        while True:
            t0 = time.perf_counter()
            _oracle_forward(cfg, host, dtype, np.arange(n))
            dt = time.perf_counter() - t0
            if dt >= target_s / 4 or n == cap:
                break
            n = min(cap, max(n * 2, int(n * target_s / max(dt, 1e-3) * 0.9)))
        runs = [dt]
        for _ in range(repeats - 1):
            t0 = time.perf_counter()
            _oracle_forward(cfg, host, dtype, np.arange(n))
            runs.append(time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(all_threads)
    dt = statistics.median(runs)
    flops = 6.0 * n * cfg.k * cfg.D * cfg.H
    if host.get("shared") is not None:
        flops += 6.0 * n * cfg.D * host["shared"][1].shape[1]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens ({n * cfg.k} routed pairs) of the same workload, "
                      f"{'median of %d runs, ' % repeats if repeats > 1 else ''}{dt:.2f} s wall, fp32 accumulation",
            "seconds": dt, "runs_s": runs, "tokens": n, "tokens_per_s": n / dt,
            "routed_pairs_per_s": n * cfg.k / dt, "cpu_model": oracle.cpu_model(),
            "build": "gcc -O3 -march=native -fopenmp -ffp-contract=off"}


def cpu_plan():
    """Every workload's oracle timing on this host: median of 3 on the tiny,
    decode and mid prefill workloads (whole batches where they fit a few
    seconds), one run on a sample of the large prefill and the MX workload,
    and one-thread runs of the tiny and decode workloads."""
    import moe_inputs as mi
    import oracle
    plan = {1: dict(target=8.0, repeats=3, single=True), 2: dict(target=12.0, repeats=3, single=True),
            3: dict(target=12.0, repeats=3), 4: dict(target=30.0, repeats=1), 5: dict(target=30.0, repeats=1)}
    out = {}
    for cid, p in plan.items():
        cfg = mi.CONFIGS[cid]
        log(f"[cpu-plan] {cfg.name}: generating inputs")
        if cfg.dtype == "bf16":
            host = mi.make_bf16(cfg, 0)
        else:
            s = mi.make_mx_sources(cfg, 0)
            host = dict(topk_ids=s["topk_ids"], topk_weights=s["topk_weights"],
                        xq=oracle.mx_quantize(s["x"]), w1q=oracle.mx_quantize(s["w1"]),
                        w2q=oracle.mx_quantize(s["w2"]))
            del s
        log(f"[cpu-plan] {cfg.name}: timing")
        rec = {"all_threads": cpu_baseline(cfg, host, cfg.dtype, p["target"], repeats=p["repeats"])}
        if p.get("single"):
            rec["one_thread"] = cpu_baseline(cfg, host, cfg.dtype, p["target"] / 2, threads=1, repeats=1)
        out[cfg.name] = rec
        del host
    return {"kind": "cpu_oracle_plan", "cpu_model": oracle.cpu_model(), "nproc": os.cpu_count(),
            "workloads": out}


# ---------------- one workload on the GPU ----------------

def graph_replay_ms(step, n):
    """The same pass captured once in a HIP graph and replayed n times after the
    timed eager steps (not part of `value`), between one pair of events on the
    replaying stream: the mean replay time."""
    import torch
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
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    del graph
    return {"mean": ms, "replays": n}


class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def rows(self, n):
        out = []
        for _ in range(n):
            row = []
            for _ in range(5):
                e = ctypes.c_void_p()
                assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
                row.append(e.value)
            out.append(row)
        return out

    def elapsed(self, a, b):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, rows):
        for row in rows:
            for e in row:
                self.hip.hipEventDestroy(e)


def run_workload(cfg, mode_req, steps, warmup, event_every, hip, dev, shared_hs=0, use_logits=False,
                 want_graph=True, cpu_target=0.0, cpu_single=False, copy_mib=0):
    """Time one workload on the GPU; returns its result fields."""
    import torch
    import moe_inputs as mi
    import grouped_gemm_amd as g

    dtype = cfg.dtype
    log(f"[bench] generating {cfg.name} {dtype} inputs (seeded)")
    host = {}
    if dtype == "bf16":
        d = mi.make_bf16(cfg, 0)
        host.update(d)
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        w1 = torch.from_numpy(d["w1"].view(np.int16)).to(dev).view(torch.bfloat16)
        w2 = torch.from_numpy(d["w2"].view(np.int16)).to(dev).view(torch.bfloat16)
        scales = {}
    else:
        s = mi.make_mx_sources(cfg, 0)
        host.update(topk_ids=s["topk_ids"], topk_weights=s["topk_weights"])
        q = {}
        for n in ("x", "w1", "w2"):
            quant = g.moe_ffn_mxfp4_quantize if (dtype == "mxfp4" and n != "x") else g.moe_ffn_mx_quantize
            src = torch.from_numpy(s[n]).to(dev)
            q[n] = quant(src)
            del src
        torch.cuda.synchronize()
        x, w1, w2 = q["x"][0], q["w1"][0], q["w2"][0]
        scales = dict(x_scale=q["x"][1], w1_scale=q["w1"][1], w2_scale=q["w2"][1])
        if cpu_target > 0:
            host["xq"] = tuple(t.cpu().numpy() for t in q["x"])
            host["w1q"] = tuple(t.cpu().numpy() for t in q["w1"])
            host["w2q"] = tuple(t.cpu().numpy() for t in q["w2"])
        del s
    ids = torch.from_numpy(host["topk_ids"]).to(dev)
    wts = torch.from_numpy(host["topk_weights"]).to(dev)
    shared = None
    if shared_hs:
        host["shared"] = mi.shared_expert(cfg, shared_hs, 0)
        shared = tuple(torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16) for a in host["shared"])
    logits = None
    if use_logits:
        # the pass routes from these logits; ids / wts become its outputs
        host["logits"] = mi.router_logits(cfg, 0)
        logits = torch.from_numpy(host["logits"]).to(dev)
    mode_id = g.moe_ffn_resolve_mode(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dtype, mode_req)
    mode = {g.MOE_FFN_FUSED: "fused", g.MOE_FFN_SPLIT: "split"}[mode_id]
    nbytes = g.moe_ffn_workspace_bytes(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dtype, mode)
    if shared_hs:
        pr = g.make_problem(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dtype)
        nbytes = g.library().moe_ffn_shared_workspace_bytes(ctypes.byref(pr), shared_hs, mode_id)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if shared is not None:
            g.moe_ffn_forward_shared(x, w1, w2, ids, wts, shared[0], shared[1], out=out, mode=mode, workspace=ws,
                                     events=ev)
        elif logits is not None:
            g.moe_ffn_forward_logits(x, w1, w2, logits, cfg.k, out=out, mode=mode, workspace=ws, topk_ids=ids,
                                     topk_weights=wts, events=ev, **scales)
        else:
            g.moe_ffn_forward(x, w1, w2, ids, wts, out=out, mode=mode, workspace=ws, events=ev, **scales)

    events = hip.rows(steps)
    log(f"[bench] {cfg.name} mode={mode}: {warmup} warmup + {steps} timed steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i] if i % event_every == 0 else None)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3

    names = list(STAGES[mode])
    if logits is not None:
        names[0] = "router_route"
    if shared is not None:
        names[0] = "shared_expert_route"
    stage_ms = {n: 0.0 for n in names}
    timed = [events[i] for i in range(steps) if i % event_every == 0]
    for row in timed:
        for j, n in enumerate(names):
            stage_ms[n] += hip.elapsed(row[j], row[j + 1]) / len(timed)
    hip.destroy(events)

    graph_ms = None
    if want_graph and shared is None and logits is None:
        graph_ms = graph_replay_ms(step, steps)

    if copy_mib:
        a = torch.empty(copy_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if logits is not None:
        host["topk_ids"] = ids.cpu().numpy()  # the routes the timed passes took
    hit = hit_experts(host["topk_ids"], cfg.E)
    work = kernel_work(cfg, mode, hit, dtype)
    dom = max(names[1:], key=lambda n: stage_ms[n])
    dbytes, dflops = work[dom]
    dsec = stage_ms[dom] * 1e-3
    peak_tf = MFMA_PEAK_TFLOPS[dtype]
    intensity = dflops / dbytes if dbytes else 0.0
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    workload = f"{cfg.name} {dtype} T={cfg.T} D={cfg.D} H={cfg.H} E={cfg.E} k={cfg.k}"
    if logits is not None:
        workload += " from router logits"
    if shared is not None:
        workload += f" + shared expert Hs={shared_hs}"
    symbol = kernel_symbol(cfg, mode, dom)
    if intensity > ridge:
        roof = {"bound": "mfma", "achieved": dflops / dsec / 1e12, "peak": peak_tf, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dbytes / dsec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, symbol, workload)
    roof["kernel"] = dom
    roof["kernel_symbol"] = symbol
    roof["algorithmic_bytes"] = dbytes
    roof["algorithmic_flops"] = dflops
    roof["avg_launch_ms"] = stage_ms[dom]

    flops = cfg.flops + (6.0 * cfg.T * cfg.D * shared_hs if shared is not None else 0.0)
    tflops = flops / (ms * 1e-3) / 1e12
    all_bytes = hit * 3 * cfg.H * cfg.D * {"bf16": 2, "mxfp8": 1, "mxfp4": 0.5}[dtype] + 2 * cfg.T * cfg.D * 2
    res = {
        "workload": workload, "mode": mode, "dtype": dtype, "ms_per_step": ms, "tflops": tflops,
        "routed_tokens_per_s": cfg.P / (ms * 1e-3), "tokens_per_s": cfg.T / (ms * 1e-3),
        "pct_mfma_peak": tflops / peak_tf, "effective_hbm_gbs": all_bytes / (ms * 1e-3) / 1e9,
        "pct_hbm_peak": all_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stage_ms": stage_ms, "graph_replay_ms": graph_ms, "stage_events_every": event_every,
        "roofline": roof, "experts_hit": hit, "steps": steps, "warmup": warmup,
    }
    del x, w1, w2, ws, out, ids, wts, scales, shared, logits
    torch.cuda.empty_cache()
    if cpu_target > 0:
        log(f"[bench] timing the CPU oracle on a sample of {cfg.name}")
        if use_logits:
            import oracle
            host["topk_ids"], host["topk_weights"] = oracle.router(host["logits"], cfg.k)
        res["cpu_baseline"] = cpu_baseline(cfg, host, dtype, cpu_target)
        if cpu_single:
            res["cpu_baseline"]["one_thread"] = cpu_baseline(cfg, host, dtype, cpu_target / 4, threads=1)
    else:
        res["cpu_baseline"] = None
    return res


def main(argv=None):
    args = parse_args(argv)
    args.event_every = max(1, args.event_every)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU expert-parallel layout is a design note, not built)", file=sys.stderr)
        return 2
    if args.cpu_plan:
        print(json.dumps(cpu_plan()), flush=True)
        return 0
    import torch
    import moe_inputs as mi

    cfg = mi.CONFIGS[args.config]
    if args.tokens:
        cfg = mi.custom(args.tokens, cfg.D, cfg.H, cfg.E, cfg.k, cfg.routing, cfg.dtype, cid=cfg.cid,
                        name=f"{cfg.name}_T{args.tokens}")
    if args.mxfp4:
        cfg = mi.custom(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, cfg.routing, "mxfp4", cid=cfg.cid, name=cfg.name)
    if args.shared_ffn and (args.logits or cfg.dtype != "bf16"):
        print("bench.py: --shared-ffn runs the bf16 pass from given routes only", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    hip = HipEvents()
    if args.crossover:
        import grouped_gemm_amd as g
        rows = []
        for T in (int(t) for t in args.crossover.split(",")):
            c = mi.custom(T, cfg.D, cfg.H, cfg.E, cfg.k, cfg.routing, cfg.dtype, cid=cfg.cid, name=f"{cfg.name}_T{T}")
            row = {"T": T, "pairs": c.P}
            for mode in ("split", "fused"):
                r = run_workload(c, mode, args.steps, args.warmup, args.event_every, hip, dev)
                row[mode] = {"ms_per_step": r["ms_per_step"], "graph_replay_ms": r["graph_replay_ms"]["mean"],
                             "stage_ms": r["stage_ms"],
                             "kernel": g.moe_ffn_gemm_kernel(T, c.D, c.H, c.E, c.k, c.dtype, mode, 1)}
            row["auto"] = {g.MOE_FFN_FUSED: "fused", g.MOE_FFN_SPLIT: "split"}[
                g.moe_ffn_resolve_mode(T, c.D, c.H, c.E, c.k, c.dtype, "auto")]
            log(f"[crossover] T={T}: split {row['split']['graph_replay_ms']:.3f} ms, "
                f"fused {row['fused']['graph_replay_ms']:.3f} ms (graph replays)")
            rows.append(row)
        print(json.dumps({"kind": "crossover", "dims": f"D={cfg.D} H={cfg.H} E={cfg.E} k={cfg.k} {cfg.dtype}",
                          "routing": cfg.routing, "steps": args.steps, "rows": rows}), flush=True)
        return 0
    cpu = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    head = run_workload(cfg, args.mode, args.steps, args.warmup, args.event_every, hip, dev,
                        shared_hs=args.shared_ffn, use_logits=args.logits, want_graph=not args.no_graph,
                        cpu_target=cpu, cpu_single=True, copy_mib=args.copy_mib)

    result = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; routing, x and random-init expert weights of the stated shape)",
        "config": {"workload": head["workload"], "mode": head["mode"], "tokens": cfg.T, "experts": cfg.E,
                   "topk": cfg.k, "hidden": cfg.D, "ffn": cfg.H, "experts_hit": head["experts_hit"],
                   "parallelism": "single GPU"},
    }
    for key in ("routed_tokens_per_s", "tokens_per_s", "pct_mfma_peak", "effective_hbm_gbs", "pct_hbm_peak",
                "stage_ms", "graph_replay_ms", "stage_events_every", "roofline", "cpu_baseline"):
        result[key] = head[key]

    plain = not (args.tokens or args.mxfp4 or args.shared_ffn or args.logits or args.config != 2)
    if plain and not args.no_extra:
        extra = {}
        for cid, mode in EXTRA:
            c = mi.CONFIGS[cid]
            r = run_workload(c, mode, args.extra_steps, 3, 4, hip, dev, want_graph=not args.no_graph,
                             cpu_target=0.0 if args.no_cpu_baseline else 4.0)
            extra[f"{c.name}_{mode}"] = r
        result["configs"] = extra
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
