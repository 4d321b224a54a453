#!/usr/bin/env python3
"""Benchmark of the routed MoE SwiGLU FFN forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--mode auto]

One step = one whole forward pass (route -> GEMM1 + SwiGLU -> GEMM2 +
routing weight -> combine) over one batch of seeded synthetic inputs that are
resident in HBM before timing starts. W untimed steps, then K timed steps
bracketed by torch.cuda.synchronize(); rank 0 (the only rank) prints one JSON
line on stdout. The default workload is the decode shape (T=64 tokens,
E=32 experts, top-8, D=6144, H=2048, bf16): one GPU's share of an 8-way
expert-parallel deployment, bound by streaming the expert weights from HBM.

Per-kernel durations come from HIP events that the library records on the
pass's own stream at its stage boundaries (moe_ffn_forward_events) during
the timed steps: every --event-every-th timed step (default 8, starting with
the first) carries the five events and the others run bare, because each
event record adds a gap to the stream (about 14 us per step on the decode
pass when every step carries them). The dominant kernel's roofline fraction
uses its algorithmic bytes (weights of the experts hit + activations in and
out) or flops (6*P*D*H split 4:2 over the two GEMMs) per launch, over the
instrumented steps.

The CPU baseline is the oracle (oracle/, plain C, OpenMP) timed on a bounded
sample of the same workload on the host's cores.

After the timed steps, the same pass is captured once in a HIP graph and
replayed K times (`graph_replay_ms`, median and mean of the replays); this
is reported beside `value`, which stays the eager rate (--no-graph skips it).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
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
                    help="target wall time of the CPU-baseline sample")
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


KERNEL_FILES = {"dma_split_kernel": "gemm_skinny.hip", "dma_skinny_kernel": "gemm_skinny.hip",
                "mx_fused_kernel": "mx.hip",
                "mx_skinny_kernel": "gemm_skinny.hip",
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
    defining `symbol` plus the shared header: a change to either invalidates
    counters stored for that kernel."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "grouped_gemm_amd", "csrc")
    for f in ("common.h", KERNEL_FILES.get(symbol, "")):
        path = os.path.join(d, f)
        if f and os.path.isfile(path):
            h.update(f.encode())
            h.update(_code_only(open(path, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def kernel_symbol(cfg, mode, stage):
    """The HIP kernel a stage runs for this workload (the GEMM stages ask the
    library's own dispatch, moe_ffn_gemm_kernel)."""
    if mode == "fused" and stage != "fused_ffn":
        return {"acc_fill": "fill_zero_f32_kernel", "acc_to_bf16": "f32_to_bf16_kernel",
                "route": "route kernels"}[stage]
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


def cpu_baseline(cfg, inputs, dtype, target_s):
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    order = np.arange(cfg.T)
    n = min(cfg.T, 2)
    while True:
        tok = order[:n]
        t0 = time.perf_counter()
        if dtype == "bf16":
            oracle.forward_bf16(inputs["x"], inputs["w1"], inputs["w2"], inputs["topk_ids"],
                                inputs["topk_weights"], tokens=tok, shared=inputs.get("shared"))
        elif dtype == "mxfp4":
            oracle.forward_mx4(*inputs["xq"], *inputs["w1q"], *inputs["w2q"], inputs["topk_ids"],
                               inputs["topk_weights"], tokens=tok)
        else:
            oracle.forward_mx(*inputs["xq"], *inputs["w1q"], *inputs["w2q"], inputs["topk_ids"],
                              inputs["topk_weights"], tokens=tok)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n == cfg.T:
            break
        n = min(cfg.T, max(n * 2, int(n * target_s / max(dt, 1e-3) * 0.9)))
    flops = 6.0 * n * cfg.k * cfg.D * cfg.H
    if inputs.get("shared") is not None:
        flops += 6.0 * n * cfg.D * inputs["shared"][1].shape[1]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens ({n * cfg.k} routed pairs) of the same workload, "
                      f"{dt:.2f} s wall, fp32 accumulation",
            "seconds": dt, "tokens_per_s": n / dt}


def graph_replay_ms(step, n):
    """The same pass captured once in a HIP graph and replayed n times after the
    timed eager steps (not part of `value`): median and mean of the replays,
    each bracketed by events on the replaying stream."""
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
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in marks:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in marks)
    del graph
    return {"median": t[len(t) // 2], "mean": sum(t) / len(t), "replays": n}


def main(argv=None):
    args = parse_args(argv)
    args.event_every = max(1, args.event_every)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU expert-parallel layout is a design note, not built)", file=sys.stderr)
        return 2
    import torch
    import moe_inputs as mi
    import grouped_gemm_amd as g

    cfg = mi.CONFIGS[args.config]
    if args.tokens:
        cfg = mi.custom(args.tokens, cfg.D, cfg.H, cfg.E, cfg.k, cfg.routing, cfg.dtype, cid=cfg.cid,
                        name=f"{cfg.name}_T{args.tokens}")
    if args.mxfp4:
        cfg = mi.custom(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, cfg.routing, "mxfp4", cid=cfg.cid, name=cfg.name)
    dtype = cfg.dtype
    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name} inputs (seeded)")
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
            q[n] = quant(torch.from_numpy(s[n]).to(dev))
        torch.cuda.synchronize()
        x, w1, w2 = q["x"][0], q["w1"][0], q["w2"][0]
        scales = dict(x_scale=q["x"][1], w1_scale=q["w1"][1], w2_scale=q["w2"][1])
        if not args.no_cpu_baseline:
            host["xq"] = tuple(t.cpu().numpy() for t in q["x"])
            host["w1q"] = tuple(t.cpu().numpy() for t in q["w1"])
            host["w2q"] = tuple(t.cpu().numpy() for t in q["w2"])
        del s
    ids = torch.from_numpy(host["topk_ids"]).to(dev)
    wts = torch.from_numpy(host["topk_weights"]).to(dev)
    shared = None
    if args.shared_ffn:
        if args.logits or dtype != "bf16":
            print("bench.py: --shared-ffn runs the bf16 pass from given routes only", file=sys.stderr)
            return 2
        host["shared"] = mi.shared_expert(cfg, args.shared_ffn, 0)
        shared = tuple(torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16) for a in host["shared"])
    logits = None
    if args.logits:
        # the pass routes from these logits; ids / wts become its outputs
        host["logits"] = mi.router_logits(cfg, 0)
        logits = torch.from_numpy(host["logits"]).to(dev)
    mode_id = g.moe_ffn_resolve_mode(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dtype, args.mode)
    mode = {g.MOE_FFN_FUSED: "fused", g.MOE_FFN_SPLIT: "split"}[mode_id]
    nbytes = g.moe_ffn_workspace_bytes(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dtype, mode)
    if args.shared_ffn:
        import ctypes as _ct
        pr = g.make_problem(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dtype)
        nbytes = g.library().moe_ffn_shared_workspace_bytes(_ct.byref(pr), args.shared_ffn, mode_id)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device=dev)

    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    events = []
    for _ in range(args.steps):
        row = []
        for _ in range(5):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            row.append(e.value)
        events.append(row)

    def step(ev=None):
        if shared is not None:
            g.moe_ffn_forward_shared(x, w1, w2, ids, wts, shared[0], shared[1], out=out, mode=mode, workspace=ws,
                                     events=ev)
        elif logits is not None:
            g.moe_ffn_forward_logits(x, w1, w2, logits, cfg.k, out=out, mode=mode, workspace=ws, topk_ids=ids,
                                     topk_weights=wts, events=ev, **scales)
        else:
            g.moe_ffn_forward(x, w1, w2, ids, wts, out=out, mode=mode, workspace=ws, events=ev, **scales)

    log(f"[bench] {cfg.name} mode={mode}: {args.warmup} warmup + {args.steps} timed steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i] if i % args.event_every == 0 else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3

    names = list(STAGES[mode])
    if logits is not None:
        names[0] = "router_route"
    if shared is not None:
        names[0] = "shared_expert_route"
    stage_ms = {n: 0.0 for n in names}
    f = ctypes.c_float()
    timed = [events[i] for i in range(args.steps) if i % args.event_every == 0]
    for row in timed:
        for j, n in enumerate(names):
            assert hip.hipEventElapsedTime(ctypes.byref(f), row[j], row[j + 1]) == 0
            stage_ms[n] += f.value / len(timed)
    for row in events:
        for e in row:
            hip.hipEventDestroy(e)

    graph_ms = None
    if not args.no_graph and shared is None and logits is None:
        graph_ms = graph_replay_ms(step, args.steps)

    if args.copy_mib:
        a = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

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
        workload += f" + shared expert Hs={args.shared_ffn}"
    traffic = measured_traffic(dom, kernel_symbol(cfg, mode, dom), workload)
    if intensity > ridge:
        roof = {"bound": "mfma", "achieved": dflops / dsec / 1e12, "peak": peak_tf, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dbytes / dsec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["kernel_symbol"] = kernel_symbol(cfg, mode, dom)
    roof["algorithmic_bytes"] = dbytes
    roof["algorithmic_flops"] = dflops
    roof["avg_launch_ms"] = stage_ms[dom]

    flops = cfg.flops + (6.0 * cfg.T * cfg.D * args.shared_ffn if shared is not None else 0.0)
    tflops = flops / (ms * 1e-3) / 1e12
    all_bytes = hit * 3 * cfg.H * cfg.D * {"bf16": 2, "mxfp8": 1, "mxfp4": 0.5}[dtype] + 2 * cfg.T * cfg.D * 2
    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; routing, x and random-init expert weights of the stated shape)",
        "config": {"workload": workload, "mode": mode, "tokens": cfg.T, "experts": cfg.E,
                   "topk": cfg.k, "hidden": cfg.D, "ffn": cfg.H, "experts_hit": hit,
                   "parallelism": "single GPU"},
        "routed_tokens_per_s": cfg.P / (ms * 1e-3),
        "tokens_per_s": cfg.T / (ms * 1e-3),
        "pct_mfma_peak": tflops / peak_tf,
        "effective_hbm_gbs": all_bytes / (ms * 1e-3) / 1e9,
        "stage_ms": stage_ms,
        "graph_replay_ms": graph_ms,
        "stage_events_every": args.event_every,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        if logits is not None:
            import oracle
            host["topk_ids"], host["topk_weights"] = oracle.router(host["logits"], cfg.k)
        result["cpu_baseline"] = cpu_baseline(cfg, host, dtype, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
