"""The forward pass captured once in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capturing stream) and replayed.

The library enqueues only its own kernels on the caller's stream (no memset,
no allocation, no host synchronization), so the whole pass can be captured.
Each replay here runs after eager work and synchronizations of the test's
own, with new inputs copied into the captured buffers beforehand, and must
give what an eager call on the same inputs gives: bit for bit on the split
pipeline (no atomics), within the oracle's tolerance on the fused one (fp32
atomics make its last bits order-dependent)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import assert_close, bf16_to_gpu, gpu_bf16_to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _load(dst: dict, d: dict):
    """Copy a seeded host case into the captured GPU buffers."""
    dst["x"].copy_(bf16_to_gpu(d["x"]))
    dst["w1"].copy_(bf16_to_gpu(d["w1"]))
    dst["w2"].copy_(bf16_to_gpu(d["w2"]))
    dst["ids"].copy_(to_gpu(d["topk_ids"]))
    dst["wts"].copy_(to_gpu(d["topk_weights"]))


def _graph_case(cfg, mode, seeds=(3, 4, 5), mutate=None):
    import grouped_gemm_amd as g
    print(f"graph {cfg.name} T={cfg.T} D={cfg.D} H={cfg.H} E={cfg.E} k={cfg.k} mode={mode}", flush=True)
    dev = torch.device("cuda:0")
    d0 = mi.make_bf16(cfg, 0)
    buf = dict(x=bf16_to_gpu(d0["x"]), w1=bf16_to_gpu(d0["w1"]), w2=bf16_to_gpu(d0["w2"]),
               ids=to_gpu(d0["topk_ids"]), wts=to_gpu(d0["topk_weights"]))
    nbytes = g.moe_ffn_workspace_bytes(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, "bf16", mode)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    ws_eager = torch.empty_like(ws)
    out_eager = torch.empty_like(out)

    def fwd(o, w):
        g.moe_ffn_forward(buf["x"], buf["w1"], buf["w2"], buf["ids"], buf["wts"], out=o, mode=mode, workspace=w)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(out, ws)                       # the warm-up call torch asks for before a capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(out, ws)
    torch.cuda.synchronize()

    for i, seed in enumerate(seeds):
        d = mi.make_bf16(cfg, seed)
        if mutate is not None:
            mutate(i, d)
        _load(buf, d)
        # eager work of the program's own between replays: the same pass eagerly,
        # on other output and workspace buffers
        fwd(out_eager, ws_eager)
        torch.cuda.synchronize()
        out.fill_(float("nan"))            # a replay must overwrite every element
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, want = gpu_bf16_to_f64(out), gpu_bf16_to_f64(out_eager)
        if mode == "split":
            assert np.array_equal(out.view(torch.int16).cpu().numpy(), out_eager.view(torch.int16).cpu().numpy()), \
                f"replay {i} differs from the eager pass"
        else:
            assert np.isfinite(got).all()
            assert_close(got, want, what=f"replay {i} vs eager")
        ref = mi.bf16_bits_to_f32(oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"],
                                                      d["topk_weights"])).astype(np.float64)
        rel, cos = assert_close(got, ref, what=f"replay {i} vs oracle")
        print(f"  replay {i}: max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)
    del graph


@pytest.mark.parametrize("T,D,H,E,k,routing,mode", [
    (64, 512, 512, 8, 2, "softmax", "split"),     # decode kernels (<= 32 rows per expert)
    (300, 384, 640, 16, 4, "zipf", "split"),      # generic tiles, ragged
    (2100, 256, 384, 3, 2, "zipf", "split"),      # prefill kernels and their m-tile table
    (37, 256, 256, 5, 3, "softmax", "fused"),     # fused pipeline (fp32 atomics, then the conversion)
])
def test_forward_graph_replays_match_eager(T, D, H, E, k, routing, mode):
    _graph_case(mi.custom(T, D, H, E, k, routing), mode)


def test_graph_replays_follow_the_routing():
    """One capture, replays whose routing differs in how many m-tiles it makes:
    the decode kernels read the m-tile count the route step produces and deal
    their blocks out on the device, so a replay with a hot expert (two 32-row
    m-tiles) must match an eager pass as bit-exactly as one without."""
    def hot(i, d):
        if i % 2 == 1:  # replays 1 (and 3): expert 5 takes 56 of the 64 tokens
            ids = d["topk_ids"]
            sel = np.arange(ids.shape[0]) < 56
            ids[sel, 0] = 5
            ids[sel, 1:] = np.where(ids[sel, 1:] == 5, 6, ids[sel, 1:])
    _graph_case(mi.custom(64, 512, 512, 16, 4, "uniform"), "split", seeds=(3, 4, 5, 6), mutate=hot)
