"""bf16 forward pass on the GPU through the C ABI against the CPU oracle:
both pipelines, tiny to full-size workloads, ragged tiles and edge cases."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import (assert_close, gpu_bf16_to_f64, cover_sample, to_gpu, upload_bf16,
                          bf16_to_gpu)

pytestmark = pytest.mark.gpu

MODES = ["split", "fused"]


def _run(d, mode):
    """The pass into an output that starts as NaN, so a row the pass leaves
    unwritten fails the comparison."""
    import grouped_gemm_amd as g
    t = upload_bf16(d)
    T, D = d["x"].shape
    out = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], out=out, mode=mode)
    torch.cuda.synchronize()
    return gpu_bf16_to_f64(out)


def _ref(d, tokens=None):
    r = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"],
                            tokens=tokens)
    return mi.bf16_bits_to_f32(r).astype(np.float64)


def _case(cfg, mode, tokens=None, seed=0):
    print(f"forward {cfg.name} T={cfg.T} D={cfg.D} H={cfg.H} E={cfg.E} k={cfg.k} mode={mode}",
          flush=True)
    d = mi.make_bf16(cfg, seed)
    out = _run(d, mode)
    ref = _ref(d, tokens)
    if tokens is not None:
        out, ref = out[tokens], ref[tokens]
    rel, cos = assert_close(out, ref, what=f"{cfg.name}/{mode}")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


@pytest.mark.parametrize("mode", MODES)
def test_tiny_config(mode):
    _case(mi.CONFIGS[1], mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (37, 256, 256, 5, 3, "softmax"),        # one ragged m-tile per expert
    (300, 384, 640, 16, 4, "zipf"),         # several m-tiles, ragged tails, skew
    (1, 128, 128, 4, 2, "uniform"),         # a single token
    (513, 128, 256, 3, 3, "uniform"),       # k = E: every token on every expert
    (260, 256, 128, 1, 1, "softmax"),       # E = 1, k = 1: a dense SwiGLU FFN
    (500, 512, 384, 8, 2, "zipf"),          # prefill tiles of 128 rows, ragged, skewed
    (2100, 256, 384, 3, 2, "zipf"),         # prefill tiles of 256 rows, ragged, skewed
    (97, 192, 320, 6, 3, "softmax"),        # D and H multiples of 64 only
    (640, 320, 192, 5, 2, "zipf"),          # the same, several m-tiles per expert
    (7, 64, 64, 4, 2, "uniform"),           # the smallest dims
])
def test_ragged_shapes(mode, T, D, H, E, k, routing):
    _case(mi.custom(T, D, H, E, k, routing), mode)


@pytest.mark.parametrize("mode", MODES)
def test_all_tokens_on_one_expert(mode):
    cfg = mi.custom(400, 256, 256, 8, 2, "softmax")
    d = mi.make_bf16(cfg, 1)
    d["topk_ids"][:, 0] = 6
    d["topk_ids"][:, 1] = 2
    out = _run(d, mode)
    assert_close(out, _ref(d), what=f"one-expert/{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_dropped_and_zero_weight_routes(mode):
    cfg = mi.custom(200, 256, 256, 8, 4, "uniform")
    d = mi.make_bf16(cfg, 2)
    d["topk_ids"][::3, 1] = -1
    d["topk_ids"][1::5, 2] = 8           # == E: dropped
    d["topk_weights"][::4, 3] = 0.0
    d["topk_ids"][7, :] = -1             # a token with no route at all -> zeros
    out = _run(d, mode)
    ref = _ref(d)
    assert np.all(out[7] == 0)
    assert_close(out, ref, what=f"dropped/{mode}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,D,H,E,k", [
    (64, 512, 512, 16, 4),     # decode kernels: the route leaves no m-tile, every block of the grid exits
    (2100, 256, 384, 3, 2),    # prefill kernels: an empty tile table
])
def test_every_route_dropped(mode, T, D, H, E, k):
    """Every id out of range: no pair reaches an expert, and the output is all zeros
    (it is still written in full: it starts as NaN here)."""
    import grouped_gemm_amd as g
    d = mi.make_bf16(mi.custom(T, D, H, E, k, "uniform"), 9)
    d["topk_ids"][:, :] = -1
    d["topk_ids"][::2, 0] = E               # == E: dropped as well
    t = upload_bf16(d)
    out = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], out=out, mode=mode)
    torch.cuda.synchronize()
    assert np.all(gpu_bf16_to_f64(out) == 0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,D,H,E,k", [
    (40, 256, 256, 1000, 4),    # the decode kernels' m-tile lookup in two rounds (64 and more experts)
    (16, 256, 128, 4100, 4),    # past 4095 experts: the lookup falls back to the binary search
])
def test_many_experts(mode, T, D, H, E, k):
    """Decode-shaped passes over many experts, most of them without a routed row."""
    import grouped_gemm_amd as g
    assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "bf16", mode, 1) == (
        "fused_dma_kernel" if mode == "fused" else "dma_kmajor_kernel")
    _case(mi.custom(T, D, H, E, k, "uniform"), mode)


@pytest.mark.parametrize("mode", MODES)
def test_decode_config_full(mode):
    _case(mi.CONFIGS[2], mode)


@pytest.mark.parametrize("mode", MODES)
def test_mid_prefill_sampled(mode):
    cfg = mi.CONFIGS[3]
    ids, _ = mi.routing(cfg)
    _case(cfg, mode, tokens=cover_sample(cfg, ids, mode, extra=64))


def test_large_prefill_sampled():
    cfg = mi.CONFIGS[4]
    ids, _ = mi.routing(cfg)
    _case(cfg, "split", tokens=cover_sample(cfg, ids, "split", extra=32))


@pytest.mark.parametrize("T,D,H,E,k", [
    (2100, 256, 128, 3, 2),     # short K in GEMM2: hand-over after the ring drains
    (2100, 512, 384, 3, 2),     # hand-over inside the ring
    (500, 512, 384, 8, 2),      # 128-row tiles
])
def test_prefill_many_tiles_per_workgroup(T, D, H, E, k, monkeypatch):
    # with 8 workgroups each one walks many tiles, so the cross-tile hand-over runs
    monkeypatch.setenv("MOE_FFN_GRID_LIMIT", "8")
    _case(mi.custom(T, D, H, E, k, "zipf"), "split")


def test_prefill_descriptor_reload(monkeypatch):
    # 8 workgroups x more than 512 tiles each: the tile descriptors are reloaded
    monkeypatch.setenv("MOE_FFN_GRID_LIMIT", "8")
    cfg = mi.custom(65536, 256, 4096, 2, 1, "uniform")
    ids, _ = mi.routing(cfg)
    _case(cfg, "split", tokens=cover_sample(cfg, ids, "split", extra=16))


def test_split_is_deterministic():
    import grouped_gemm_amd as g
    d = mi.make_bf16(mi.custom(700, 256, 384, 16, 4, "zipf"), 3)
    t = upload_bf16(d)
    a = g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], mode="split")
    b = g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], mode="split")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_out_is_overwritten_and_int64_ids_accepted():
    import grouped_gemm_amd as g
    d = mi.make_bf16(mi.CONFIGS[1], 4)
    t = upload_bf16(d)
    ref = _ref(d)
    for mode in MODES:
        out = torch.full((64, 256), 7.0, dtype=torch.bfloat16, device="cuda")
        g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"].long(), t["topk_weights"],
                          out=out, mode=mode)
        torch.cuda.synchronize()
        assert_close(gpu_bf16_to_f64(out), ref, what=mode)


def test_empty_batch_is_a_noop():
    import grouped_gemm_amd as g
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((4, 256, 256), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((4, 256, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    out = g.moe_ffn_forward(x, w1, w2, ids, w, mode="split")
    assert out.shape == (0, 256)


def _duplicate_ids(ids):
    """The same expert in several slots of one token: such routes count once
    per slot (the sum over the token's slots runs over slots, not experts)."""
    ids = ids.copy()
    k = ids.shape[1]
    ids[::2, 1] = ids[::2, 0]
    ids[::3, k - 1] = ids[::3, 0]
    ids[5, :] = ids[5, 0]                # one token with every slot on one expert
    return ids


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,D,H,E,k,kernel", [
    (32, 512, 512, 8, 3, "dma_kmajor_kernel"),      # decode kernels
    (40, 2048, 768, 128, 8, "dma_kmajor_kernel"),   # decode kernels, more m-tiles than row-group pairs per CU
    (500, 512, 384, 8, 2, "big_gemm_kernel<128>"),  # prefill ring, 128-row tiles
    (2100, 256, 384, 3, 2, "big_gemm_kernel<256>"), # prefill ring, 256-row tiles
    (300, 384, 256, 6, 3, "gemm1_swiglu_kernel"),   # generic kernels
])
def test_duplicate_expert_ids(mode, T, D, H, E, k, kernel):
    import grouped_gemm_amd as g
    cfg = mi.custom(T, D, H, E, k, "zipf")
    assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "bf16", "split", 1) == kernel
    print(f"forward duplicate ids {cfg.name} mode={mode}", flush=True)
    d = mi.make_bf16(cfg, 6)
    d["topk_ids"] = _duplicate_ids(d["topk_ids"])
    rel, cos = assert_close(_run(d, mode), _ref(d), what=f"duplicates/{mode}")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


def test_side_stream_with_int64_ids():
    """The pass on a caller's side stream: the wrapper's own temporaries (the
    int32 ids, the workspace) are made on that stream after the current
    stream's work, and the result matches the oracle."""
    import grouped_gemm_amd as g
    d = mi.make_bf16(mi.custom(300, 256, 256, 8, 4, "zipf"), 7)
    ref = _ref(d)
    t = upload_bf16(d)
    side = torch.cuda.Stream()
    for mode in MODES:
        ids64 = t["topk_ids"].long()         # produced on the current stream
        out = g.moe_ffn_forward(t["x"], t["w1"], t["w2"], ids64, t["topk_weights"], mode=mode, stream=side)
        side.synchronize()
        assert_close(gpu_bf16_to_f64(out), ref, what=f"side stream/{mode}")


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (2100, 256, 512, 3, 2, "zipf"),     # many 32-row m-tiles per expert, ragged last tiles (64-wide slices)
    (96, 512, 768, 16, 4, "softmax"),   # twelve 64-wide slices of H, two W2 row groups
    (1, 256, 256, 4, 2, "uniform"),     # a single token
    (64, 256, 256, 4, 4, "uniform"),    # k = E
    (4096, 256, 512, 8, 2, "zipf"),     # enough m-tiles for 256-wide slices
    (40, 2048, 768, 128, 8, "zipf"),    # 128-wide slices, hot experts with several m-tiles
    (16, 2048, 768, 128, 8, "uniform"), # 256-wide slices, three of them
])
def test_fused_decode_kernel(T, D, H, E, k, routing):
    """The fused pass on the decode kernels' rings (32-row m-tiles, act slice in
    LDS, split-K down projection added into the fp32 accumulator, each token's
    row converted by the block that adds its last partial; the slice width
    follows the expected block count)."""
    import grouped_gemm_amd as g
    assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "bf16", "fused", 1) == "fused_dma_kernel"
    _case(mi.custom(T, D, H, E, k, routing), "fused")


@pytest.mark.parametrize("T,D,H,E,k,routing,gemms", [
    (64, 1664, 512, 32, 8, "softmax", (2,)),     # GEMM2: 13 row groups per block, super-groups of 7 and 6
    (64, 512, 1664, 32, 8, "uniform", (1,)),     # GEMM1: the same plan on gate/up rows
    (64, 3200, 256, 64, 8, "uniform", (2,)),     # GEMM2: 25 groups (9 + 8 + 8), one K chunk per group
    (2048, 256, 512, 1, 1, "softmax", (1,)),     # GEMM1: 64 m-tiles of one expert, 4 groups per block
    (1024, 1024, 256, 1, 1, "softmax", (2,)),    # GEMM2: 32 m-tiles of one expert, rotated group order
    (40, 2048, 768, 128, 8, "zipf", (1, 2)),     # both GEMMs, skewed: hot experts hold several m-tiles
    (16, 2048, 768, 128, 8, "uniform", (1, 2)),  # both GEMMs, 128 tokens' routes over 128 experts
    (64, 2048, 1024, 32, 8, "zipf", (1, 2)),     # skewed: the extra m-tiles share the CUs with the rest
    (64, 256, 256, 512, 8, "uniform", (1, 2)),   # more m-tiles than CUs: a block per m-tile, all its groups
])
def test_kmajor_decode_kernel(T, D, H, E, k, routing, gemms):
    """The k-major decode GEMMs (token chunk fetched once per K chunk and
    reused across a block's row groups; rows split over the waves; GEMM1's
    gate and up rows interleaved per 16-row block; the work dealt out on the
    device from the real m-tile count) through every super-group plan and
    work split: minimum size, uneven sizes, several m-tiles per expert, more
    m-tiles than compute units."""
    import grouped_gemm_amd as g
    for gemm in gemms:
        assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "bf16", "split", gemm) == "dma_kmajor_kernel"
    _case(mi.custom(T, D, H, E, k, routing), "split")


def test_skewed_decode_batch():
    """A decode-shaped batch whose routing is skewed: expert 5 takes 56 or more of
    the 64 tokens, so it holds two 32-row m-tiles and the other experts few rows.
    The dispatch sees the shape only, so the decode kernels run, with the
    extra m-tiles of the hot expert."""
    import grouped_gemm_amd as g
    cfg = mi.custom(64, 512, 512, 16, 4, "uniform")
    assert g.moe_ffn_gemm_kernel(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, "bf16", "split", 1) == "dma_kmajor_kernel"
    assert g.moe_ffn_gemm_kernel(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, "bf16", "split", 2) == "dma_kmajor_kernel"
    d = mi.make_bf16(cfg, 8)
    ids = d["topk_ids"]
    hot = np.arange(64) < 56
    ids[hot, 0] = 5
    ids[hot, 1:] = np.where(ids[hot, 1:] == 5, 6, ids[hot, 1:])   # expert 5 once per hot token
    assert mi.expert_histogram(ids, cfg.E)[5] >= 56
    for mode in MODES:
        rel, cos = assert_close(_run(d, mode), _ref(d), what=f"skewed decode/{mode}")
        print(f"  {mode}: max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)
