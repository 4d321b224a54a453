"""The activation variant on the GPU through the C ABI ("Porting Block-Scaled
GEMM Kernels from Blackwell to Rubin", section 5.3: per-expert scale alpha,
gpt-oss style clamp; "GC-MoE on SM120", section 4.8: the route weight before
the activation) against the CPU oracle's variant, on every GEMM path of the
split pipeline: the skinny kernels (few rows per expert), the prefill ring
with 128- and 256-row tiles (including many tiles per workgroup, where the
GEMM1 row weights travel through the ring's hand-over), and the generic
kernels (D not a multiple of 256)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import assert_close, gpu_bf16_to_f64, cover_sample, to_gpu, upload_bf16

pytestmark = pytest.mark.gpu

VARIANTS = [  # (kind, limit, alpha, weight_before_act)
    (1, 0.5, False, False),
    (1, 0.7, True, True),
    (0, 0.0, True, False),
    (0, 0.0, False, True),
]


def _case(cfg, kind, limit, use_alpha, wba, tokens=None):
    import grouped_gemm_amd as g
    print(f"act {cfg.name} kind={kind} limit={limit} alpha={use_alpha} wba={wba}", flush=True)
    d = mi.make_bf16(cfg, 0)
    alpha = None
    if use_alpha:
        alpha = np.random.default_rng([cfg.E, 9]).uniform(0.5, 2.0, cfg.E).astype(np.float32)
    t = upload_bf16(d)
    out = g.moe_ffn_forward_act(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], kind=kind, limit=limit,
                                alpha=None if alpha is None else to_gpu(alpha), weight_before_act=wba)
    torch.cuda.synchronize()
    out = gpu_bf16_to_f64(out)
    ref = mi.bf16_bits_to_f32(oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"],
                                                      kind, limit, alpha, wba, tokens=tokens)).astype(np.float64)
    if tokens is not None:
        out, ref = out[tokens], ref[tokens]
    rel, cos = assert_close(out, ref, what=f"{cfg.name}/act")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (64, 256, 512, 8, 2, "softmax"),      # skinny kernels
    (40, 2048, 768, 128, 8, "zipf"),      # k-major decode kernels (gate/up rows interleaved)
    (300, 384, 256, 6, 3, "zipf"),        # generic kernels (D = 384)
    (500, 512, 384, 8, 2, "zipf"),        # prefill ring, 128-row tiles
    (2100, 256, 512, 3, 2, "zipf"),       # prefill ring, 256-row tiles
    (97, 192, 320, 6, 3, "softmax"),      # D and H multiples of 64 only
])
def test_variant_matches_oracle(T, D, H, E, k, routing, variant):
    _case(mi.custom(T, D, H, E, k, routing), *variant)


@pytest.mark.parametrize("variant", VARIANTS[:2])
def test_variant_many_tiles_per_workgroup(variant, monkeypatch):
    monkeypatch.setenv("MOE_FFN_GRID_LIMIT", "8")
    _case(mi.custom(2100, 512, 768, 3, 2, "zipf"), *variant)


def test_variant_decode_and_large_prefill():
    _case(mi.CONFIGS[2], 1, 0.5, True, True)
    cfg = mi.CONFIGS[4]
    ids, _ = mi.routing(cfg, 0)
    _case(cfg, 1, 0.5, True, True, tokens=cover_sample(cfg, ids, "split", extra=8))
