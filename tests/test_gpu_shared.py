"""The pass with one shared expert ("GC-MoE on SM120", section 4.7: a shared
expert on every token, added into the same fp32 sum as the routed slots) on
the GPU through the C ABI, against the CPU oracle with the same shared
expert: both pipelines, every GEMM path the shared pass can take (the
skinny kernel for up to 32 tokens, the prefill ring with 128- and 256-row
tiles, the generic kernel when D is not a multiple of 256), and the decode
and large prefill workloads with a shared expert of their own size."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import assert_close, bf16_to_gpu, gpu_bf16_to_f64, cover_sample, upload_bf16

pytestmark = pytest.mark.gpu


def _case(cfg, Hs, mode, tokens=None):
    import grouped_gemm_amd as g
    print(f"shared {cfg.name} Hs={Hs} mode={mode}", flush=True)
    d = mi.make_bf16(cfg, 0)
    ws1, ws2 = mi.shared_expert(cfg, Hs, 0)
    t = upload_bf16(d)
    out = g.moe_ffn_forward_shared(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], bf16_to_gpu(ws1),
                                   bf16_to_gpu(ws2), mode=mode)
    torch.cuda.synchronize()
    out = gpu_bf16_to_f64(out)
    ref = mi.bf16_bits_to_f32(oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"],
                                                  tokens=tokens, shared=(ws1, ws2))).astype(np.float64)
    if tokens is not None:
        out, ref = out[tokens], ref[tokens]
    rel, cos = assert_close(out, ref, what=f"{cfg.name}/shared/{mode}")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("T,D,H,E,k,Hs", [
    (64, 256, 512, 8, 2, 256),      # the tiny workload's shape
    (20, 256, 256, 4, 2, 384),      # shared pass on the skinny kernel (T <= 32)
    (300, 384, 256, 6, 3, 256),     # D not a multiple of 256: the generic GEMM kernels
    (500, 512, 384, 8, 2, 128),     # prefill ring, 128-row tiles
    (2100, 256, 256, 3, 2, 640),    # prefill ring, 256-row tiles; Hs > H
    (90, 192, 320, 4, 2, 192),      # D, H and Hs multiples of 64 only (generic kernels)
    (1024, 512, 256, 8, 2, 512),    # shared GEMM1 on the k-major decode kernel (32 m-tiles of one group)
])
def test_shared_expert_matches_oracle(mode, T, D, H, E, k, Hs):
    _case(mi.custom(T, D, H, E, k, "zipf"), Hs, mode)


@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("T,D,H,E,k,Hs", [
    (48, 512, 256, 8, 2, 256),      # fused: the decode-ring kernel writes the unrouted tokens' rows
    (300, 384, 256, 6, 3, 256),     # fused: the generic kernel and the conversion kernel
])
def test_shared_expert_with_unrouted_tokens(mode, T, D, H, E, k, Hs):
    """Tokens whose routes are all dropped receive the shared expert's row alone
    (the output starts as NaN, so every row must be written)."""
    import grouped_gemm_amd as g
    cfg = mi.custom(T, D, H, E, k, "uniform")
    print(f"shared + unrouted tokens {cfg.name} Hs={Hs} mode={mode}", flush=True)
    d = mi.make_bf16(cfg, 4)
    d["topk_ids"][::5, :] = -1                # every fifth token: no route reaches an expert
    d["topk_ids"][3, :] = E                   # == E: dropped as well
    d["topk_ids"][1::7, 0] = -1               # some tokens keep only part of their routes
    ws1, ws2 = mi.shared_expert(cfg, Hs, 4)
    t = upload_bf16(d)
    out = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    g.moe_ffn_forward_shared(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], bf16_to_gpu(ws1),
                             bf16_to_gpu(ws2), mode=mode, out=out)
    torch.cuda.synchronize()
    got = gpu_bf16_to_f64(out)
    ref = mi.bf16_bits_to_f32(oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"],
                                                  shared=(ws1, ws2))).astype(np.float64)
    rel, cos = assert_close(got, ref, what=f"{cfg.name}/shared+unrouted/{mode}")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


def test_shared_expert_decode():
    _case(mi.CONFIGS[2], 2048, "split")


def test_shared_expert_large_prefill_sampled():
    cfg = mi.CONFIGS[4]
    ids, _ = mi.routing(cfg, 0)
    _case(cfg, 768, "split", tokens=cover_sample(cfg, ids, "split", extra=8, dense_bm=256))


def test_shared_expert_rejects_mx_and_bad_sizes():
    import grouped_gemm_amd as g
    cfg = mi.custom(8, 256, 256, 4, 2, "softmax")
    d = upload_bf16(mi.make_bf16(cfg, 0))
    ws1 = torch.zeros((2 * 200, 256), dtype=torch.bfloat16, device="cuda")
    ws2 = torch.zeros((256, 200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.MoeFfnError):
        g.moe_ffn_forward_shared(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], ws1, ws2)
