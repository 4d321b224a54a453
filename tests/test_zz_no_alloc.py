"""moe_ffn_forward_noalloc (the pass on the library's static scratch array,
for callers that cannot allocate) through the C ABI against moe_ffn_forward
on the same inputs: two calls in a row, the second on a smaller problem, in
both pipelines, and the oracle on both; a problem too large for the array is
refused before anything runs."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import assert_close, gpu_bf16_to_f64, upload_bf16

pytestmark = pytest.mark.gpu


def _ref(d):
    r = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    return mi.bf16_bits_to_f32(r).astype(np.float64)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_noalloc_matches_forward_on_two_calls(mode):
    import grouped_gemm_amd as g
    cases = [mi.CONFIGS[2], mi.custom(300, 256, 384, 8, 3, "zipf")]   # the second call is smaller
    for i, cfg in enumerate(cases):
        print(f"noalloc call {i}: {cfg.name} mode={mode}", flush=True)
        d = mi.make_bf16(cfg, 4)
        t = upload_bf16(d)
        want = g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], mode=mode)
        out = torch.full((cfg.T, cfg.D), 3.0, dtype=torch.bfloat16, device="cuda")
        g.moe_ffn_forward_noalloc(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], out, mode=mode)
        torch.cuda.synchronize()
        got, ref = gpu_bf16_to_f64(out), gpu_bf16_to_f64(want)
        if mode == "split":           # the same deterministic kernels: bit-identical
            assert np.array_equal(got, ref)
        assert_close(got, ref, what=f"noalloc vs forward/{mode}/{i}")
        rel, cos = assert_close(got, _ref(d), what=f"noalloc vs oracle/{mode}/{i}")
        print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


def test_noalloc_refuses_a_problem_beyond_the_array():
    import grouped_gemm_amd as g
    cfg = mi.CONFIGS[3]                                   # split workspace ~190 MB > 64 MiB
    assert g.moe_ffn_workspace_bytes(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, "bf16", "split") > g.MOE_FFN_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((cfg.T, cfg.D), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((cfg.E, 2 * cfg.H, cfg.D), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((cfg.E, cfg.D, cfg.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    out = torch.full((cfg.T, cfg.D), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.MoeFfnError) as e:
        g.moe_ffn_forward_noalloc(x, w1, w2, ids, w, out, mode="split")
    assert e.value.code == g.MOE_FFN_ESCRATCH
    torch.cuda.synchronize()
    assert torch.all(out.float() == 5.0)                 # nothing ran
