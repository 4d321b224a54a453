"""MXFP4-weight path on the GPU ("GC-MoE on SM120", scale formats: E2M1
weights with a UE8M0 exponent per 32 along K, MX-fp8 activations): the fp4
quantizer must equal the oracle's MXQ4 bit for bit, and the forward pass
must match the oracle's fp4-weight forward within the MX tolerance.

Each side quantizes the same fp32 sources with its own quantizers (e4m3 for
x, e2m1 for the weights); the GPU forward consumes the GPU's codes and the
oracle its own, after the test has checked that the codes are identical."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import MX_COS, MX_TOL, assert_close, gpu_bf16_to_f64, cover_sample, to_gpu

pytestmark = pytest.mark.gpu


def _quant4_gpu(src: np.ndarray):
    import grouped_gemm_amd as g
    c, s = g.moe_ffn_mxfp4_quantize(to_gpu(src.astype(np.float32)))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _quant8_gpu(src: np.ndarray):
    import grouped_gemm_amd as g
    c, s = g.moe_ffn_mx_quantize(to_gpu(src.astype(np.float32)))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def test_mxfp4_quantizer_bit_exact_random_and_edges():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal((512, 256)) * np.exp(rng.normal(0, 4, (512, 1)))).astype(np.float32)
    a[0] = 0.0                                        # all-zero blocks
    a[1, :32] = 6.0                                   # amax exactly 6 * 2^0
    a[2, :32] = np.float32(6.0 * 2.0 ** -20)
    a[3] = -a[3]
    a[4, 5] = 1e30                                    # huge amax in one block
    a[5] = 1e-40                                      # subnormal inputs
    a[6, :32] = -0.0                                  # signed zeros
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mids = [(mags[i] + mags[i + 1]) / 2 for i in range(7)]
    a[7, :32] = 6.0                                   # scale 0, so the block holds the exact ties
    a[7, 1:8] = mids
    a[7, 8:15] = -np.array(mids)
    a[8, :64] = rng.choice(mags, 64) * 2.0 ** -3      # exactly representable
    c_ref, s_ref = oracle.mx4_quantize(a)
    c, s = _quant4_gpu(a)
    assert c.shape == (512, 128) and s.shape == (512, 8)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(c, c_ref)


def _inputs(cfg, seed=0):
    src = mi.make_mx_sources(cfg, seed)
    q = {}
    c, s = _quant8_gpu(src["x"])
    cr, sr = oracle.mx_quantize(src["x"])
    assert np.array_equal(c, cr) and np.array_equal(s, sr), "x"
    q["x"] = (c, s)
    for n in ("w1", "w2"):
        c, s = _quant4_gpu(src[n])
        cr, sr = oracle.mx4_quantize(src[n])
        assert np.array_equal(c, cr) and np.array_equal(s, sr), n
        q[n] = (c, s)
    return src, q


def _case(cfg, tokens=None, seed=0, ids=None):
    import grouped_gemm_amd as g
    print(f"mxfp4 forward {cfg.name} T={cfg.T} D={cfg.D} H={cfg.H} E={cfg.E} k={cfg.k}", flush=True)
    src, q = _inputs(cfg, seed)
    (xc, xs), (w1c, w1s), (w2c, w2s) = q["x"], q["w1"], q["w2"]
    topk_ids = src["topk_ids"] if ids is None else ids
    out = g.moe_ffn_forward(to_gpu(xc), to_gpu(w1c), to_gpu(w2c), to_gpu(topk_ids),
                            to_gpu(src["topk_weights"]), mode="split", x_scale=to_gpu(xs),
                            w1_scale=to_gpu(w1s), w2_scale=to_gpu(w2s))
    torch.cuda.synchronize()
    out = gpu_bf16_to_f64(out)
    ref = mi.bf16_bits_to_f32(oracle.forward_mx4(xc, xs, w1c, w1s, w2c, w2s, topk_ids,
                                                 src["topk_weights"], tokens=tokens))
    if tokens is not None:
        out, ref = out[tokens], ref[tokens]
    rel, cos = assert_close(out, ref, tol=MX_TOL, cos_min=MX_COS, what=cfg.name)
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)
    return src


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (64, 256, 256, 8, 2, "softmax"),     # a few rows per expert
    (300, 384, 640, 16, 4, "zipf"),      # ragged experts, several K stages, H tiles of 64 act columns
    (1, 128, 128, 4, 2, "uniform"),      # one token, one K stage
    (2000, 512, 256, 6, 3, "zipf"),      # many m-tiles per expert
])
def test_mxfp4_forward_matches_oracle(T, D, H, E, k, routing):
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (64, 512, 512, 8, 2, "softmax"),     # one K stage per 512; 8 m-tiles, 4 row groups per block
    (1, 512, 512, 4, 2, "uniform"),      # one token
    (60, 1024, 512, 16, 4, "zipf"),      # ragged, several K stages
    (128, 512, 1024, 16, 2, "zipf"),     # skewed: experts with several 32-row m-tiles
    (64, 512, 512, 32, 8, "softmax"),    # 32 m-tiles
])
def test_mxfp4_decode_kernel_matches_oracle(T, D, H, E, k, routing):
    """Shapes the decode-shaped MXFP4 kernel takes (fewer than 0.5 experts expected
    past 32 rows, D and H multiples of 512)."""
    import grouped_gemm_amd as g
    for gemm in (1, 2):
        assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "mxfp4", "split", gemm) == "mx_kmajor_kernel"
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


@pytest.mark.parametrize("T,D,H,E,k,routing,gemms", [
    (64, 1024, 2048, 32, 8, "softmax", (1,)),     # GEMM1: 4 row groups per block (the fewest it takes)
    (64, 4096, 1536, 64, 6, "zipf", (1, 2)),      # 4 or 8 groups (4 + 4) per block; skewed: extra m-tiles
])
def test_mxfp4_kmajor_decode_kernel(T, D, H, E, k, routing, gemms):
    """The k-major MX decode GEMMs with e2m1 weights (four 32-row blocks per
    group, one per wave, all k-steps: no cross-wave sum)."""
    import grouped_gemm_amd as g
    for gemm in gemms:
        assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "mxfp4", "split", gemm) == "mx_kmajor_kernel"
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


def test_mxfp4_decode_workload_in_full():
    """The decode workload's dims (T=64, D=6144, H=2048, E=32, top-8) with fp4 weights, every token."""
    _case(mi.CONFIGS[2])


def test_mxfp4_decode_kernel_dropped_routes():
    cfg = mi.custom(64, 512, 512, 8, 3, "softmax", dtype="mxfp8")
    ids, _ = mi.routing(cfg, 0)
    ids = ids.copy()
    ids[::5, 0] = -1
    ids[::9, 2] = cfg.E + 3
    _case(cfg, ids=ids)


def test_mxfp4_forward_dropped_routes():
    cfg = mi.custom(200, 256, 256, 8, 3, "softmax", dtype="mxfp8")
    ids, _ = mi.routing(cfg, 0)
    ids = ids.copy()
    ids[::7, 1] = -1                     # dropped routes contribute nothing
    ids[::11, 2] = cfg.E
    _case(cfg, ids=ids)


def test_mxfp4_forward_mx_workload_sampled():
    """The MX workload's dims (T=16384, D=4096, H=1536, E=64, top-6) with fp4 weights; sampled tokens."""
    cfg = mi.CONFIGS[5]
    ids, _ = mi.routing(cfg, 0)
    _case(cfg, tokens=cover_sample(cfg, ids, "split", dtype="mxfp4", extra=8))


def test_mxfp4_fused_mode_is_unsupported():
    import grouped_gemm_amd as g
    assert g.moe_ffn_validate(64, 256, 256, 8, 2, "mxfp4", "fused") == g.MOE_FFN_EUNSUPPORTED
    assert g.moe_ffn_resolve_mode(64, 256, 256, 8, 2, "mxfp4", "auto") == g.MOE_FFN_SPLIT
