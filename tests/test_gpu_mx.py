"""MX-fp8 path on the GPU: the quantizer must equal the oracle's MXQ bit for
bit, and the forward pass must match the oracle within the MX tolerance.

Each side quantizes the same fp32 sources with its own quantizer; the GPU
forward consumes the GPU's codes and the oracle its own, after the test has
checked that the two sets of codes are identical."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import MX_COS, MX_TOL, assert_close, gpu_bf16_to_f64, cover_sample, to_gpu

pytestmark = pytest.mark.gpu


def _quant_gpu(src: np.ndarray):
    import grouped_gemm_amd as g
    c, s = g.moe_ffn_mx_quantize(to_gpu(src.astype(np.float32)))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def test_quantizer_bit_exact_random_and_edges():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal((512, 256)) * np.exp(rng.normal(0, 4, (512, 1)))).astype(np.float32)
    a[0] = 0.0                                        # all-zero blocks
    a[1, :32] = 448.0                                 # amax exactly 448 * 2^0
    a[2, :32] = np.float32(448.0) * np.float32(2.0 ** -20)
    a[3] = -a[3]
    a[4, 5] = 1e30                                    # huge amax in one block
    a[5] = 1e-40                                      # subnormal inputs
    a[6, :32] = np.array([(i - 16) * 2.0 ** -9 for i in range(32)], np.float32)
    pos = np.array([oracle.e4m3_decode(c) for c in range(127)])
    a[7, :126] = ((pos[1:] + pos[:-1]) / 2)[:126]     # exact ties between codes
    a[7, 126:] = 448.0
    c_ref, s_ref = oracle.mx_quantize(a)
    c, s = _quant_gpu(a)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(c, c_ref)


def _mx_inputs(cfg, seed=0):
    src = mi.make_mx_sources(cfg, seed)
    q = {}
    for n in ("x", "w1", "w2"):
        c, s = _quant_gpu(src[n])
        cr, sr = oracle.mx_quantize(src[n])
        assert np.array_equal(c, cr) and np.array_equal(s, sr), n
        q[n] = (c, s)
    return src, q


def _case(cfg, tokens=None, seed=0, mode="split", ids=None):
    import grouped_gemm_amd as g
    print(f"mx forward {cfg.name} T={cfg.T} D={cfg.D} H={cfg.H} E={cfg.E} k={cfg.k} mode={mode}", flush=True)
    src, q = _mx_inputs(cfg, seed)
    if ids is not None:
        src["topk_ids"] = ids
    (xc, xs), (w1c, w1s), (w2c, w2s) = q["x"], q["w1"], q["w2"]
    # the output starts as NaN, so a row the pass leaves unwritten fails the comparison
    out = torch.full((cfg.T, cfg.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    g.moe_ffn_forward(to_gpu(xc), to_gpu(w1c), to_gpu(w2c), to_gpu(src["topk_ids"]),
                      to_gpu(src["topk_weights"]), out=out, mode=mode, x_scale=to_gpu(xs),
                      w1_scale=to_gpu(w1s), w2_scale=to_gpu(w2s))
    torch.cuda.synchronize()
    out = gpu_bf16_to_f64(out)
    ref = mi.bf16_bits_to_f32(oracle.forward_mx(xc, xs, w1c, w1s, w2c, w2s, src["topk_ids"],
                                                src["topk_weights"], tokens=tokens))
    if tokens is not None:
        out, ref = out[tokens], ref[tokens]
    rel, cos = assert_close(out, ref, tol=MX_TOL, cos_min=MX_COS, what=cfg.name)
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (64, 256, 256, 8, 2, "softmax"),
    (300, 384, 640, 16, 4, "zipf"),
    (1, 128, 128, 4, 2, "uniform"),
])
def test_mx_forward_small(T, D, H, E, k, routing):
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (2100, 256, 256, 3, 2, "zipf"),     # prefill tiles, short K: hand-over after the ring drains
    (2100, 512, 768, 3, 2, "zipf"),     # prefill tiles, hand-over inside the ring
])
@pytest.mark.parametrize("grid_limit", [None, "8"])
def test_mx_forward_prefill_tiles(T, D, H, E, k, routing, grid_limit, monkeypatch):
    # with 8 workgroups each one walks many tiles, so the cross-tile hand-over runs
    if grid_limit:
        monkeypatch.setenv("MOE_FFN_GRID_LIMIT", grid_limit)
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (64, 512, 512, 8, 2, "softmax"),     # one K stage per 512; 8 m-tiles, each with 4 of its row groups per block
    (1, 512, 512, 4, 2, "uniform"),      # one token
    (60, 1024, 512, 16, 4, "zipf"),      # ragged, several K stages
    (128, 512, 1024, 16, 2, "zipf"),     # skewed: experts with several 32-row m-tiles
    (64, 512, 512, 32, 8, "softmax"),    # 32 m-tiles
])
def test_mx_decode_kernel(T, D, H, E, k, routing):
    """Shapes the decode-shaped MX kernel takes with e4m3 weights (fewer than 0.5
    experts expected past 32 rows, D and H multiples of 512)."""
    import grouped_gemm_amd as g
    for gemm in (1, 2):
        assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "mxfp8", "split", gemm) == "mx_kmajor_kernel"
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


@pytest.mark.parametrize("T,D,H,E,k,routing,gemms", [
    (16, 2048, 1024, 32, 8, "uniform", (1, 2)),   # 4 row groups per block (the fewest it takes)
    (64, 1024, 2048, 32, 8, "softmax", (1,)),     # GEMM1: 8 groups, one super-group
    (64, 4096, 1536, 64, 6, "zipf", (1, 2)),      # 12 and 16 groups (6 + 6, 8 + 8) and more; skewed: extra m-tiles
    (64, 512, 512, 512, 8, "uniform", (1, 2)),    # more m-tiles than CUs: a block per m-tile, all its groups
])
def test_mx_kmajor_decode_kernel(T, D, H, E, k, routing, gemms):
    """The k-major MX decode GEMMs (e4m3 weights: two 32-row blocks per group,
    each wave half the k-steps, the halves summed at the end of a super-group;
    GEMM1's act requantized from 16-column halves whose maxima meet in LDS)."""
    import grouped_gemm_amd as g
    for gemm in gemms:
        assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "mxfp8", "split", gemm) == "mx_kmajor_kernel"
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))


def test_mx_decode_dims_in_full():
    """The MX workload's dims at 64 tokens (D=4096, H=1536, E=64, top-6): the
    decode kernel on every token."""
    _case(mi.custom(64, 4096, 1536, 64, 6, "softmax", dtype="mxfp8"))


def test_mx_decode_kernel_dropped_routes():
    cfg = mi.custom(64, 512, 512, 8, 3, "softmax", dtype="mxfp8")
    ids, _ = mi.routing(cfg, 0)
    ids = ids.copy()
    ids[::5, 0] = -1                     # dropped routes contribute nothing
    ids[::9, 2] = cfg.E + 3
    _case(cfg, ids=ids)


def test_mx_prefill_descriptor_reload(monkeypatch):
    # 8 workgroups x more than 128 tiles each: the tile descriptors are reloaded
    monkeypatch.setenv("MOE_FFN_GRID_LIMIT", "8")
    cfg = mi.custom(16384, 256, 4096, 2, 1, "uniform", dtype="mxfp8")
    ids, _ = mi.routing(cfg)
    _case(cfg, tokens=cover_sample(cfg, ids, "split", extra=16))


def test_mx_config_sampled():
    cfg = mi.CONFIGS[5]
    ids, _ = mi.routing(cfg)
    _case(cfg, tokens=cover_sample(cfg, ids, "split", extra=16))


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (64, 256, 256, 8, 2, "softmax"),    # the tiny workload's size class
    (300, 384, 640, 16, 4, "zipf"),     # ragged m-tiles, skew, H slices of 64 over 640
    (1, 128, 128, 4, 2, "uniform"),     # a single token
    (513, 128, 256, 3, 3, "uniform"),   # k = E
    (700, 512, 384, 5, 3, "zipf"),
])
def test_mx_forward_fused(T, D, H, E, k, routing):
    """The fused MX pipeline: the act requantized in LDS feeds a split-K down
    projection per 64-wide H slice (two scale blocks: one scaled-MFMA K step)."""
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"), mode="fused")


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    pytest.param(64, 4096, 1536, 64, 6, "softmax", marks=pytest.mark.skip(
        reason="a variant of the kernel with its GEMM1 epilogue after the K loop faulted the GPU on this shape "
               "(illegal memory access); the variant was withdrawn, its cause is not found, so the shape stays off "
               "the GPU; the kernel as built had passed it")),  # the MX workload's dims at 64 tokens
    (1, 512, 256, 4, 2, "uniform"),      # a single token
    (40, 1024, 640, 16, 8, "zipf"),      # five slices of H, hot experts with several m-tiles
    (64, 512, 384, 4, 4, "uniform"),     # k = E
    (300, 1024, 256, 8, 2, "zipf"),      # many 32-row m-tiles per expert, ragged last tiles
])
def test_mx_fused_ring_kernel(T, D, H, E, k, routing):
    """The fused MX pass on the decode kernels' rings: GEMM1 k-major, the act
    requantized by MXQ into LDS per 32 columns, the down projection with the
    tokens as the scaled MFMA's rows added into the fp32 accumulator, each
    token's row converted by the block that adds its last partial."""
    import grouped_gemm_amd as g
    assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "mxfp8", "fused", 1) == "mx_fused_dma_kernel"
    _case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"), mode="fused")


def test_mx_auto_small_batch_runs_fused():
    """AUTO takes the fused MX pipeline for a batch whose fused blocks fit one
    round of the CUs (4 tokens: about 13 m-tiles x 8 slices)."""
    import grouped_gemm_amd as g
    assert g.moe_ffn_resolve_mode(4, 2048, 1024, 32, 4, dtype="mxfp8") == g.MOE_FFN_FUSED
    assert g.moe_ffn_gemm_kernel(4, 2048, 1024, 32, 4, "mxfp8", "auto", 1) == "mx_fused_dma_kernel"
    _case(mi.custom(4, 2048, 1024, 32, 4, "softmax", dtype="mxfp8"), mode="auto")


def test_mx_fused_ring_kernel_dropped_routes():
    """Dropped routes, tokens with no route at all (their rows are zeros) and
    zero routing weights on the fused MX ring kernel."""
    cfg = mi.custom(96, 512, 512, 8, 4, "uniform", dtype="mxfp8")
    ids, _ = mi.routing(cfg, 0)
    ids = ids.copy()
    ids[::3, 1] = -1
    ids[1::5, 2] = 8                      # == E: dropped
    ids[7, :] = -1                        # no route at all
    ids[11, :] = 9
    _case(cfg, ids=ids, mode="fused")


def test_mx_fused_config_sampled():
    cfg = mi.CONFIGS[5]
    ids, _ = mi.routing(cfg)
    _case(cfg, tokens=cover_sample(cfg, ids, "fused", extra=16), mode="fused")


@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("T,D,H,E,k,kernel", [
    (32, 512, 512, 8, 3, "mx_kmajor_kernel"),       # decode kernel
    (2100, 256, 512, 3, 2, "big_gemm_kernel<256>"), # prefill ring
    (300, 384, 640, 16, 4, "mx_gemm1_kernel"),      # generic kernels
])
def test_mx_duplicate_expert_ids(mode, T, D, H, E, k, kernel):
    """The same expert in several slots of one token counts once per slot."""
    import grouped_gemm_amd as g
    cfg = mi.custom(T, D, H, E, k, "zipf", dtype="mxfp8")
    assert g.moe_ffn_gemm_kernel(T, D, H, E, k, "mxfp8", "split", 1) == kernel
    ids, _ = mi.routing(cfg, 0)
    ids = ids.copy()
    ids[::2, 1] = ids[::2, 0]
    ids[::3, k - 1] = ids[::3, 0]
    ids[5, :] = ids[5, 0]
    _case(cfg, ids=ids, mode=mode)
