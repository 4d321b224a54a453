"""The router (softmax -> top-k -> renormalize) on the GPU through the C ABI
against the CPU oracle's router: ids bit-exact, weights within fp32
rounding; and the pass that starts from logits (moe_ffn_forward_logits)
against the oracle's router followed by the oracle's forward pass.

Weight tolerance: the GPU evaluates exp(l_j - l_0) / sum in fp32 (the
subtraction rounds at 2^-24 relative to |l_j - l_0|, expf is within a few
ulps, the sum of k terms and the division add k + 1 roundings), so each
weight (at most 1) is within a few 1e-6 of the oracle's double evaluation
for logit spreads up to ~30; 1e-5 is the bar.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.parity import (MX_COS, MX_TOL, assert_close, gpu_bf16_to_f64, cover_sample, to_gpu,
                          upload_bf16)

pytestmark = pytest.mark.gpu

W_TOL = 1e-5


def _router_gpu(logits, k):
    import grouped_gemm_amd as g
    ids, wts = g.moe_ffn_router(to_gpu(logits), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wts.cpu().numpy()


def _check_router(logits, k, what):
    print(f"router {what}: T={logits.shape[0]} E={logits.shape[1]} k={k}", flush=True)
    ids, wts = _router_gpu(logits, k)
    rid, rw = oracle.router(logits, k)
    np.testing.assert_array_equal(ids, rid, err_msg=what)
    assert np.array_equal(np.isnan(wts), np.isnan(rw)), f"{what}: NaN weights differ"
    both = ~np.isnan(rw)
    err = np.abs(wts[both].astype(np.float64) - rw[both]).max() if both.any() else 0.0
    assert err <= W_TOL, f"{what}: weight error {err}"


@pytest.mark.parametrize("T,E,k", [
    (1, 8, 2), (100, 8, 2), (257, 32, 8), (1000, 128, 8), (333, 64, 6), (77, 1000, 5),
    (50, 3, 3), (129, 16, 16), (64, 256, 8), (65, 512, 1), (19, 2048, 64), (7, 8192, 8),
    (300, 5, 1), (4097, 100, 7),
])
def test_router_matches_oracle(T, E, k):
    rng = np.random.default_rng([T, E, k, 1])
    _check_router(rng.standard_normal((T, E)).astype(np.float32), k, "normal")


def test_router_ties_and_masks():
    rng = np.random.default_rng(5)
    # integer logits: many exact ties, broken toward the lower id
    _check_router(rng.integers(-3, 4, size=(500, 40)).astype(np.float32), 7, "ties")
    _check_router(np.zeros((33, 64), np.float32), 8, "all equal")
    # masked experts (-inf) come last; a token with fewer than k finite logits
    # gets them with weight 0
    lg = rng.standard_normal((200, 24)).astype(np.float32)
    lg[rng.random((200, 24)) < 0.5] = -np.inf
    lg[:, 0] = np.where(np.isfinite(lg[:, 0]), lg[:, 0], 0.0)  # keep one finite logit per token
    _check_router(lg, 6, "masked")
    # NaN ranks last, -0 ties +0
    sp = rng.standard_normal((130, 20)).astype(np.float32)
    sp[rng.random((130, 20)) < 0.2] = np.nan
    sp[rng.random((130, 20)) < 0.2] = -0.0
    sp[rng.random((130, 20)) < 0.2] = 0.0
    _check_router(sp, 5, "nan and signed zeros")
    _check_router(np.full((3, 2100), np.nan, np.float32), 4, "all NaN, scan path")
    # a wide logit range
    _check_router((rng.standard_normal((300, 64)) * 20).astype(np.float32), 8, "wide")


@pytest.mark.parametrize("cid", [1, 3, 4, 5])
def test_router_full_size(cid):
    """Every token of the workload's logits (the large prefill: 131072 x 128)."""
    cfg = mi.CONFIGS[cid]
    _check_router(mi.router_logits(cfg, 0), cfg.k, cfg.name)


def _forward_logits(t, logits, k, mode, **mx):
    import grouped_gemm_amd as g
    out, ids, wts = g.moe_ffn_forward_logits(t["x"], t["w1"], t["w2"], to_gpu(logits), k, mode=mode, **mx)
    torch.cuda.synchronize()
    return gpu_bf16_to_f64(out), ids.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("T,D,H,E,k,routing,mode", [
    (64, 256, 512, 8, 2, "softmax", "fused"),     # the tiny workload's shape, fused pipeline
    (64, 256, 512, 8, 2, "softmax", "split"),     # one-wave route
    (1500, 256, 256, 16, 4, "zipf", "split"),     # one-workgroup route
    (2600, 256, 256, 16, 8, "softmax", "split"),  # multi-kernel route: router builds the histogram
    (3001, 128, 256, 7, 6, "zipf", "split"),      # k does not divide the route segment
])
def test_forward_logits_matches_oracle(T, D, H, E, k, routing, mode):
    cfg = mi.custom(T, D, H, E, k, routing)
    print(f"forward_logits {cfg.name} mode={mode}", flush=True)
    d = mi.make_bf16(cfg, 0)
    logits = mi.router_logits(cfg, 0)
    out, ids, wts = _forward_logits(upload_bf16(d), logits, k, mode)
    rid, rw = oracle.router(logits, k)
    np.testing.assert_array_equal(ids, rid)
    assert np.abs(wts.astype(np.float64) - rw).max() <= W_TOL
    ref = mi.bf16_bits_to_f32(oracle.forward_bf16(d["x"], d["w1"], d["w2"], rid, rw)).astype(np.float64)
    rel, cos = assert_close(out, ref, what=f"{cfg.name}/{mode}")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


def test_forward_logits_large_prefill_sampled():
    """The large prefill from logits, in the benchmark's launch configuration;
    ids and weights of every token, outputs of sampled tokens."""
    cfg = mi.CONFIGS[4]
    print("forward_logits large_prefill (sampled tokens)", flush=True)
    d = mi.make_bf16(cfg, 0)
    logits = mi.router_logits(cfg, 0)
    out, ids, wts = _forward_logits(upload_bf16(d), logits, cfg.k, "split")
    rid, rw = oracle.router(logits, cfg.k)
    np.testing.assert_array_equal(ids, rid)
    assert np.abs(wts.astype(np.float64) - rw).max() <= W_TOL
    tokens = cover_sample(cfg, rid, "split", extra=16)
    ref = mi.bf16_bits_to_f32(oracle.forward_bf16(d["x"], d["w1"], d["w2"], rid, rw, tokens=tokens))
    rel, cos = assert_close(out[tokens], ref[tokens].astype(np.float64), what="large_prefill/logits")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)


def test_forward_logits_mx():
    """MX-fp8 from logits: each side quantizes the same fp32 sources with its
    own quantizer (checked identical), then routes from the same logits."""
    import grouped_gemm_amd as g
    cfg = mi.custom(700, 256, 256, 6, 3, "softmax", dtype="mxfp8")
    print(f"forward_logits mx {cfg.name}", flush=True)
    s = mi.make_mx_sources(cfg, 0)
    t, scales, q = {}, {}, {}
    for n in ("x", "w1", "w2"):
        c, sc = g.moe_ffn_mx_quantize(to_gpu(s[n].astype(np.float32)))
        q[n] = oracle.mx_quantize(s[n])
        assert np.array_equal(c.cpu().numpy(), q[n][0]) and np.array_equal(sc.cpu().numpy(), q[n][1]), n
        t[n], scales[n + "_scale"] = c, sc
    logits = mi.router_logits(cfg, 0)
    out, ids, wts = _forward_logits(t, logits, cfg.k, "split", **scales)
    rid, rw = oracle.router(logits, cfg.k)
    np.testing.assert_array_equal(ids, rid)
    ref = oracle.forward_mx(q["x"][0], q["x"][1], q["w1"][0], q["w1"][1], q["w2"][0], q["w2"][1], rid, rw)
    rel, cos = assert_close(out, mi.bf16_bits_to_f32(ref).astype(np.float64), tol=MX_TOL, cos_min=MX_COS,
                            what="mx/logits")
    print(f"  max err / max|ref| = {rel:.3e}, cosine = {cos:.7f}", flush=True)
