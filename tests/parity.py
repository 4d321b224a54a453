"""Helpers shared by the GPU parity tests: host<->device transfer of the
seeded inputs and the acceptance checks.

Acceptance (bf16): max |gpu - ref| <= 2e-2 * max |ref| and cosine >= 0.9999
over every compared value; MX-fp8: max |gpu - ref| <= 6e-2 * max |ref| and
cosine >= 0.999. Index maps: bit-exact.
"""
import numpy as np
import torch

import moe_inputs as mi

BF16_TOL, BF16_COS = 2e-2, 0.9999
MX_TOL, MX_COS = 6e-2, 0.999


def dev():
    return torch.device("cuda:0")


def bf16_to_gpu(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def gpu_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def metrics(out: np.ndarray, ref: np.ndarray):
    out = out.astype(np.float64).ravel()
    ref = ref.astype(np.float64).ravel()
    scale = np.abs(ref).max()
    err = np.abs(out - ref).max()
    denom = np.linalg.norm(out) * np.linalg.norm(ref)
    cos = float(out @ ref / denom) if denom > 0 else (1.0 if np.abs(out).max() == 0 else 0.0)
    return float(err), float(scale), cos


def assert_close(out: np.ndarray, ref: np.ndarray, tol=BF16_TOL, cos_min=BF16_COS, what=""):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err, scale, cos = metrics(out, ref)
    assert err <= tol * scale, f"{what}: max err {err:.4g} > {tol} * {scale:.4g} (cos {cos:.6f})"
    assert cos >= cos_min, f"{what}: cosine {cos:.7f} < {cos_min}"
    return err / scale if scale else 0.0, cos


def upload_bf16(d: dict):
    """Seeded host inputs (bf16 bits) -> GPU tensors."""
    return dict(x=bf16_to_gpu(d["x"]), w1=bf16_to_gpu(d["w1"]), w2=bf16_to_gpu(d["w2"]),
                topk_ids=to_gpu(d["topk_ids"]), topk_weights=to_gpu(d["topk_weights"]))


def sample_tokens(cfg: mi.Config, ids: np.ndarray, n: int, seed: int = 0) -> np.ndarray:
    """n tokens spread over the batch, always including the first and last token
    and a token routed to the least popular expert that has any routes."""
    rng = np.random.default_rng([seed, cfg.cid, 7])
    picks = set(rng.choice(cfg.T, size=min(n, cfg.T), replace=False).tolist())
    picks.update({0, cfg.T - 1})
    hist = mi.expert_histogram(ids, cfg.E)
    live = np.nonzero(hist)[0]
    rare = live[np.argmin(hist[live])]
    picks.add(int(np.nonzero((ids == rare).any(axis=1))[0][0]))
    return np.array(sorted(picks), np.int64)
