"""Seeded synthetic inputs for the routed MoE SwiGLU FFN forward pass.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It holds no arithmetic of the pass itself (no GEMM, no
SwiGLU, no combine, no quantization): it draws random tensors, rounds
them to bf16 storage, and draws the router's choices that the pass takes as
given inputs (Prime Flash MoE, section 1 "The computation": the pass
starts from each token's k chosen experts and their normalized weights,
which a router upstream produced).

Each tensor role (routing, x, W1, W2) has its own numpy PCG64 stream keyed
by (config id, role, seed), so a change of shape in one tensor does not
perturb the others.

Workload recipes (names follow the pages: T tokens, D hidden, H FFN
intermediate, E experts, k = top-k):

* tiny      T=64     D=256  H=512  E=8   k=2   softmax-top-k routing
* decode    T=64     D=6144 H=2048 E=32  k=8   uniform distinct experts,
                                                Dirichlet(1) weights
  (the decode example of "Optimizing Grouped GEMM for MoE on Blackwell":
  m=64 tokens per GPU, 32 local experts, top-8, W1 per expert 6144->4096)
* mid       T=4096   D=2048 H=768  E=128 k=8   softmax-top-k routing
* large     T=131072 D=2048 H=768  E=128 k=8   Zipf(s=1.1) log-prior added
                                                to the logits (expert 0 most
                                                popular), then softmax-top-k
* mx        T=16384  D=4096 H=1536 E=64  k=6   softmax-top-k routing; fp32
                                                sources to be MX-quantized

x ~ N(0, 1); W1 [E, 2H, D] ~ N(0, 1/D); W2 [E, D, H] ~ N(0, 1/H); rows of W1
are gate rows [0, H) followed by up rows [H, 2H) (Prime Flash MoE, section 1:
gate and up projections concatenated along W1's output dimension).

softmax-top-k: logits ~ N(0, 1) [T, E] -> softmax -> the k largest
probabilities in descending order (ties to the lower expert id) ->
renormalized to sum to 1, cast to fp32. For the pass that starts from the
router's logits, router_logits() hands out the logits alone.
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np

ROLE_ROUTING, ROLE_X, ROLE_W1, ROLE_W2 = 0, 1, 2, 3
ROLE_WS1, ROLE_WS2 = 5, 6  # shared expert


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    T: int
    D: int
    H: int
    E: int
    k: int
    routing: str          # "softmax" | "uniform" | "zipf"
    dtype: str = "bf16"   # "bf16" | "mxfp8" | "mxfp4" (fp4 weights, MX-fp8 activations)
    zipf_s: float = 1.1

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def flops(self) -> float:
        """6*P*D*H: two GEMMs over 2H and one over H, 2 flops per MAC."""
        return 6.0 * self.P * self.D * self.H


CONFIGS = {
    1: Config(1, "tiny", 64, 256, 512, 8, 2, "softmax"),
    2: Config(2, "decode", 64, 6144, 2048, 32, 8, "uniform"),
    3: Config(3, "mid_prefill", 4096, 2048, 768, 128, 8, "softmax"),
    4: Config(4, "large_prefill", 131072, 2048, 768, 128, 8, "zipf"),
    5: Config(5, "mx", 16384, 4096, 1536, 64, 6, "softmax", dtype="mxfp8"),
}


def custom(T, D, H, E, k, routing="softmax", dtype="bf16", cid=100, name=None):
    """A config of arbitrary size with the same recipes (for edge cases)."""
    return Config(cid, name or f"custom_T{T}_D{D}_H{H}_E{E}_k{k}", T, D, H, E, k,
                  routing, dtype)


def _rng(cfg: Config, role: int, seed: int, chunk: int = -1) -> np.random.Generator:
    key = [cfg.cid, role, seed, cfg.T, cfg.D, cfg.H, cfg.E, cfg.k]
    if chunk >= 0:
        key.append(chunk)
    return np.random.default_rng(key)


_CHUNK = 1 << 22
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _bf16_round_into(u: np.ndarray, out: np.ndarray) -> None:
    """out[:] = bf16 bits of the finite fp32 values viewed by u (uint32, modified)."""
    lsb = (u >> 16) & 1
    u += 0x7FFF
    u += lsb
    u >>= 16
    out[:] = u


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 to bf16 storage (round to nearest, ties to even), as uint16.

    u + 0x7FFF + 1 cannot wrap for a finite float (the largest finite bit
    pattern is 0xFF7FFFFF).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, np.uint16)
    for i in range(0, flat.size, _CHUNK):
        _bf16_round_into(flat[i:i + _CHUNK].view(np.uint32).copy(), out[i:i + _CHUNK])
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(cfg: Config, role: int, seed: int, shape, std, bf16: bool):
    """N(0, std^2) values, drawn in chunks of 2^22 from streams keyed by the
    chunk index (so the result does not depend on the thread count); fp32, or
    bf16 bits if `bf16`."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if bf16 else np.float32)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        v = _rng(cfg, role, seed, c).standard_normal(size=hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if bf16:
            _bf16_round_into(v.view(np.uint32), out[lo:hi])
        else:
            out[lo:hi] = v

    list(_pool().map(fill, range((n + _CHUNK - 1) // _CHUNK)))
    return out.reshape(shape)


def routing(cfg: Config, seed: int = 0):
    """topk_ids int32 [T, k], topk_weights fp32 [T, k]."""
    rng = _rng(cfg, ROLE_ROUTING, seed)
    T, E, k = cfg.T, cfg.E, cfg.k
    if cfg.routing == "uniform":
        # k distinct experts: the first k entries of a random permutation of E;
        # weights ~ Dirichlet(1) = normalized i.i.d. Exp(1).
        keys = rng.random((T, E))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
        w = rng.exponential(1.0, size=(T, k))
        w = w / w.sum(axis=1, keepdims=True)
        return np.ascontiguousarray(ids), np.ascontiguousarray(w.astype(np.float32))
    logits = rng.standard_normal((T, E))
    if cfg.routing == "zipf":
        logits = logits - cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))[None, :]
    elif cfg.routing != "softmax":
        raise ValueError(cfg.routing)
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, ids, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return (np.ascontiguousarray(ids.astype(np.int32)),
            np.ascontiguousarray(w.astype(np.float32)))


def shared_expert(cfg: Config, Hs: int, seed: int = 0):
    """One shared expert's weights as bf16 bits: ws1 [2Hs, D] ~ N(0, 1/D) (gate
    rows, then up rows) and ws2 [D, Hs] ~ N(0, 1/Hs), from streams of their own."""
    ws1 = _normal(cfg, ROLE_WS1, seed * 1000003 + Hs, (2 * Hs, cfg.D), 1.0 / np.sqrt(cfg.D), True)
    ws2 = _normal(cfg, ROLE_WS2, seed * 1000003 + Hs, (cfg.D, Hs), 1.0 / np.sqrt(Hs), True)
    return ws1, ws2


def router_logits(cfg: Config, seed: int = 0) -> np.ndarray:
    """Router logits fp32 [T, E] of the recipe above, for the pass that starts
    from logits: the draws routing() makes for softmax and Zipf configs (the
    same stream, so the routes agree up to fp32 rounding of near-ties), N(0, 1)
    for the others. The softmax/top-k itself is not done here."""
    rng = _rng(cfg, ROLE_ROUTING, seed)
    logits = rng.standard_normal((cfg.T, cfg.E))
    if cfg.routing == "zipf":
        logits = logits - cfg.zipf_s * np.log(np.arange(1, cfg.E + 1, dtype=np.float64))[None, :]
    return np.ascontiguousarray(logits.astype(np.float32))


def _tensors(cfg: Config, seed: int, bf16: bool):
    x = _normal(cfg, ROLE_X, seed, (cfg.T, cfg.D), 1.0, bf16)
    w1 = _normal(cfg, ROLE_W1, seed, (cfg.E, 2 * cfg.H, cfg.D), 1.0 / np.sqrt(cfg.D), bf16)
    w2 = _normal(cfg, ROLE_W2, seed, (cfg.E, cfg.D, cfg.H), 1.0 / np.sqrt(cfg.H), bf16)
    return x, w1, w2


def sources_f32(cfg: Config, seed: int = 0):
    """fp32 x [T, D], W1 [E, 2H, D], W2 [E, D, H] before any rounding."""
    return _tensors(cfg, seed, bf16=False)


def make_bf16(cfg: Config, seed: int = 0):
    """Dict of host arrays for the bf16 path (bf16 tensors as uint16 bits).

    Identical to rounding sources_f32() to bf16, without the fp32 copy."""
    x, w1, w2 = _tensors(cfg, seed, bf16=True)
    ids, wts = routing(cfg, seed)
    return dict(x=x, w1=w1, w2=w2, topk_ids=ids, topk_weights=wts)


def make_mx_sources(cfg: Config, seed: int = 0):
    """Dict of fp32 sources for the MX-fp8 path; each side quantizes them."""
    x, w1, w2 = sources_f32(cfg, seed)
    ids, wts = routing(cfg, seed)
    return dict(x=x, w1=w1, w2=w2, topk_ids=ids, topk_weights=wts)


def expert_histogram(ids: np.ndarray, E: int) -> np.ndarray:
    flat = ids.reshape(-1)
    flat = flat[(flat >= 0) & (flat < E)]
    return np.bincount(flat, minlength=E)
