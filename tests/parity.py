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


# Token rows per m-tile of each GEMM kernel family the dispatch can pick
# (the names moe_ffn_gemm_kernel reports).
TILE_ROWS = {
    "dma_kmajor_kernel": 32, "dma_skinny_kernel": 32, "mx_kmajor_kernel": 32,
    "big_gemm_kernel<128>": 128, "big_gemm_kernel<256>": 256,
    "gemm1_swiglu_kernel": 128, "gemm2_weight_kernel": 128,
    "mx_gemm1_kernel": 128, "mx_gemm2_kernel": 128,
    "fused_dma_kernel": 32, "fused_bf16_kernel": 128, "mx_fused_kernel": 128, "mx_fused_dma_kernel": 32,
}


def kernel_tile_rows(cfg: mi.Config, mode: str, dtype: str = None) -> int:
    """The smallest m-tile height among the GEMM kernels the library runs for
    this workload and mode (asked of the library's own dispatch)."""
    import grouped_gemm_amd as g
    dt = dtype or cfg.dtype
    rows = []
    for gemm in (1, 2):
        name = g.moe_ffn_gemm_kernel(cfg.T, cfg.D, cfg.H, cfg.E, cfg.k, dt, mode, gemm)
        assert name in TILE_ROWS, name
        rows.append(TILE_ROWS[name])
    return min(rows)


def tile_cover_tokens(ids: np.ndarray, E: int, bm: int, seed: int = 0, extra: int = 0) -> np.ndarray:
    """Tokens whose routed rows touch every m-tile of height `bm` that the
    grouped GEMMs process, plus the first and last row of every expert's
    segment and `extra` random tokens.

    The sorted order is rebuilt here from the ids (a stable sort of the pairs
    p = t*k + j by expert, dropped ids left out); m-tiles start at every
    multiple of `bm` inside an expert's segment. Each uncovered tile gets one
    row at a random position inside it, and every tile that row's token
    touches through its other slots counts as covered too.
    """
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    pairs = np.nonzero((flat >= 0) & (flat < E))[0]
    order = pairs[np.argsort(flat[pairs], kind="stable")]          # sorted row -> pair
    counts = np.bincount(flat[pairs], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rank = np.arange(order.size) - offsets[flat[order]]            # row inside its expert
    ntile_e = (counts + bm - 1) // bm
    tile_base = np.concatenate([[0], np.cumsum(ntile_e)])
    tile_of_pair = np.full(T * k, -1, np.int64)
    tile_of_pair[order] = tile_base[flat[order]] + rank // bm
    tok_tiles = tile_of_pair.reshape(T, k)
    ntiles = int(tile_base[-1])
    covered = np.zeros(ntiles, bool)
    picks = set()

    def take(t):
        picks.add(int(t))
        tt = tok_tiles[t]
        covered[tt[tt >= 0]] = True

    for e in np.nonzero(counts)[0]:
        take(order[offsets[e]] // k)
        take(order[offsets[e + 1] - 1] // k)
    rng = np.random.default_rng([seed, bm, 11])
    tile_e = np.repeat(np.arange(E), ntile_e)
    tile_j = np.arange(ntiles) - tile_base[tile_e]
    for ti in np.nonzero(~covered)[0]:
        if covered[ti]:
            continue
        e, j = tile_e[ti], tile_j[ti]
        rows = min(bm, counts[e] - j * bm)
        take(order[offsets[e] + j * bm + rng.integers(rows)] // k)
    assert covered.all()
    if extra:
        picks.update(rng.choice(T, size=min(extra, T), replace=False).tolist())
    return np.array(sorted(picks), np.int64)


def cover_sample(cfg: mi.Config, ids: np.ndarray, mode: str = "split", dtype: str = None, extra: int = 16,
                 dense_bm: int = 0, seed: int = 0) -> np.ndarray:
    """Tokens to compare on a full-size workload: every m-tile of the GEMM
    kernels the library dispatches for (cfg, mode) gets a row (see
    tile_cover_tokens), plus the first and last token, a token of the least
    popular expert, `extra` random tokens and, with `dense_bm`, one token in
    every block of `dense_bm` consecutive tokens (the m-tiles of a pass that
    runs every token through one group, such as a shared expert)."""
    bm = kernel_tile_rows(cfg, mode, dtype)
    picks = set(tile_cover_tokens(ids, cfg.E, bm, seed, extra).tolist())
    picks.update(sample_tokens(cfg, ids, 0, seed).tolist())
    if dense_bm:
        rng = np.random.default_rng([seed, dense_bm, 13])
        for t0 in range(0, cfg.T, dense_bm):
            picks.add(int(t0 + rng.integers(min(dense_bm, cfg.T - t0))))
    return np.array(sorted(picks), np.int64)
