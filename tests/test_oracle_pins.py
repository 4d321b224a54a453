"""Pins of the CPU oracle (bf16 path and route maps) against things other
than itself: a brute-force dense fp64 evaluation, the E=1/k=1 reduction to a
dense SwiGLU FFN, a closed-form worked example, Python's own sort, and
invariants of the definition (Prime Flash MoE, section 1 "The
computation").
"""
import math

import numpy as np
import pytest

import moe_inputs as mi


def _f32(b):
    return mi.bf16_bits_to_f32(b).astype(np.float64)


def dense_reference_fp64(x, w1, w2, ids, wts):
    """Every expert on every token in fp64, then a mask-weighted sum.

    A different algorithm from the oracle's per-token loop: GEMMs over all
    tokens per expert (numpy matmul), gate = first H rows of W1, up = last H
    rows, act = silu(gate) * up, y = act @ W2^T, out = sum_e M[t, e] * y_e
    with M[t, e] = sum of the token's routing weights on expert e.
    """
    X, W1, W2 = _f32(x), _f32(w1), _f32(w2)
    T, D = X.shape
    E, H2, _ = W1.shape
    H = H2 // 2
    M = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = ids[t, j]
            if 0 <= e < E:
                M[t, e] += float(wts[t, j])
    out = np.zeros((T, D))
    for e in range(E):
        gu = X @ W1[e].T
        g, u = gu[:, :H], gu[:, H:]
        act = g / (1.0 + np.exp(-g)) * u
        out += M[:, e:e + 1] * (act @ W2[e].T)
    return out


def _check_close_to_fp64(out_bits, ref):
    """bf16 output vs the exact value: bf16 rounding (2^-9 relative) plus fp32
    accumulation error, far below what any dropped term or wrong index gives."""
    o = _f32(out_bits)
    scale = np.abs(ref).max()
    err = np.abs(o - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5 * scale), err.max()


@pytest.mark.parametrize("T,D,H,E,k,routing", [
    (16, 64, 32, 4, 2, "softmax"),
    (9, 96, 64, 5, 3, "uniform"),
    (12, 32, 96, 6, 6, "zipf"),
    (7, 64, 64, 3, 1, "softmax"),
])
def test_oracle_matches_dense_fp64(oracle_lib, T, D, H, E, k, routing):
    cfg = mi.custom(T, D, H, E, k, routing)
    d = mi.make_bf16(cfg, seed=3)
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    ref = dense_reference_fp64(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    _check_close_to_fp64(out, ref)


def test_tiny_config_matches_dense_fp64(oracle_lib):
    d = mi.make_bf16(mi.CONFIGS[1])
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    ref = dense_reference_fp64(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    _check_close_to_fp64(out, ref)


def test_single_expert_top1_is_dense_swiglu_ffn(oracle_lib):
    """E=1, k=1, w=1 reduces to the dense SwiGLU FFN (silu(x Wg^T) * (x Wu^T)) W2^T."""
    cfg = mi.custom(20, 128, 64, 1, 1)
    d = mi.make_bf16(cfg, seed=5)
    ids = np.zeros((20, 1), np.int32)
    wts = np.ones((20, 1), np.float32)
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], ids, wts)
    X, W1, W2 = _f32(d["x"]), _f32(d["w1"])[0], _f32(d["w2"])[0]
    gate = X @ W1[:64].T
    up = X @ W1[64:].T
    ref = (gate * (1.0 / (1.0 + np.exp(-gate))) * up) @ W2.T
    _check_close_to_fp64(out, ref)


def _bf16(v):
    return mi.to_bf16_bits(np.asarray(v, np.float32))


def test_worked_example_closed_form(oracle_lib):
    """T=1, D=2, H=1, E=2, k=2, every input exactly representable in bf16.

    expert 0: gate = 1*1 + 0*2 = 1, up = 0*1 + 1*2 = 2, act = 2 silu(1),
              y0 = (act, act/2)
    expert 1: gate = 0*1 - 1*2 = -2, up = 1*1 + 1*2 = 3, act = 3 silu(-2),
              y1 = (2 act, -act)
    out = 0.75 y0 + 0.25 y1, silu(z) = z / (1 + e^-z).
    """
    x = _bf16([[1.0, 2.0]])
    w1 = _bf16([[[1.0, 0.0], [0.0, 1.0]], [[0.0, -1.0], [1.0, 1.0]]])
    w2 = _bf16([[[1.0], [0.5]], [[2.0], [-1.0]]])
    ids = np.array([[0, 1]], np.int32)
    wts = np.array([[0.75, 0.25]], np.float32)
    out = _f32(oracle_lib.forward_bf16(x, w1, w2, ids, wts))[0]

    def silu(z):
        return z / (1.0 + math.exp(-z))

    a0 = 2.0 * silu(1.0)
    a1 = 3.0 * silu(-2.0)
    expect = [0.75 * a0 + 0.25 * 2.0 * a1, 0.75 * a0 / 2.0 - 0.25 * a1]
    for o, e in zip(out, expect):
        assert abs(o - e) <= 2.0 ** -8 * abs(e)
    # the wrong split (up rows first) gives a different answer
    swapped = _f32(oracle_lib.forward_bf16(x, w1[:, ::-1, :].copy(), w2, ids, wts))[0]
    assert abs(swapped[0] - expect[0]) > 0.05


def test_token_permutation_permutes_output(oracle_lib):
    cfg = mi.custom(32, 64, 64, 4, 2)
    d = mi.make_bf16(cfg, seed=7)
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    perm = np.random.default_rng(1).permutation(32)
    out_p = oracle_lib.forward_bf16(d["x"][perm], d["w1"], d["w2"], d["topk_ids"][perm],
                                    d["topk_weights"][perm])
    assert np.array_equal(out_p, out[perm])


def test_zero_weight_routes_contribute_nothing(oracle_lib):
    cfg = mi.custom(24, 64, 64, 6, 3)
    d = mi.make_bf16(cfg, seed=8)
    wts = d["topk_weights"].copy()
    wts[:, 2] = 0.0
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], wts)
    ids2 = d["topk_ids"].copy()
    ids2[:, 2] = (ids2[:, 2] + 1) % 6
    out2 = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], ids2, wts)
    assert np.array_equal(out, out2)
    zero = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], np.zeros_like(wts))
    assert not np.any(zero & 0x7FFF)


def test_doubling_weights_doubles_output(oracle_lib):
    cfg = mi.custom(24, 64, 64, 6, 3)
    d = mi.make_bf16(cfg, seed=9)
    out = _f32(oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"]))
    out2 = _f32(oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"],
                                        2.0 * d["topk_weights"]))
    assert np.array_equal(out2, 2.0 * out)


def test_zero_w2_equals_dropping_the_expert(oracle_lib):
    cfg = mi.custom(24, 64, 64, 4, 2)
    d = mi.make_bf16(cfg, seed=10)
    w2 = d["w2"].copy()
    w2[1] = 0
    out = oracle_lib.forward_bf16(d["x"], d["w1"], w2, d["topk_ids"], d["topk_weights"])
    ids = d["topk_ids"].copy()
    ids[ids == 1] = -1
    out2 = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], ids, d["topk_weights"])
    assert np.array_equal(out, out2)


def test_out_of_range_ids_are_dropped(oracle_lib):
    cfg = mi.custom(10, 64, 32, 4, 2)
    d = mi.make_bf16(cfg, seed=11)
    ids = d["topk_ids"].copy()
    ids[::2, 1] = 4          # == E: out of range
    ids[1::3, 0] = -5
    wz = d["topk_weights"].copy()
    wz[ids < 0] = 0
    wz[ids >= 4] = 0
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], ids, d["topk_weights"])
    ref = dense_reference_fp64(d["x"], d["w1"], d["w2"], np.where((ids >= 0) & (ids < 4), ids, 0),
                               wz)
    _check_close_to_fp64(out, ref)


def test_duplicate_ids_count_once_per_slot(oracle_lib):
    """The same expert in several slots of one token: the pass sums over the
    token's slots, so expert e's output enters once per slot with that slot's
    weight (the dense reference's M[t, e] adds the weights of every slot on e)."""
    cfg = mi.custom(24, 64, 96, 5, 4, "uniform")
    d = mi.make_bf16(cfg, seed=13)
    ids = d["topk_ids"].copy()
    ids[::2, 1] = ids[::2, 0]
    ids[::3, 3] = ids[::3, 0]
    ids[5, :] = 2
    out = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], ids, d["topk_weights"])
    _check_close_to_fp64(out, dense_reference_fp64(d["x"], d["w1"], d["w2"], ids, d["topk_weights"]))
    # one expert in every slot with weights summing to 1 is that expert's
    # output alone (up to fp32 rounding of the four products' sum)
    one = np.zeros((24, 1), np.int32) + 2
    single = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], one, np.ones((24, 1), np.float32))
    w5 = d["topk_weights"][5].astype(np.float64)
    assert abs(w5.sum() - 1.0) < 1e-6
    a, b = _f32(out[5]), _f32(single[5])
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-6 * np.abs(b).max())


def test_sampled_tokens_match_full_run(oracle_lib):
    cfg = mi.custom(40, 64, 64, 5, 2)
    d = mi.make_bf16(cfg, seed=12)
    full = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    tok = np.array([39, 0, 17, 5])
    part = oracle_lib.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"],
                                   tokens=tok)
    assert np.array_equal(part[tok], full[tok])


# ---------------- route maps ----------------

def _route_brute(ids, E):
    flat = ids.reshape(-1)
    valid = [p for p in range(flat.size) if 0 <= flat[p] < E]
    order = sorted(valid, key=lambda p: (int(flat[p]), p))
    counts = np.bincount(flat[valid].astype(np.int64), minlength=E) if valid else np.zeros(E, int)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return counts, offsets, order


@pytest.mark.parametrize("T,E,k,routing", [(64, 8, 2, "softmax"), (100, 32, 8, "uniform"),
                                           (333, 128, 8, "zipf"), (1, 4, 4, "uniform"),
                                           (50, 1, 1, "softmax")])
def test_route_matches_python_sort(oracle_lib, T, E, k, routing):
    ids, _ = mi.routing(mi.custom(T, 64, 64, E, k, routing))
    counts, offsets, s2p, p2s = oracle_lib.route(ids, E)
    bc, bo, order = _route_brute(ids, E)
    assert np.array_equal(counts, bc)
    assert np.array_equal(offsets, bo)
    assert list(s2p[:len(order)]) == order
    assert np.all(s2p[len(order):] == -1)
    for i, p in enumerate(order):
        assert p2s[p] == i
    # invariants: segments hold their expert, maps are inverse permutations
    flat = ids.reshape(-1)
    for e in range(E):
        assert np.all(flat[s2p[offsets[e]:offsets[e + 1]]] == e)
    assert np.array_equal(p2s[s2p[:offsets[E]]], np.arange(offsets[E]))


def test_route_dropped_and_skewed(oracle_lib):
    ids = np.full((40, 3), 2, np.int32)
    ids[5, 1] = -1
    ids[7, 2] = 9
    counts, offsets, s2p, p2s = oracle_lib.route(ids, 4)
    assert counts.tolist() == [0, 0, 118, 0]
    assert offsets.tolist() == [0, 0, 0, 118, 118]
    assert p2s[5 * 3 + 1] == -1 and p2s[7 * 3 + 2] == -1
    assert list(s2p[:118]) == [p for p in range(120) if p not in (16, 23)]


def test_route_empty(oracle_lib):
    counts, offsets, s2p, p2s = oracle_lib.route(np.zeros((0, 4), np.int32), 5)
    assert counts.tolist() == [0] * 5 and offsets.tolist() == [0] * 6
    assert s2p.size == 0 and p2s.size == 0
