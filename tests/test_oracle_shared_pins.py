"""Pins of the CPU oracle's shared expert ("GC-MoE on SM120", section 4.7: a
shared expert runs on every token and its output joins the same fp32 sum as
the k routed slots, with weight 1) against an independent dense fp64
evaluation and against the routed pass itself.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.test_oracle_pins import _check_close_to_fp64, _f32, dense_reference_fp64


def dense_ffn_fp64(x, ws1, ws2):
    """silu(x Wg^T) * (x Wu^T) @ Ws2^T in fp64 with numpy matmuls."""
    X, W1, W2 = _f32(x), _f32(ws1), _f32(ws2)
    Hs = W1.shape[0] // 2
    g, u = X @ W1[:Hs].T, X @ W1[Hs:].T
    return (g / (1.0 + np.exp(-g)) * u) @ W2.T


@pytest.mark.parametrize("T,D,H,E,k,Hs", [(16, 64, 32, 4, 2, 32), (9, 96, 64, 5, 3, 128), (12, 32, 96, 3, 1, 48)])
def test_shared_expert_adds_a_dense_ffn(T, D, H, E, k, Hs):
    cfg = mi.custom(T, D, H, E, k, "softmax")
    d = mi.make_bf16(cfg, 0)
    ws1, ws2 = mi.shared_expert(cfg, Hs, 0)
    out = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], shared=(ws1, ws2))
    ref = dense_reference_fp64(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"]) + \
        dense_ffn_fp64(d["x"], ws1, ws2)
    _check_close_to_fp64(out, ref)
    # with every routed weight zero only the shared expert remains
    zero = np.zeros_like(d["topk_weights"])
    out0 = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], zero, shared=(ws1, ws2))
    _check_close_to_fp64(out0, dense_ffn_fp64(d["x"], ws1, ws2))


def test_shared_expert_equals_an_extra_slot():
    """A shared expert with expert e's weights is the routed pass with one more
    slot per token on e with weight 1, summed last: bit for bit."""
    cfg = mi.custom(20, 64, 64, 4, 2, "softmax")
    d = mi.make_bf16(cfg, 0)
    e = 2
    shared = (d["w1"][e], d["w2"][e])
    out = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], shared=shared)
    ids = np.concatenate([d["topk_ids"], np.full((cfg.T, 1), e, np.int32)], axis=1)
    wts = np.concatenate([d["topk_weights"], np.ones((cfg.T, 1), np.float32)], axis=1)
    np.testing.assert_array_equal(out, oracle.forward_bf16(d["x"], d["w1"], d["w2"], ids, wts))


def test_shared_expert_token_subset():
    cfg = mi.custom(30, 64, 32, 4, 2, "zipf")
    d = mi.make_bf16(cfg, 0)
    sh = mi.shared_expert(cfg, 64, 0)
    full = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], shared=sh)
    tok = np.array([0, 7, 29])
    part = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], tokens=tok, shared=sh)
    np.testing.assert_array_equal(part[tok], full[tok])
