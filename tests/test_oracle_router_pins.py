"""Pins of the CPU oracle's router (softmax -> top-k -> renormalize) against
things other than itself: numpy's stable sort, the closed forms of k = 1,
k = 2 and k = E, shift invariance of softmax, hand-made ties, and the input
generator's independent fp64 softmax-top-k (Prime Flash MoE, section 1 "The
computation": each token's top-k experts with normalized routing weights).
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle


def _softmax64(l):
    z = np.asarray(l, np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("T,E,k", [(200, 8, 2), (150, 32, 8), (64, 128, 8), (40, 64, 6), (17, 1000, 5), (9, 3, 3)])
def test_router_ids_match_stable_sort(T, E, k):
    rng = np.random.default_rng([T, E, k])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, wts = oracle.router(logits, k)
    # brute force: a full stable sort of -logits (lower id first among equals)
    ref_ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref_ids)
    # weights: full fp64 softmax over E, the selected entries, renormalized
    p = _softmax64(logits)
    sel = np.take_along_axis(p, ref_ids, axis=1)
    ref_w = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(wts, ref_w, rtol=2e-7, atol=1e-30)
    assert np.all(np.diff(wts, axis=1) <= 0)
    np.testing.assert_allclose(wts.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)


def test_router_ties_go_to_the_lower_id():
    logits = np.array([[1.0, 3.0, 3.0, 2.0],
                       [0.0, 0.0, 0.0, 0.0],
                       [5.0, -1.0, 5.0, 5.0],
                       [-2.0, -2.0, 7.0, -2.0]], np.float32)
    ids, wts = oracle.router(logits, 2)
    np.testing.assert_array_equal(ids, [[1, 2], [0, 1], [0, 2], [2, 0]])
    np.testing.assert_array_equal(wts[:3], np.full((3, 2), 0.5, np.float32))
    # integer logits from a small range: many ties, still the stable order
    rng = np.random.default_rng(7)
    many = rng.integers(-3, 4, size=(300, 40)).astype(np.float32)
    ids, _ = oracle.router(many, 7)
    np.testing.assert_array_equal(ids, np.argsort(-many, axis=1, kind="stable")[:, :7])


def test_router_special_values():
    """-inf ranks after finite logits; NaN after everything (numpy's sort
    agrees); -0 and +0 tie and go to the lower id."""
    logits = np.array([[np.nan, 1.0, -np.inf, 0.0],
                       [-0.0, 0.0, -1.0, np.nan],
                       [0.0, -0.0, np.nan, np.nan]], np.float32)
    ids, wts = oracle.router(logits, 4)
    np.testing.assert_array_equal(ids, np.argsort(-logits, axis=1, kind="stable"))
    np.testing.assert_array_equal(ids, [[1, 3, 2, 0], [0, 1, 2, 3], [0, 1, 2, 3]])
    assert np.isnan(wts).all()                   # a NaN among the picks
    ids, wts = oracle.router(logits, 3)
    np.testing.assert_array_equal(ids[0], [1, 3, 2])
    e = np.e
    np.testing.assert_allclose(wts[0], [e / (e + 1), 1 / (e + 1), 0.0], rtol=1e-7)
    np.testing.assert_allclose(wts[1], np.array([1, 1, np.exp(-1.0)]) / (2 + np.exp(-1.0)), rtol=1e-7)


def test_router_closed_forms():
    rng = np.random.default_rng(11)
    logits = rng.normal(0.0, 3.0, size=(100, 16)).astype(np.float32)
    # k = 1: the arg-max with weight exactly 1
    ids, wts = oracle.router(logits, 1)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(logits, axis=1))
    np.testing.assert_array_equal(wts, np.ones((100, 1), np.float32))
    # k = 2: the weights are sigmoid(a - b) and sigmoid(b - a)
    ids, wts = oracle.router(logits, 2)
    a = np.take_along_axis(logits, ids[:, :1], axis=1)[:, 0].astype(np.float64)
    b = np.take_along_axis(logits, ids[:, 1:], axis=1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(wts[:, 0], 1.0 / (1.0 + np.exp(b - a)), rtol=2e-7)
    np.testing.assert_allclose(wts[:, 1], 1.0 / (1.0 + np.exp(a - b)), rtol=2e-7)
    # k = E: the weights are the softmax itself, in sorted order
    ids, wts = oracle.router(logits, 16)
    p = _softmax64(logits)
    np.testing.assert_allclose(wts, np.take_along_axis(p, ids, axis=1), rtol=2e-7)
    np.testing.assert_array_equal(np.sort(ids, axis=1), np.tile(np.arange(16), (100, 1)))


def test_router_shift_invariance():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((80, 24)).astype(np.float32)
    ids0, w0 = oracle.router(logits, 4)
    # adding a power of two keeps the order (exact for these magnitudes) and
    # cancels in the softmax
    ids1, w1 = oracle.router(logits + np.float32(8.0), 4)
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_allclose(w0, w1, rtol=2e-6)


@pytest.mark.parametrize("cid", [1, 3, 4])
def test_router_agrees_with_generator(cid):
    """The generator's fp64 softmax-top-k on the same draws (an independent
    implementation) picks the same experts and weights up to fp32 rounding."""
    base = mi.CONFIGS[cid]
    cfg = mi.custom(min(base.T, 512), base.D, base.H, base.E, base.k, base.routing, cid=base.cid)
    ids_g, w_g = mi.routing(cfg, 0)
    ids, wts = oracle.router(mi.router_logits(cfg, 0), cfg.k)
    np.testing.assert_array_equal(ids, ids_g)
    np.testing.assert_allclose(wts, w_g, rtol=1e-5, atol=1e-7)


def test_router_zipf_prior_skews_toward_low_ids():
    cfg = mi.custom(2048, 64, 64, 128, 8, "zipf", cid=4)
    ids, _ = oracle.router(mi.router_logits(cfg, 0), 8)
    h = np.bincount(ids.reshape(-1), minlength=128)
    assert h[0] > h[10] > h[100]
