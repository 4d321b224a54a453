"""Pins of the CPU oracle's activation variant ("Porting Block-Scaled GEMM
Kernels from Blackwell to Rubin", section 5.3: gate and up scaled by the
expert's global scale alpha, clamped gpt-oss style -- the gate from above
only, up on both sides -- then up * silu(gate); "GC-MoE on SM120", section
4.8: the route weight multiplies gate and up before the activation) against
an independent dense fp64 evaluation and against the plain pass."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.test_oracle_pins import _check_close_to_fp64, _f32


def dense_variant_fp64(x, w1, w2, ids, wts, kind, limit, alpha, wba):
    """Every expert on every token in fp64 with numpy matmuls, then the
    token's slots picked out; the activation written from its definition."""
    X, W1, W2 = _f32(x), _f32(w1), _f32(w2)
    T, D = X.shape
    E, H2, _ = W1.shape
    H = H2 // 2
    out = np.zeros((T, D))
    for e in range(E):
        gu = X @ W1[e].T
        for t in range(T):
            for j in range(ids.shape[1]):
                if ids[t, j] != e:
                    continue
                w = float(wts[t, j])
                s = (alpha[e] if alpha is not None else 1.0) * (w if wba else 1.0)
                g, u = s * gu[t, :H], s * gu[t, H:]
                if kind == 1:
                    g = np.minimum(g, limit)
                    u = np.clip(u, -limit, limit)
                act = g / (1.0 + np.exp(-g)) * u
                out[t] += (1.0 if wba else w) * (act @ W2[e].T)
    return out


def _data(T=14, D=64, H=32, E=4, k=2, seed=0):
    cfg = mi.custom(T, D, H, E, k, "softmax")
    return mi.make_bf16(cfg, seed)


def test_default_variant_is_the_plain_pass():
    d = _data()
    a = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    b = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    np.testing.assert_array_equal(a, b)
    # a clamp nothing reaches changes nothing
    c = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], kind=1, limit=1e30)
    np.testing.assert_array_equal(c, b)


@pytest.mark.parametrize("kind,limit,use_alpha,wba", [
    (1, 0.5, False, False), (1, 0.2, True, False), (0, 0.0, True, True), (1, 0.3, True, True), (1, 1e30, False, True),
])
def test_variant_matches_dense_fp64(kind, limit, use_alpha, wba):
    d = _data()
    alpha = np.array([1.5, 0.5, 2.0, 0.75], np.float32) if use_alpha else None
    out = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], kind, limit, alpha,
                                  wba)
    ref = dense_variant_fp64(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], kind, limit, alpha, wba)
    _check_close_to_fp64(out, ref)


def test_clamp_bites():
    """With a small limit the clamp changes the result (a wrong clamp side or
    a missing clamp would not pass the dense comparison above either)."""
    d = _data()
    a = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], kind=1, limit=0.1)
    b = oracle.forward_bf16(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"])
    assert np.mean(a != b) > 0.5


def test_alpha_is_a_scale_of_w1():
    """alpha[e] = 2^j scales gate and up exactly like scaling W1[e] by 2^j
    (exact in bf16): bit-equal outputs."""
    d = _data()
    alpha = np.array([2.0, 0.5, 4.0, 1.0], np.float32)
    a = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], d["topk_weights"], kind=1, limit=0.4,
                                alpha=alpha)
    w1s = mi.to_bf16_bits(mi.bf16_bits_to_f32(d["w1"]) * alpha[:, None, None])
    b = oracle.forward_bf16_act(d["x"], w1s, d["w2"], d["topk_ids"], d["topk_weights"], kind=1, limit=0.4)
    np.testing.assert_array_equal(a, b)


def test_weight_before_activation_with_unit_weights():
    """With every routing weight 1 the weight's placement does not matter."""
    d = _data(k=1)
    ones = np.ones_like(d["topk_weights"])
    a = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], ones, kind=1, limit=0.3,
                                weight_before_act=True)
    b = oracle.forward_bf16_act(d["x"], d["w1"], d["w2"], d["topk_ids"], ones, kind=1, limit=0.3)
    np.testing.assert_array_equal(a, b)
