"""Pins of the oracle's MXFP4-weight pieces: the e2m1 format (its value set,
tests/golden/e2m1_values.json), round-to-nearest-even by brute-force search
over the 8 magnitudes, the MXQ4 scale rule, the nibble packing, and the
fp4-weight forward against the already pinned MX-fp8 forward on weights
that both formats hold exactly.

MXFP4 ("GC-MoE on SM120", scale formats): weights as E2M1 codes (4 bits
each) in blocks of 32 along K, each block carrying one UE8M0 power-of-two
scale; activations stay MX-fp8. The
pages give no fp4 scale rule; MXQ4 reads the MX-fp8 rule with E2M1's
largest magnitude 6 in place of 448: s = the smallest integer with
amax <= 6 * 2^s, codes e2m1(v * 2^-s), nearest with ties to the even code.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs as mi

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.json")))
MAGS = GOLDEN["magnitudes_by_code"]


def test_e2m1_values(oracle_lib):
    for c in range(16):
        v = oracle_lib.e2m1_decode(c)
        mag = MAGS[c & 7]
        sign = -1.0 if c & GOLDEN["sign_bit"] else 1.0
        assert v == sign * mag and math.copysign(1, v) == sign, (c, v)


def _brute(v):
    """Nearest e2m1 code by search over the 8 magnitudes, ties to the even code, saturating at 6."""
    a = abs(v)
    if a >= 6.0:
        return 7 | (8 if math.copysign(1, v) < 0 else 0)
    best = min(abs(m - a) for m in MAGS)
    tied = [c for c in range(8) if abs(MAGS[c] - a) == best]
    even = [c for c in tied if c % 2 == 0]
    c = (even or tied)[0]
    return c | (8 if math.copysign(1, v) < 0 else 0)


def test_e2m1_encode_rne_brute_force(oracle_lib):
    rng = np.random.default_rng(3)
    mids = [(MAGS[i] + MAGS[i + 1]) / 2 for i in range(7)]
    vals = [0.0, -0.0, 6.0, 6.5, 7.0, 100.0, 1e30] + mids + [np.nextafter(np.float32(m), np.float32(0)) for m in mids] \
        + [np.nextafter(np.float32(m), np.float32(10)) for m in mids] + list(rng.uniform(-7, 7, 400)) \
        + list(rng.uniform(-1, 1, 200))
    for v in vals:
        v = float(np.float32(v))
        for s in (v, -v):
            assert oracle_lib.e2m1_encode(s) == _brute(s), s
    # the ties named: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0
    for v, want in ((0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0)):
        assert oracle_lib.e2m1_decode(oracle_lib.e2m1_encode(v)) == want, v


def test_mx4_scale_rule_boundaries(oracle_lib):
    def block(amax):
        b = np.zeros(32, np.float32)
        b[7] = amax
        b[3] = -amax / 3
        return b
    for s in (-20, -3, 0, 1, 5, 30):
        edge = np.float32(6.0 * 2.0 ** s)
        assert oracle_lib.mx4_scale_exp(block(edge)) == s
        assert oracle_lib.mx4_scale_exp(block(np.nextafter(edge, np.float32(np.inf)))) == s + 1
        assert oracle_lib.mx4_scale_exp(block(np.float32(4.0 * 2.0 ** s))) == s     # 4*2^s <= 6*2^s, > 6*2^(s-1)
        assert oracle_lib.mx4_scale_exp(block(np.float32(3.0 * 2.0 ** s))) == s - 1  # 3*2^s == 6*2^(s-1)
    assert oracle_lib.mx4_scale_exp(np.zeros(32, np.float32)) == -127
    assert oracle_lib.mx4_scale_exp(block(np.float32(1e-44))) == -127               # clamped
    assert oracle_lib.mx4_scale_exp(block(np.float32(3e38))) == 126                 # 6 * 2^126 ~ 5.1e38


def test_mx4_packing_even_index_low_nibble(oracle_lib):
    for k in range(64):
        src = np.zeros((1, 64), np.float32)
        src[0, k] = 3.0
        codes, scales = oracle_lib.mx4_quantize(src)
        assert codes.shape == (1, 32) and scales.shape == (1, 2)
        byte = int(codes[0, k // 2])
        nib = byte & 15 if k % 2 == 0 else byte >> 4
        other = byte >> 4 if k % 2 == 0 else byte & 15
        assert MAGS[nib & 7] * 2.0 ** (int(scales[0, k // 32]) - 127) == 3.0 and other == 0, k
        assert np.count_nonzero(codes) == 1


def test_mx4_quantize_roundtrips_representable_blocks(oracle_lib):
    rng = np.random.default_rng(4)
    for _ in range(200):
        s = int(rng.integers(-30, 30))
        mags = rng.choice(MAGS, 32)
        mags[rng.integers(32)] = 6.0                      # the block's amax is 6 * 2^s
        v = (mags * np.where(rng.random(32) < 0.5, -1, 1) * 2.0 ** s).astype(np.float32)
        codes, scales = oracle_lib.mx4_quantize(v[None])
        assert int(scales[0, 0]) - 127 == s
        dq = np.array([oracle_lib.e2m1_decode((int(codes[0, i // 2]) >> (4 * (i % 2))) & 15) for i in range(32)])
        assert np.array_equal(dq * 2.0 ** s, v.astype(np.float64))


def _shared_weights(rng, rows, K):
    """Weights whose values both e2m1 (with its scale) and e4m3 (with its scale) hold exactly:
    e2m1 magnitudes times 2^s per 32-block, each block's amax 6 * 2^s."""
    v = rng.choice(MAGS, (rows, K)) * np.where(rng.random((rows, K)) < 0.5, -1.0, 1.0)
    v = v.reshape(rows, K // 32, 32)
    v[:, :, 5] = 6.0
    s = rng.integers(-9, -3, (rows, K // 32, 1))
    return (v * 2.0 ** s).reshape(rows, K).astype(np.float32)


@pytest.mark.parametrize("T,D,H,E,k", [(37, 64, 64, 3, 2), (20, 128, 96, 4, 3)])
def test_mx4_forward_equals_mx8_forward_on_shared_values(oracle_lib, T, D, H, E, k):
    rng = np.random.default_rng([T, D, H])
    w1 = _shared_weights(rng, E * 2 * H, D).reshape(E, 2 * H, D)
    w2 = _shared_weights(rng, E * D, H).reshape(E, D, H)
    x = rng.standard_normal((T, D)).astype(np.float32)
    cfg = mi.custom(T, D, H, E, k, "softmax")
    ids, wts = mi.routing(cfg, 0)
    xc, xs = oracle_lib.mx_quantize(x)
    w1c8, w1s8 = oracle_lib.mx_quantize(w1)
    w2c8, w2s8 = oracle_lib.mx_quantize(w2)
    w1c4, w1s4 = oracle_lib.mx4_quantize(w1)
    w2c4, w2s4 = oracle_lib.mx4_quantize(w2)
    assert w1c4.shape == (E, 2 * H, D // 2) and w2c4.shape == (E, D, H // 2)
    for req in (True, False):
        o8 = oracle_lib.forward_mx(xc, xs, w1c8, w1s8, w2c8, w2s8, ids, wts, requant=req)
        o4 = oracle_lib.forward_mx4(xc, xs, w1c4, w1s4, w2c4, w2s4, ids, wts, requant=req)
        assert np.array_equal(o4, o8)
        assert np.count_nonzero(o4) > 0


def test_mx4_forward_dense_reduction(oracle_lib):
    """E = 1, k = 1, w = 1 with requant off: a dense SwiGLU FFN of the dequantized operands (numpy fp64)."""
    rng = np.random.default_rng(8)
    T, D, H = 9, 64, 64
    w1 = (rng.standard_normal((1, 2 * H, D)) / 8).astype(np.float32)
    w2 = (rng.standard_normal((1, D, H)) / 8).astype(np.float32)
    x = rng.standard_normal((T, D)).astype(np.float32)
    xc, xs = oracle_lib.mx_quantize(x)
    w1c, w1s = oracle_lib.mx4_quantize(w1)
    w2c, w2s = oracle_lib.mx4_quantize(w2)

    def deq4(c, s, K):
        lo, hi = c & 15, c >> 4
        codes = np.stack([lo, hi], -1).reshape(c.shape[:-1] + (K,))
        mags = np.array(MAGS)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
        return mags * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, -1)

    xd = np.array([oracle_lib.e4m3_decode(c) for c in range(256)])[xc] * np.repeat(2.0 ** (xs - 127.0), 32, -1)
    W1, W2 = deq4(w1c, w1s, D)[0], deq4(w2c, w2s, H)[0]
    gu = xd @ W1.T
    act = gu[:, :H] / (1 + np.exp(-gu[:, :H])) * gu[:, H:]
    ref = act @ W2.T
    out = oracle_lib.forward_mx4(xc, xs, w1c, w1s, w2c, w2s, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32),
                                 requant=False)
    got = mi.bf16_bits_to_f32(out).astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max()
