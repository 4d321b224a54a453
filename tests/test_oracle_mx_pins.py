"""Pins of the oracle's MX-fp8 pieces: the e4m3fn format (golden points
from the format's definition), round-to-nearest-even by brute-force search
over all 256 codes, the e8m0 scale rule, and the MX forward against the
already pinned bf16 oracle.

Scale rule (MXQ), read from "Porting Block-Scaled GEMM Kernels from
Blackwell to Rubin", section 6.2: the scale is the power of two found by
rounding amax/448 up, i.e. s = the smallest integer with amax <= 448 * 2^s;
codes are e4m3fn(v * 2^-s) with round-to-nearest-even and saturation.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_points.json")


@pytest.fixture(scope="module")
def table(oracle_lib):
    return np.array([oracle_lib.e4m3_decode(c) for c in range(256)], np.float64)


def test_e4m3_golden_points(oracle_lib):
    pts = json.load(open(GOLDEN))["points"]
    for p in pts:
        v = oracle_lib.e4m3_decode(p["code"])
        if p["value"] == "nan":
            assert math.isnan(v), p
        else:
            assert v == p["value"] and math.copysign(1, v) == math.copysign(1, p["value"]), p


def test_e4m3_table_shape(table):
    pos = table[:127]                      # codes 0x00..0x7E
    assert np.all(np.diff(pos) > 0)        # strictly increasing
    assert np.array_equal(table[128:255], -pos)
    assert np.isnan(table[127]) and np.isnan(table[255])
    # each binade above the subnormals holds 8 evenly spaced values
    for ex in range(1, 16):
        vals = pos[ex * 8: ex * 8 + 8] if ex < 15 else pos[120:127]
        steps = np.diff(vals)
        assert np.allclose(steps, steps[0])


def _nearest_even_brute(v, table):
    """Nearest finite e4m3 value by search; ties go to the even code; |v| >= 448 saturates."""
    if abs(v) >= 448.0:
        return 0x7E | (0x80 if math.copysign(1, v) < 0 else 0)
    cands = [c for c in range(256) if not math.isnan(table[c])]
    best = min(abs(table[c] - v) for c in cands)
    tied = [c for c in cands if abs(table[c] - v) == best]
    # among equal magnitudes prefer the sign of v (only matters at 0)
    same_sign = [c for c in tied if (c >> 7) == (1 if math.copysign(1, v) < 0 else 0)]
    tied = same_sign or tied
    even = [c for c in tied if c % 2 == 0]
    return (even or tied)[0]


def test_e4m3_encode_rne_brute_force(oracle_lib, table):
    rng = np.random.default_rng(0)
    vals = list(rng.normal(0, 50, 400)) + list(rng.normal(0, 0.01, 200))
    pos = table[:127]
    mids = list((pos[1:] + pos[:-1]) / 2)        # exact ties
    vals += mids + [-m for m in mids]
    vals += list(pos) + [-v for v in pos[1:]]
    vals += [448.0, 449.0, 463.9, 464.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11,
             0.0, -0.0, 1e-30]
    for v in vals:
        v32 = float(np.float32(v))
        assert oracle_lib.e4m3_encode(v32) == _nearest_even_brute(v32, table), v32


def test_scale_rule_boundaries(oracle_lib):
    for s in (-20, -9, -1, 0, 1, 5):
        blk = np.zeros(32, np.float32)
        blk[3] = 448.0 * 2.0 ** s
        assert oracle_lib.mx_scale_exp(blk) == s
        blk[3] = np.nextafter(np.float32(448.0 * 2.0 ** s), np.float32(np.inf))
        assert oracle_lib.mx_scale_exp(blk) == s + 1
        blk[3] = -448.0 * 2.0 ** s * 0.5000001
        assert oracle_lib.mx_scale_exp(blk) == s
    assert oracle_lib.mx_scale_exp(np.zeros(32, np.float32)) == -127
    assert oracle_lib.mx_scale_exp(np.full(32, 1e-45, np.float32)) == -127   # clamped


def test_quantize_properties(oracle_lib, table):
    rng = np.random.default_rng(1)
    src = (rng.standard_normal((64, 256)) * np.exp(rng.normal(0, 3, (64, 1)))).astype(np.float32)
    codes, scales = oracle_lib.mx_quantize(src)
    assert codes.shape == src.shape and scales.shape == (64, 8)
    deq = table[codes] * 2.0 ** (scales.astype(np.float64)[:, :, None].repeat(32, 2).reshape(64, 256) - 127)
    blocks = src.reshape(64, 8, 32).astype(np.float64)
    amax = np.abs(blocks).max(-1)
    s = scales.astype(np.float64) - 127
    # smallest s with amax <= 448 * 2^s: the block max lands in (224, 448]
    top = amax * 2.0 ** -s
    assert np.all(top <= 448.0) and np.all(top > 224.0)
    # relative error of RNE to 3 mantissa bits, plus the subnormal floor
    err = np.abs(deq - src)
    assert np.all(err <= 2.0 ** -4 * np.abs(src) + 2.0 ** -10 * 2.0 ** np.repeat(s, 32, 1))


def test_quantize_roundtrips_representable_blocks(oracle_lib, table):
    rng = np.random.default_rng(2)
    finite = [c for c in range(256) if not math.isnan(table[c])]
    codes = rng.choice(finite, size=(16, 64)).astype(np.uint8)
    codes[:, 0] = 0x7E                         # block max 448 -> scale exactly s
    codes[:, 32] = 0xFE
    s = rng.integers(-30, 30, size=(16, 2))
    vals = table[codes] * 2.0 ** np.repeat(s, 32, 1)
    c2, s2 = oracle_lib.mx_quantize(vals.astype(np.float32))
    assert np.array_equal(s2.astype(int) - 127, s)
    assert np.array_equal(table[c2], table[codes])   # same values (+-0 may differ in sign only)


def _dequant(codes, scales, table):
    K = codes.shape[-1]
    sc = np.repeat(scales.astype(np.float64) - 127, 32, axis=-1).reshape(codes.shape)
    return table[codes] * 2.0 ** sc


@pytest.mark.parametrize("requant", [False, True])
def test_mx_forward_against_bf16_oracle(oracle_lib, table, requant):
    """Without the act requant, the MX oracle on MX inputs equals the bf16
    oracle on the same values written as bf16 (every e4m3 value times a
    power of two at these magnitudes is a bf16 number); with it, the two
    stay close (cosine >= 0.999)."""
    cfg = mi.custom(24, 128, 96, 4, 2, dtype="mxfp8")
    s = mi.make_mx_sources(cfg, seed=4)
    q = {n: oracle_lib.mx_quantize(s[n]) for n in ("x", "w1", "w2")}
    deq = {n: _dequant(*q[n], table).astype(np.float32) for n in q}
    bits = {n: mi.to_bf16_bits(deq[n]) for n in deq}
    for n in deq:
        assert np.array_equal(mi.bf16_bits_to_f32(bits[n]), deq[n])
    ref = oracle_lib.forward_bf16(bits["x"], bits["w1"], bits["w2"], s["topk_ids"],
                                  s["topk_weights"])
    out = oracle_lib.forward_mx(*q["x"], *q["w1"], *q["w2"], s["topk_ids"], s["topk_weights"],
                                requant=requant)
    if not requant:
        assert np.array_equal(out, ref)
    else:
        a = mi.bf16_bits_to_f32(out).astype(np.float64).ravel()
        b = mi.bf16_bits_to_f32(ref).astype(np.float64).ravel()
        cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
        assert 0.999 <= cos < 1.0
        assert not np.array_equal(out, ref)


def test_mx_act_requant_is_per_32_along_h(oracle_lib, table):
    """k=1, w=1 and W2 = identity (D = H): the output is exactly the
    requantized SwiGLU output, which must equal MXQ of an fp64 evaluation of
    silu(gate) * up (a code may differ only where fp32 and fp64 fall on
    different sides of a rounding boundary)."""
    T, D, H, E = 16, 64, 64, 2
    rng = np.random.default_rng(3)
    x = rng.standard_normal((T, D)).astype(np.float32)
    w1 = (rng.standard_normal((E, 2 * H, D)) / 8).astype(np.float32)
    xq, w1q = oracle_lib.mx_quantize(x), oracle_lib.mx_quantize(w1)
    eye = np.zeros((E, D, H), np.float32)
    for e in range(E):
        np.fill_diagonal(eye[e], 1.0)
    w2q = oracle_lib.mx_quantize(eye)
    ids = (np.arange(T) % E).astype(np.int32)[:, None]
    wts = np.ones((T, 1), np.float32)
    out = mi.bf16_bits_to_f32(oracle_lib.forward_mx(*xq, *w1q, *w2q, ids, wts))
    X, W1 = _dequant(*xq, table), _dequant(*w1q, table)
    exp = np.zeros((T, H))
    for t in range(T):
        gu = W1[ids[t, 0]] @ X[t]
        g, u = gu[:H], gu[H:]
        exp[t] = g / (1 + np.exp(-g)) * u
    ec, es = oracle_lib.mx_quantize(exp.astype(np.float32))
    expect = _dequant(ec, es, table)
    mismatch = np.mean(out != expect)
    assert mismatch <= 0.01, mismatch
