"""The seeded generator: determinism and the stated routing recipes."""
import numpy as np
import pytest

import moe_inputs as mi


def test_same_seed_same_bytes():
    cfg = mi.custom(33, 64, 96, 5, 2)
    a, b = mi.make_bf16(cfg, 1), mi.make_bf16(cfg, 1)
    for n in a:
        assert np.array_equal(a[n], b[n])
    c = mi.make_bf16(cfg, 2)
    assert not np.array_equal(a["x"], c["x"])


def test_bf16_rounding_is_rne():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    assert mi.to_bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]


@pytest.mark.parametrize("routing", ["softmax", "uniform", "zipf"])
def test_routing_recipes(routing):
    cfg = mi.custom(2000, 64, 64, 16, 4, routing)
    ids, w = mi.routing(cfg)
    assert ids.shape == w.shape == (2000, 4) and ids.dtype == np.int32 and w.dtype == np.float32
    assert np.all((ids >= 0) & (ids < 16))
    assert all(len(set(r)) == 4 for r in ids.tolist())          # distinct experts
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    if routing != "uniform":
        assert np.all(np.diff(w, axis=1) <= 0)                 # descending probability
    hist = mi.expert_histogram(ids, 16)
    if routing == "zipf":
        assert hist[0] > hist[-1] * 3                           # expert 0 most popular
    else:
        assert hist.min() > 0.5 * hist.mean()


def test_config_table():
    c = mi.CONFIGS
    assert (c[2].T, c[2].D, c[2].H, c[2].E, c[2].k) == (64, 6144, 2048, 32, 8)
    assert c[4].P == 1048576 and c[5].dtype == "mxfp8"
    assert abs(c[4].flops - 9.8956e12) / 9.8956e12 < 1e-3
