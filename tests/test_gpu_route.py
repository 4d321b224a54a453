"""Route step on the GPU (moe_ffn_route through the C ABI): the index maps
must equal the oracle's stable counting sort bit for bit."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.parity import to_gpu

pytestmark = pytest.mark.gpu


def _check(ids: np.ndarray, E: int):
    import grouped_gemm_amd as g
    print(f"route T={ids.shape[0]} k={ids.shape[1]} E={E}", flush=True)
    counts, offsets, s2p, p2s = g.moe_ffn_route(to_gpu(ids), E)
    rc, ro, rs, rp = oracle.route(ids, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(s2p.cpu().numpy(), rs)
    assert np.array_equal(p2s.cpu().numpy(), rp)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_route_configs(cid):
    cfg = mi.CONFIGS[cid]
    ids, _ = mi.routing(cfg)
    _check(ids, cfg.E)


@pytest.mark.parametrize("T,E,k,routing", [
    (1, 8, 2, "softmax"), (1, 4, 4, "uniform"), (77, 16, 1, "softmax"), (129, 8, 8, "uniform"),
    (1000, 256, 6, "zipf"), (3000, 1024, 8, "uniform"), (5, 8192, 3, "uniform"),
])
def test_route_edge_shapes(T, E, k, routing):
    ids, _ = mi.routing(mi.custom(T, 128, 128, E, k, routing))
    _check(ids, E)


def test_route_all_on_one_expert_and_empty_experts():
    ids = np.full((5000, 2), 3, np.int32)
    _check(ids, 16)


def test_route_dropped_ids():
    rng = np.random.default_rng(4)
    ids = rng.integers(-3, 11, size=(2049, 4)).astype(np.int32)   # E = 8: some out of range
    _check(ids, 8)


@pytest.mark.parametrize("T,E,k", [(32, 64, 8), (33, 64, 8), (20, 65, 8), (31, 64, 2)])
def test_route_one_wave_limits(T, E, k):
    # up to 256 pairs and 64 experts one wave routes the batch; just past either limit one workgroup does
    ids, _ = mi.routing(mi.custom(T, 128, 128, E, k, "uniform"))
    _check(ids, E)


def test_route_dropped_ids_one_wave():
    rng = np.random.default_rng(6)
    ids = rng.integers(-3, 11, size=(60, 4)).astype(np.int32)     # E = 8, 240 pairs
    _check(ids, 8)


def test_route_large_segments():
    """P large enough that the segment length grows past its minimum."""
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 2048, size=(600000, 8)).astype(np.int32)
    _check(ids, 2048)


def test_route_repeatable():
    import grouped_gemm_amd as g
    ids, _ = mi.routing(mi.CONFIGS[3])
    t = to_gpu(ids)
    a = [x.cpu().numpy() for x in g.moe_ffn_route(t, 128)]
    b = [x.cpu().numpy() for x in g.moe_ffn_route(t, 128)]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
