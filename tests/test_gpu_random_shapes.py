"""Seeded random shapes through every pipeline against the CPU oracle: the
shape, routing and mode of each case are drawn once from a fixed seed, so the
cases are the same on every run. They cover the decode, prefill-ring, fused
and generic kernel families in the combinations the fixed cases do not
(dims that are and are not multiples of 256 / 512, one to tens of experts,
k from 1 to E, every routing recipe, AUTO as well as forced modes)."""
import numpy as np
import pytest

import moe_inputs as mi
from tests import test_gpu_forward as bf
from tests import test_gpu_mx as mx

pytestmark = pytest.mark.gpu


def _draw(n, seed, mult, big_mult, mx_dtype):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        T = int(rng.choice([1, 2, 7, 33, 64, 129, 300, 513, 700, 1100, 2100]))
        m = big_mult if rng.random() < 0.5 else mult
        D = m * int(rng.integers(1, max(2, 1024 // m) + 1))
        H = mult * int(rng.integers(1, 1024 // mult + 1))
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64]))
        k = int(rng.integers(1, min(8, E) + 1))
        routing = str(rng.choice(["uniform", "softmax", "zipf"]))
        mode = str(rng.choice(["auto", "split", "fused"]))
        if T * k * D * H > 3e9:   # keeps the oracle's share of the test around a second a case
            continue
        cases.append((T, D, H, E, k, routing, mode))
    return cases


BF16_CASES = _draw(40, 20261202, 64, 256, False)
MX_CASES = _draw(20, 20261203, 128, 512, True)


@pytest.mark.parametrize("T,D,H,E,k,routing,mode", BF16_CASES)
def test_random_bf16(T, D, H, E, k, routing, mode):
    bf._case(mi.custom(T, D, H, E, k, routing), mode)


@pytest.mark.parametrize("T,D,H,E,k,routing,mode", MX_CASES)
def test_random_mxfp8(T, D, H, E, k, routing, mode):
    mx._case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"), mode=mode)


def _draw_extra(n, seed, mult):
    """(T, D, H, E, k, routing, extra) with extra drawn from [0, 1000) for the per-family choice."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        T = int(rng.choice([1, 5, 33, 64, 200, 513, 1100, 2100]))
        D = mult * int(rng.integers(1, 1024 // mult + 1))
        H = mult * int(rng.integers(1, 1024 // mult + 1))
        E = int(rng.choice([1, 2, 4, 8, 16, 32]))
        k = int(rng.integers(1, min(8, E) + 1))
        routing = str(rng.choice(["uniform", "softmax", "zipf"]))
        if T * k * D * H > 3e9:
            continue
        cases.append((T, D, H, E, k, routing, int(rng.integers(0, 1000))))
    return cases


@pytest.mark.parametrize("T,D,H,E,k,routing,extra", _draw_extra(12, 20261204, 64))
def test_random_shared_expert(T, D, H, E, k, routing, extra):
    from tests import test_gpu_shared as sh
    Hs = 64 * (1 + extra % 12)
    mode = ("auto", "split", "fused")[extra % 3]
    sh._case(mi.custom(T, D, H, E, k, routing), Hs, mode)


@pytest.mark.parametrize("T,D,H,E,k,routing,extra", _draw_extra(12, 20261205, 64))
def test_random_activation_variant(T, D, H, E, k, routing, extra):
    from tests import test_gpu_act as act
    act._case(mi.custom(T, D, H, E, k, routing), *act.VARIANTS[extra % len(act.VARIANTS)])


@pytest.mark.parametrize("T,D,H,E,k,routing,extra", _draw_extra(12, 20261206, 128))
def test_random_mxfp4(T, D, H, E, k, routing, extra):
    from tests import test_gpu_mx4 as mx4
    mx4._case(mi.custom(T, D, H, E, k, routing, dtype="mxfp8"))   # MX sources; the case quantizes W to e2m1
