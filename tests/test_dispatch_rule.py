"""The decode-kernel rule that bench.py mirrors from the library's dispatch
(fewer than 0.5 experts expected past 32 rows when each token's k routes go
to k distinct experts uniformly), checked against scipy's binomial tail."""
import pytest
from scipy.stats import binom

import bench


@pytest.mark.parametrize("T,k,E", [(64, 8, 32), (80, 8, 32), (96, 8, 32), (128, 8, 32), (192, 6, 64),
                                   (256, 6, 64), (384, 8, 128), (256, 8, 128), (37, 3, 5), (1, 2, 4),
                                   (5000, 1, 1024), (40, 8, 8), (33, 8, 8)])
def test_decode_rule_matches_binomial_tail(T, k, E):
    p = k / E
    want = T * p <= 32 and E * binom.sf(32, T, p) < 0.5
    assert bench.decode_kernels_fit(T, k, E) == want
