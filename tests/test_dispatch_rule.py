"""Which GEMM kernels the library picks for a shape (moe_ffn_gemm_kernel, host
only, the launchers' own predicates), on the CPU. The decode-shaped kernels
are used while fewer than 0.5 experts are expected past 32 rows when each
token's k routes go to k distinct experts uniformly; that rule is checked
here against scipy's binomial tail."""
import pytest
from scipy.stats import binom

import grouped_gemm_amd as g


def _kernel(T, D, H, E, k, dtype="bf16", mode="split", gemm=1):
    return g.moe_ffn_gemm_kernel(T, D, H, E, k, dtype, mode, gemm)


@pytest.mark.parametrize("T,k,E", [(64, 8, 32), (80, 8, 32), (96, 8, 32), (128, 8, 32), (192, 6, 64),
                                   (256, 6, 64), (384, 8, 128), (256, 8, 128), (37, 3, 5), (1, 2, 4),
                                   (5000, 1, 1024), (40, 8, 8), (33, 8, 8)])
def test_decode_rule_matches_binomial_tail(T, k, E):
    p = k / E
    want = T * p <= 32 and E * binom.sf(32, T, p) < 0.5
    got = _kernel(T, 2048, 1024, E, k) == "dma_kmajor_kernel"
    assert got == want
    mx = _kernel(T, 2048, 1024, E, k, dtype="mxfp8") == "mx_kmajor_kernel"
    assert mx == want


def test_workload_paths():
    assert _kernel(64, 6144, 2048, 32, 8) == "dma_kmajor_kernel"             # decode: 8 row groups per block
    assert _kernel(64, 6144, 2048, 32, 8, gemm=2) == "dma_kmajor_kernel"     # 12 row groups per block
    assert _kernel(64, 384, 2048, 32, 8) == "dma_skinny_kernel"             # K not a multiple of 256
    assert _kernel(4096, 2048, 768, 128, 8) == "big_gemm_kernel<256>"       # mid prefill: 256 rows/expert
    assert _kernel(1024, 2048, 768, 128, 8) == "big_gemm_kernel<128>"       # 64 rows/expert
    assert _kernel(131072, 2048, 768, 128, 8, gemm=2) == "big_gemm_kernel<256>"
    assert _kernel(300, 384, 640, 16, 4) == "gemm1_swiglu_kernel"           # D not a multiple of 256
    assert _kernel(300, 384, 640, 16, 4, gemm=2) == "gemm2_weight_kernel"
    assert _kernel(64, 256, 512, 8, 2, mode="auto") == "fused_dma_kernel"   # AUTO: fused (launch-bound)
    assert _kernel(1024, 256, 512, 8, 2, mode="auto") == "big_gemm_kernel<256>"  # AUTO: split
    assert _kernel(64, 256, 512, 8, 2, mode="fused") == "fused_dma_kernel"
    assert _kernel(64, 384, 512, 8, 2, mode="fused") == "fused_bf16_kernel"  # D not a multiple of 256
    assert _kernel(16384, 4096, 1536, 64, 6, dtype="mxfp8") == "big_gemm_kernel<256>"
    assert _kernel(2048, 4096, 1536, 64, 6, dtype="mxfp8") == "big_gemm_kernel<256>"   # 192 rows/expert
    assert _kernel(1024, 4096, 1536, 64, 6, dtype="mxfp8") == "mx_gemm1_kernel"        # 96 rows/expert
    assert _kernel(64, 4096, 1536, 64, 6, dtype="mxfp8") == "mx_kmajor_kernel"     # 12 row groups per block
    assert _kernel(64, 6144, 2048, 32, 8, dtype="mxfp4", gemm=2) == "mx_kmajor_kernel"
    assert _kernel(64, 512, 512, 32, 8, dtype="mxfp8") == "mx_kmajor_kernel"      # 16 and 8 row groups
    assert _kernel(64, 256, 512, 8, 2, dtype="mxfp8", mode="fused") == "mx_fused_kernel"
    # E = 1 (one group of every token): the decode kernels while the prefill
    # ring would get fewer tiles than half of the 256 compute units
    assert _kernel(260, 256, 128, 1, 1) == "dma_kmajor_kernel"             # 3 ring tiles
    assert _kernel(260, 256, 128, 1, 1, gemm=2) == "dma_skinny_kernel"     # K = H = 128
    assert _kernel(2048, 256, 512, 1, 1) == "dma_kmajor_kernel"            # (16 + 1) x 4 = 68 ring tiles
    assert _kernel(2048, 256, 512, 1, 1, gemm=2) == "dma_kmajor_kernel"    # 4 row groups over 64 m-tiles
    assert _kernel(4096, 256, 1024, 1, 1) == "big_gemm_kernel<256>"        # (32 + 1) x 8 = 264 ring tiles
    assert _kernel(0, 256, 512, 8, 2) == "none"
    assert _kernel(64, 256, 512, 8, 2, gemm=3) is None
    assert _kernel(64, 250, 512, 8, 2) is None                              # invalid shape
    assert _kernel(64, 256, 512, 8, 2, dtype="mxfp4", mode="fused") is None  # unsupported
