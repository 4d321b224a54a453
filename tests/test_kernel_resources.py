"""Resource checks of the DMA-ring kernels, on the CPU (hipcc cross-compiles).

The prefill and decode GEMMs keep their LDS DMA in flight across many
steps; the compiler does not see those DMAs (they are issued from inline
assembly), so any memory access it adds itself inside the loop, such as a
scratch load of a spilled register or of a dynamically indexed private
array, comes with a wait for every memory operation in flight and drains
the ring. These kernels must use no scratch memory at all."""
import os
import re
import shutil
import subprocess

import pytest

from grouped_gemm_amd import build as b

HIPCC = b.HIPCC
RING_KERNELS = {"gemm_big.hip": ("big_gemm_kernel",),
                "gemm_skinny.hip": ("dma_skinny_kernel", "dma_kmajor_kernel", "mx_kmajor_kernel"),
                "gemm_fused.hip": ("fused_dma_kernel",)}
LDS_BYTES = 160 * 1024


def _kernel_metadata(src: str, tmp_path) -> list[dict]:
    out = os.path.join(tmp_path, os.path.basename(src) + ".s")
    cmd = [HIPCC, *b.FLAGS, "-S", "--cuda-device-only", "-o", out, os.path.join(b.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = open(out).read()
    kernels = []
    for block in re.split(r"\n\s+- \.agpr_count", text)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        field = lambda k: int(re.search(rf"\.{k}:\s+(\d+)", block).group(1))
        kernels.append({"name": name.group(1), "private": field("private_segment_fixed_size"),
                        "lds": field("group_segment_fixed_size"), "vspill": field("vgpr_spill_count"),
                        "vgpr": field("vgpr_count")})
    return kernels, text


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", sorted(RING_KERNELS))
def test_ring_kernels_use_no_scratch(src, tmp_path):
    kernels, text = _kernel_metadata(src, str(tmp_path))
    for want in RING_KERNELS[src]:
        assert any(want in k["name"] for k in kernels), f"no {want} instances found in {src}"
    ring = [k for k in kernels if any(want in k["name"] for want in RING_KERNELS[src])]
    for k in ring:
        assert k["private"] == 0, f"{k['name']} uses {k['private']} bytes of scratch"
        assert k["vspill"] == 0, f"{k['name']} spills {k['vspill']} VGPRs"
        assert k["lds"] <= LDS_BYTES, f"{k['name']} needs {k['lds']} bytes of LDS"
    assert "scratch_load" not in text and "scratch_store" not in text
