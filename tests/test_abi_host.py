"""The C-ABI library loads without a GPU, exports every function the header
declares, and its host-only entry points validate shapes (no GPU call)."""
import ctypes

import pytest

import grouped_gemm_amd as g


def test_library_exports_every_header_function():
    lib = g.library()
    names = g.header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == {
        "moe_ffn_workspace_bytes", "moe_ffn_validate", "moe_ffn_resolve_mode", "moe_ffn_gemm_kernel", "moe_ffn_forward",
        "moe_ffn_forward_events", "moe_ffn_forward_noalloc", "moe_ffn_router", "moe_ffn_forward_logits",
        "moe_ffn_shared_workspace_bytes", "moe_ffn_forward_shared", "moe_ffn_forward_act",
        "moe_ffn_route_workspace_bytes", "moe_ffn_route", "moe_ffn_mx_quantize", "moe_ffn_mxfp4_quantize",
        "moe_ffn_strerror"}


@pytest.mark.parametrize("shape,expect", [
    ((64, 256, 512, 8, 2), g.MOE_FFN_OK),
    ((0, 256, 512, 8, 2), g.MOE_FFN_OK),
    ((-1, 256, 512, 8, 2), g.MOE_FFN_EINVAL_SHAPE),
    ((64, 200, 512, 8, 2), g.MOE_FFN_EINVAL_SHAPE),     # D not a multiple of 64
    ((64, 256, 500, 8, 2), g.MOE_FFN_EINVAL_SHAPE),     # H not a multiple of 64
    ((64, 192, 320, 8, 2), g.MOE_FFN_OK),               # bf16: multiples of 64
    ((64, 64, 64, 8, 2), g.MOE_FFN_OK),
    ((64, 256, 512, 8, 9), g.MOE_FFN_EINVAL_SHAPE),     # k > E
    ((64, 256, 512, 0, 1), g.MOE_FFN_EINVAL_SHAPE),
    ((64, 256, 512, 8, 0), g.MOE_FFN_EINVAL_SHAPE),
    ((64, 256, 512, 9000, 2), g.MOE_FFN_EINVAL_SHAPE),  # E above the route limit
    ((1 << 30, 256, 512, 8, 4), g.MOE_FFN_EINVAL_SHAPE),  # T*k overflows int32
])
def test_validate_shapes(shape, expect):
    assert g.moe_ffn_validate(*shape) == expect


def test_validate_dtype_and_mode():
    assert g.moe_ffn_validate(64, 256, 512, 8, 2, dtype=7) == g.MOE_FFN_EUNSUPPORTED
    # MXFP4 weights: split (AUTO resolves to it), no fused pipeline; workspace as for MX-fp8
    assert g.moe_ffn_validate(64, 256, 512, 8, 2, dtype="mxfp4", mode="split") == g.MOE_FFN_OK
    assert g.moe_ffn_validate(64, 256, 512, 8, 2, dtype="mxfp4", mode="fused") == g.MOE_FFN_EUNSUPPORTED
    assert g.moe_ffn_resolve_mode(64, 256, 512, 8, 2, dtype="mxfp4") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_workspace_bytes(64, 256, 512, 8, 2, "mxfp4", "split") == \
        g.moe_ffn_workspace_bytes(64, 256, 512, 8, 2, "mxfp8", "split")
    assert g.moe_ffn_validate(64, 256, 512, 8, 2, mode=5) == g.MOE_FFN_EUNSUPPORTED
    assert g.moe_ffn_validate(64, 256, 512, 8, 2, dtype="mxfp8", mode="fused") == g.MOE_FFN_OK
    assert g.moe_ffn_resolve_mode(64, 256, 512, 8, 2, dtype="mxfp8", mode="auto") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_validate(64, 256, 512, 8, 2, dtype="mxfp8", mode="split") == g.MOE_FFN_OK
    lib = g.library()
    assert lib.moe_ffn_validate(None, 0) == g.MOE_FFN_EINVAL_PTR


def test_resolve_mode():
    assert g.moe_ffn_resolve_mode(64, 256, 512, 8, 2, mode="split") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_resolve_mode(64, 256, 512, 8, 2, mode="fused") == g.MOE_FFN_FUSED
    # measured crossover: fused where the pass is launch-bound (up to 16 MB of expert
    # weights streamed, one expert's weights per 32 rows), split everywhere else
    assert g.moe_ffn_resolve_mode(64, 256, 512, 8, 2, mode="auto") == g.MOE_FFN_FUSED
    assert g.moe_ffn_resolve_mode(16, 256, 512, 8, 2, mode="auto") == g.MOE_FFN_FUSED
    assert g.moe_ffn_resolve_mode(1, 256, 512, 8, 2, mode="auto") == g.MOE_FFN_FUSED
    assert g.moe_ffn_resolve_mode(256, 256, 512, 8, 2, mode="auto") == g.MOE_FFN_FUSED   # 64 rows per expert
    assert g.moe_ffn_resolve_mode(1024, 256, 512, 8, 2, mode="auto") == g.MOE_FFN_SPLIT  # 50 MB streamed
    assert g.moe_ffn_resolve_mode(64, 384, 512, 8, 2, mode="auto") == g.MOE_FFN_SPLIT    # not the fused ring's shapes
    assert g.moe_ffn_resolve_mode(64, 256, 2048, 8, 2, mode="auto") == g.MOE_FFN_SPLIT   # 25 MB of weights
    assert g.moe_ffn_resolve_mode(64, 6144, 2048, 32, 8, mode="auto") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_resolve_mode(16, 2048, 768, 128, 8, mode="auto") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_resolve_mode(131072, 2048, 768, 128, 8, mode="auto") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_resolve_mode(64, 256, 512, 8, 2, dtype="mxfp8") == g.MOE_FFN_SPLIT   # not the MX ring's shapes
    # MX-fp8: fused while its (m-tile, 128-wide slice) blocks fit one round of the 256 CUs
    # (expected m-tiles x H/128: 72, 250 and 419 blocks at 1, 4 and 8 tokens)
    assert g.moe_ffn_resolve_mode(1, 4096, 1536, 64, 6, dtype="mxfp8") == g.MOE_FFN_FUSED
    assert g.moe_ffn_resolve_mode(4, 4096, 1536, 64, 6, dtype="mxfp8") == g.MOE_FFN_FUSED
    assert g.moe_ffn_resolve_mode(8, 4096, 1536, 64, 6, dtype="mxfp8") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_resolve_mode(16384, 4096, 1536, 64, 6, dtype="mxfp8") == g.MOE_FFN_SPLIT
    assert g.moe_ffn_resolve_mode(4, 4096, 1536, 64, 6, dtype="mxfp4") == g.MOE_FFN_SPLIT


def test_workspace_sizes():
    T, D, H, E, k = 4096, 2048, 768, 128, 8
    P = T * k
    split = g.moe_ffn_workspace_bytes(T, D, H, E, k, mode="split")
    fused = g.moe_ffn_workspace_bytes(T, D, H, E, k, mode="fused")
    assert split >= P * H * 2 + P * D * 2 + 2 * P * 4          # act + ypair + maps
    assert fused >= T * D * 4 + 2 * P * 4                      # fp32 accumulator + maps
    mx = g.moe_ffn_workspace_bytes(T, D, H, E, k, dtype="mxfp8", mode="split")
    assert mx >= P * H + P * H // 32 + P * D * 2
    assert split % 256 == 0 and fused % 256 == 0
    assert g.moe_ffn_workspace_bytes(64, 200, 512, 8, 2) == 0   # invalid -> 0
    assert g.library().moe_ffn_route_workspace_bytes(100, 8, 32) > 0
    assert g.library().moe_ffn_route_workspace_bytes(100, 8, 0) == 0


def test_forward_rejects_bad_arguments_without_gpu_work():
    """Errors found on the host return before any launch."""
    lib = g.library()
    p = g.make_problem(64, 256, 512, 8, 2)
    VP = ctypes.c_void_p
    # null pointers
    assert lib.moe_ffn_forward(ctypes.byref(p), None, None, None, None, None, None, 2, None) == \
        g.MOE_FFN_EINVAL_PTR
    # misaligned pointer
    bad = VP(0x1001)
    ok = VP(0x1000)
    assert lib.moe_ffn_forward(ctypes.byref(p), bad, ok, ok, ok, ok, ok, 2, None) == g.MOE_FFN_EINVAL_PTR
    # missing workspace
    assert lib.moe_ffn_forward(ctypes.byref(p), ok, ok, ok, ok, ok, ok, 2, None) == g.MOE_FFN_EWORKSPACE
    # MX path without scales
    pm = g.make_problem(64, 256, 512, 8, 2, dtype="mxfp8")
    assert lib.moe_ffn_forward(ctypes.byref(pm), ok, ok, ok, ok, ok, ok, 2, None) == g.MOE_FFN_EINVAL_PTR
    # T = 0 is a no-op that touches nothing
    p0 = g.make_problem(0, 256, 512, 8, 2)
    assert lib.moe_ffn_forward(ctypes.byref(p0), None, None, None, None, None, None, 2, None) == g.MOE_FFN_OK
    assert lib.moe_ffn_mx_quantize(None, 4, 48, None, None, None) == g.MOE_FFN_EINVAL_SHAPE
    assert lib.moe_ffn_mx_quantize(None, 4, 64, None, None, None) == g.MOE_FFN_EINVAL_PTR
    assert lib.moe_ffn_mxfp4_quantize(None, 4, 48, None, None, None) == g.MOE_FFN_EINVAL_SHAPE
    assert lib.moe_ffn_mxfp4_quantize(None, 4, 64, None, None, None) == g.MOE_FFN_EINVAL_PTR
    assert lib.moe_ffn_mxfp4_quantize(None, 0, 64, None, None, None) == g.MOE_FFN_OK
    # MXFP4 path without scales, and in the fused pipeline
    p4 = g.make_problem(64, 256, 512, 8, 2, dtype="mxfp4")
    assert lib.moe_ffn_forward(ctypes.byref(p4), ok, ok, ok, ok, ok, ok, 2, None) == g.MOE_FFN_EINVAL_PTR
    assert lib.moe_ffn_forward(ctypes.byref(p4), ok, ok, ok, ok, ok, ok, 1, None) == g.MOE_FFN_EUNSUPPORTED


def test_strerror():
    for c in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(g.moe_ffn_strerror(c), str) and g.moe_ffn_strerror(c)


def test_forward_events_argument_checks():
    lib = g.library()
    p = g.make_problem(64, 256, 512, 8, 2)
    ok = ctypes.c_void_p(0x1000)
    assert lib.moe_ffn_forward_events(ctypes.byref(p), ok, ok, ok, ok, ok, ok, 2, None, None, 3) == \
        g.MOE_FFN_EINVAL_PTR
    assert lib.moe_ffn_forward_events(ctypes.byref(p), ok, ok, ok, ok, ok, ok, 2, None, None, 5) == \
        g.MOE_FFN_EINVAL_PTR


@pytest.mark.parametrize("T,E,k,expect", [
    (0, 8, 2, g.MOE_FFN_OK),                 # empty: a no-op before any pointer check
    (-1, 8, 2, g.MOE_FFN_EINVAL_SHAPE),
    (4, 0, 1, g.MOE_FFN_EINVAL_SHAPE),
    (4, 8, 0, g.MOE_FFN_EINVAL_SHAPE),
    (4, 8, 9, g.MOE_FFN_EINVAL_SHAPE),       # k > E
    (4, 100, 65, g.MOE_FFN_EINVAL_SHAPE),    # k > 64
    (4, 9000, 2, g.MOE_FFN_EINVAL_SHAPE),    # E > 8192
    (4, 8, 2, g.MOE_FFN_EINVAL_PTR),         # null buffers
])
def test_router_argument_checks(T, E, k, expect):
    """Host-side checks of moe_ffn_router: they return before any GPU call."""
    assert g.library().moe_ffn_router(None, T, E, k, None, None, None) == expect


def test_forward_logits_argument_checks():
    lib = g.library()
    p = g.make_problem(4, 256, 512, 8, 2)
    # null logits with tokens to route
    assert lib.moe_ffn_forward_logits(ctypes.byref(p), None, None, None, None, None, None, None, 0, None,
                                      None, 0) == g.MOE_FFN_EINVAL_PTR
    bad = g.make_problem(4, 200, 512, 8, 2)  # D not a multiple of 128
    fake = ctypes.c_void_p(256)
    assert lib.moe_ffn_forward_logits(ctypes.byref(bad), None, None, None, fake, None, None, None, 0, None,
                                      None, 0) == g.MOE_FFN_EINVAL_SHAPE
    empty = g.make_problem(0, 256, 512, 8, 2)
    assert lib.moe_ffn_forward_logits(ctypes.byref(empty), None, None, None, None, None, None, None, 0, None,
                                      None, 0) == g.MOE_FFN_OK


def test_shared_expert_host_checks():
    lib = g.library()
    p = g.make_problem(64, 256, 512, 8, 2)
    base = lib.moe_ffn_workspace_bytes(ctypes.byref(p), g.MOE_FFN_SPLIT)
    with_shared = lib.moe_ffn_shared_workspace_bytes(ctypes.byref(p), 384, g.MOE_FFN_SPLIT)
    assert with_shared > base > 0
    assert lib.moe_ffn_shared_workspace_bytes(ctypes.byref(p), 100, g.MOE_FFN_SPLIT) == 0   # Hs % 128
    mx = g.make_problem(64, 256, 512, 8, 2, "mxfp8")
    assert lib.moe_ffn_shared_workspace_bytes(ctypes.byref(mx), 256, g.MOE_FFN_SPLIT) == 0
    assert lib.moe_ffn_forward_shared(ctypes.byref(mx), None, None, None, None, None, None, None, 256, None, 0,
                                      None, None, 0) == g.MOE_FFN_EUNSUPPORTED
    assert lib.moe_ffn_forward_shared(ctypes.byref(p), None, None, None, None, None, None, None, 200, None, 0,
                                      None, None, 0) == g.MOE_FFN_EINVAL_SHAPE


@pytest.mark.parametrize("kind,limit,mode,dtype,expect", [
    (1, 0.0, "split", "bf16", g.MOE_FFN_EINVAL_SHAPE),       # the clamp needs a positive limit
    (1, float("inf"), "split", "bf16", g.MOE_FFN_EINVAL_SHAPE),
    (2, 1.0, "split", "bf16", g.MOE_FFN_EUNSUPPORTED),        # unknown kind
    (1, 7.0, "fused", "bf16", g.MOE_FFN_EUNSUPPORTED),        # the variant runs on the split pipeline
    (1, 7.0, "split", "mxfp8", g.MOE_FFN_EUNSUPPORTED),
    (1, 7.0, "split", "bf16", g.MOE_FFN_EINVAL_PTR),          # valid: null tensors are rejected next
])
def test_activation_variant_host_checks(kind, limit, mode, dtype, expect):
    lib = g.library()
    p = g.make_problem(4, 256, 512, 8, 2, dtype)
    act = g.moe_ffn_activation(kind, limit, None, 0)
    assert lib.moe_ffn_forward_act(ctypes.byref(p), None, None, None, None, None, ctypes.byref(act), None,
                                   g._mode(mode), None, None, 0) == expect
    assert lib.moe_ffn_forward_act(ctypes.byref(p), None, None, None, None, None, None, None, 0, None, None,
                                   0) == g.MOE_FFN_EINVAL_PTR


# ---- the binding's own shape and dtype checks (CPU tensors: nothing is launched) ----

def _cpu_pass(T=8, D=128, H=128, E=4, k=2):
    import torch
    return dict(x=torch.zeros((T, D), dtype=torch.bfloat16), w1=torch.zeros((E, 2 * H, D), dtype=torch.bfloat16),
                w2=torch.zeros((E, D, H), dtype=torch.bfloat16), topk_ids=torch.zeros((T, k), dtype=torch.int32),
                topk_weights=torch.zeros((T, k), dtype=torch.float32))


@pytest.mark.parametrize("name,shape,dtype", [
    ("out", (7, 128), "bfloat16"),             # one row short
    ("out", (8, 128), "float32"),
    ("topk_weights", (8, 1), "float32"),       # narrower than topk_ids
    ("topk_weights", (8, 2), "float64"),
    ("w2", (4, 128, 64), "bfloat16"),          # H of w1 is 128
    ("w1", (4, 256, 64), "bfloat16"),          # D of x is 128
    ("x", (8, 128), "float16"),
])
def test_binding_rejects_mismatched_tensors(name, shape, dtype):
    import torch
    import grouped_gemm_amd as g
    t = _cpu_pass()
    bad = torch.zeros(shape, dtype=getattr(torch, dtype))
    kw = {} if name == "out" else {}
    if name == "out":
        kw["out"] = bad
    else:
        t[name] = bad
    with pytest.raises(ValueError, match=name if name != "x" else "x|w1"):
        g.moe_ffn_forward(t["x"], t["w1"], t["w2"], t["topk_ids"], t["topk_weights"], **kw)


def test_binding_rejects_mx_scale_shapes():
    import torch
    import grouped_gemm_amd as g
    T, D, H, E, k = 8, 128, 128, 4, 2
    u8 = torch.uint8
    x, w1, w2 = torch.zeros((T, D), dtype=u8), torch.zeros((E, 2 * H, D), dtype=u8), torch.zeros((E, D, H), dtype=u8)
    ids, w = torch.zeros((T, k), dtype=torch.int32), torch.zeros((T, k))
    good = dict(x_scale=torch.zeros((T, D // 32), dtype=u8), w1_scale=torch.zeros((E, 2 * H, D // 32), dtype=u8),
                w2_scale=torch.zeros((E, D, H // 32), dtype=u8))
    for name in good:
        kw = dict(good)
        kw[name] = torch.zeros((1, 1), dtype=u8)
        with pytest.raises(ValueError, match=name):
            g.moe_ffn_forward(x, w1, w2, ids, w, **kw)
        kw[name] = None
        with pytest.raises(ValueError, match=name):
            g.moe_ffn_forward(x, w1, w2, ids, w, **kw)
    # matching shapes reach the device check (CPU tensors), not a launch
    with pytest.raises(ValueError, match="GPU"):
        g.moe_ffn_forward(x, w1, w2, ids, w, **good)


def test_noalloc_limit_and_error_code():
    # a problem beyond the static scratch array is refused by its size alone,
    # before any pointer is looked at (so NULL pointers are fine here)
    p = g.make_problem(4096, 2048, 768, 128, 8, "bf16")
    assert g.moe_ffn_workspace_bytes(4096, 2048, 768, 128, 8, "bf16", "split") > g.MOE_FFN_NOALLOC_SCRATCH_BYTES
    rc = g.library().moe_ffn_forward_noalloc(ctypes.byref(p), None, None, None, None, None, None,
                                            g.MOE_FFN_SPLIT, None)
    assert rc == g.MOE_FFN_ESCRATCH
    assert "scratch" in g.moe_ffn_strerror(g.MOE_FFN_ESCRATCH)
    # the decode workload fits
    assert g.moe_ffn_workspace_bytes(64, 6144, 2048, 32, 8, "bf16", "split") < g.MOE_FFN_NOALLOC_SCRATCH_BYTES


def test_mx_shapes_are_multiples_of_128():
    # the MX kernels stage K in 128-code steps: bf16 takes multiples of 64, MX of 128
    for dt in ("mxfp8", "mxfp4"):
        assert g.moe_ffn_validate(64, 192, 256, 8, 2, dtype=dt, mode="split") == g.MOE_FFN_EINVAL_SHAPE
        assert g.moe_ffn_validate(64, 256, 320, 8, 2, dtype=dt, mode="split") == g.MOE_FFN_EINVAL_SHAPE
        assert g.moe_ffn_validate(64, 384, 640, 8, 2, dtype=dt, mode="split") == g.MOE_FFN_OK


def test_64_multiples_take_the_generic_kernels():
    # D or H a multiple of 64 but not 128: neither the decode nor the prefill ring kernels
    assert g.moe_ffn_gemm_kernel(64, 192, 320, 8, 2, "bf16", "split", 1) == "gemm1_swiglu_kernel"
    assert g.moe_ffn_gemm_kernel(64, 192, 320, 8, 2, "bf16", "split", 2) == "gemm2_weight_kernel"
    assert g.moe_ffn_gemm_kernel(64, 192, 320, 8, 2, "bf16", "fused", 1) == "fused_bf16_kernel"
    assert g.moe_ffn_gemm_kernel(4096, 320, 192, 8, 2, "bf16", "split", 1) == "gemm1_swiglu_kernel"
    assert g.moe_ffn_workspace_bytes(64, 192, 320, 8, 2, "bf16", "split") > 0
