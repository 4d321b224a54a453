"""MI355X (gfx950) routed MoE SwiGLU FFN forward pass: Python binding.

A thin ctypes layer over ``libmoe_ffn.so`` whose functions carry the C ABI's
names (include/moe_ffn.h). It only marshals arguments: torch tensors are
passed as device pointers together with torch's current HIP stream; every
step of the pass runs in the library's HIP kernels. There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

    out = moe_ffn_forward(x, w1, w2, topk_ids, topk_weights, mode="split")
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ffn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe_ffn.h")

MOE_FFN_BF16, MOE_FFN_MXFP8, MOE_FFN_MXFP4 = 0, 1, 2
MOE_FFN_AUTO, MOE_FFN_FUSED, MOE_FFN_SPLIT = 0, 1, 2
MOE_FFN_OK = 0
MOE_FFN_EINVAL_SHAPE, MOE_FFN_EINVAL_PTR, MOE_FFN_EUNSUPPORTED = -1, -2, -3
MOE_FFN_EWORKSPACE, MOE_FFN_EHIP, MOE_FFN_ESCRATCH = -4, -5, -6
MOE_FFN_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_FFN_ACT_SWIGLU, MOE_FFN_ACT_CLAMPED_SWIGLU = 0, 1

_MODES = {"auto": MOE_FFN_AUTO, "fused": MOE_FFN_FUSED, "split": MOE_FFN_SPLIT}
_DTYPES = {"bf16": MOE_FFN_BF16, "mxfp8": MOE_FFN_MXFP8, "mxfp4": MOE_FFN_MXFP4}


class MoeFfnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {moe_ffn_strerror(code)} ({code})")


class moe_ffn_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("x_scale", ctypes.c_void_p), ("w1_scale", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]



class moe_ffn_activation(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("limit", ctypes.c_float), ("alpha", ctypes.c_void_p),
                ("weight_before_act", ctypes.c_int32)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libmoe_ffn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m grouped_gemm_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        VP, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        PP = ctypes.POINTER(moe_ffn_problem)
        EV = ctypes.POINTER(ctypes.c_void_p)
        INT, SZ = ctypes.c_int, ctypes.c_size_t
        signatures = {
            "moe_ffn_workspace_bytes": ([PP, INT], SZ),
            "moe_ffn_validate": ([PP, INT], INT),
            "moe_ffn_resolve_mode": ([PP, INT], INT),
            "moe_ffn_gemm_kernel": ([PP, INT, INT], ctypes.c_char_p),
            "moe_ffn_forward": ([PP, VP, VP, VP, VP, VP, VP, INT, VP], INT),
            "moe_ffn_forward_events": ([PP, VP, VP, VP, VP, VP, VP, INT, VP, EV, INT], INT),
            "moe_ffn_forward_noalloc": ([PP, VP, VP, VP, VP, VP, VP, INT, VP], INT),
            "moe_ffn_router": ([VP, I32, I32, I32, VP, VP, VP], INT),
            "moe_ffn_forward_logits": ([PP, VP, VP, VP, VP, VP, VP, VP, INT, VP, EV, INT], INT),
            "moe_ffn_shared_workspace_bytes": ([PP, I32, INT], SZ),
            "moe_ffn_forward_shared": ([PP, VP, VP, VP, VP, VP, VP, VP, I32, VP, INT, VP, EV, INT], INT),
            "moe_ffn_forward_act": ([PP, VP, VP, VP, VP, VP, ctypes.POINTER(moe_ffn_activation), VP, INT, VP, EV,
                                     INT], INT),
            "moe_ffn_route_workspace_bytes": ([I32, I32, I32], SZ),
            "moe_ffn_route": ([VP, I32, I32, I32, VP, VP, VP, VP, VP, SZ, VP], INT),
            "moe_ffn_mx_quantize": ([VP, I64, I32, VP, VP, VP], INT),
            "moe_ffn_mxfp4_quantize": ([VP, I64, I32, VP, VP, VP], INT),
            "moe_ffn_strerror": ([INT], ctypes.c_char_p),
        }
        for name, (args, res) in signatures.items():
            fn = getattr(lib, name)
            fn.argtypes, fn.restype = args, res
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/moe_ffn.h declares."""
    text = open(HEADER_PATH).read()
    return re.findall(r"MOE_FFN_API\s+[\w\s\*]+?\b(moe_ffn_\w+)\s*\(", text)


def moe_ffn_strerror(code: int) -> str:
    return library().moe_ffn_strerror(int(code)).decode()


def _mode(mode) -> int:
    return _MODES[mode] if isinstance(mode, str) else int(mode)


def _dtype(dtype) -> int:
    return _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _data_path(x, w1) -> str:
    """bf16 tensors: "bf16"; uint8 codes: "mxfp4" when w1 rows hold D/2 bytes (packed e2m1), else "mxfp8"."""
    if x.dtype != torch.uint8:
        return "bf16"
    return "mxfp4" if w1.shape[-1] * 2 == x.shape[1] else "mxfp8"


def make_problem(T, D, H, E, topk, dtype="bf16", x_scale=None, w1_scale=None, w2_scale=None,
                 workspace=None) -> moe_ffn_problem:
    p = moe_ffn_problem(int(T), int(D), int(H), int(E), int(topk), _dtype(dtype))
    for name, t in (("x_scale", x_scale), ("w1_scale", w1_scale), ("w2_scale", w2_scale)):
        setattr(p, name, t.data_ptr() if t is not None else None)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    return p


def moe_ffn_workspace_bytes(T, D, H, E, topk, dtype="bf16", mode="auto") -> int:
    p = make_problem(T, D, H, E, topk, dtype)
    return int(library().moe_ffn_workspace_bytes(ctypes.byref(p), _mode(mode)))


def moe_ffn_validate(T, D, H, E, topk, dtype="bf16", mode="auto") -> int:
    p = make_problem(T, D, H, E, topk, dtype)
    return int(library().moe_ffn_validate(ctypes.byref(p), _mode(mode)))


def moe_ffn_resolve_mode(T, D, H, E, topk, dtype="bf16", mode="auto") -> int:
    p = make_problem(T, D, H, E, topk, dtype)
    return int(library().moe_ffn_resolve_mode(ctypes.byref(p), _mode(mode)))


def moe_ffn_gemm_kernel(T, D, H, E, topk, dtype="bf16", mode="auto", gemm=1):
    """Name of the kernel family the forward pass runs for GEMM1 or GEMM2 on
    this shape (host only), or None for an invalid problem."""
    p = make_problem(T, D, H, E, topk, dtype)
    name = library().moe_ffn_gemm_kernel(ctypes.byref(p), _mode(mode), int(gemm))
    return name.decode() if name is not None else None


@contextlib.contextmanager
def _on(stream):
    """Make `stream` current for the wrapper's own allocations and its int64 ->
    int32 id conversion, after the work already queued on the caller's
    current stream. torch's caching allocator hands a freed block out again
    only on the stream it was allocated on, so the temporaries (workspace,
    converted ids) cannot be reused while the pass still reads them."""
    cur = torch.cuda.current_stream()
    if stream is None or stream == cur:
        yield cur
        return
    stream.wait_stream(cur)
    with torch.cuda.stream(stream):
        yield stream


def _sp(stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(stream.cuda_stream)


def _check_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")


def _expect(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")


def _pass_shapes(x, w1, w2, topk_ids, topk_weights, out, x_scale=None, w1_scale=None, w2_scale=None):
    """(T, D, H, E, k, data path) of a pass, after checking every tensor's
    shape and dtype against them: the C ABI sees only pointers, so this is
    where a short `out` or a narrow `topk_weights` is caught."""
    if x.dim() != 2 or w1.dim() != 3 or w2.dim() != 3 or topk_ids.dim() != 2:
        raise ValueError("x must be [T, D], w1 [E, 2H, D(/2)], w2 [E, D, H(/2)], topk_ids [T, k]")
    T, D = x.shape
    E, H2 = w1.shape[0], w1.shape[1]
    H = H2 // 2
    k = topk_ids.shape[1]
    path = _data_path(x, w1)
    if topk_ids.shape[0] != T or topk_ids.dtype not in (torch.int32, torch.int64):
        raise ValueError("topk_ids must be int32 (or int64) [T, k]")
    _expect(topk_weights, (T, k), torch.float32, "topk_weights")
    if out is not None:
        _expect(out, (T, D), torch.bfloat16, "out")
    if H2 % 2:
        raise ValueError("w1 must hold 2H rows per expert")
    if path == "bf16":
        _expect(x, (T, D), torch.bfloat16, "x")
        _expect(w1, (E, H2, D), torch.bfloat16, "w1")
        _expect(w2, (E, D, H), torch.bfloat16, "w2")
        if any(t is not None for t in (x_scale, w1_scale, w2_scale)):
            raise ValueError("the bf16 path takes no scales")
    else:
        wk = 2 if path == "mxfp4" else 1
        if D % 32 or H % 32:
            raise ValueError("MX paths need D and H multiples of 32")
        _expect(w1, (E, H2, D // wk), torch.uint8, "w1")
        _expect(w2, (E, D, H // wk), torch.uint8, "w2")
        _expect(x_scale, (T, D // 32), torch.uint8, "x_scale")
        _expect(w1_scale, (E, H2, D // 32), torch.uint8, "w1_scale")
        _expect(w2_scale, (E, D, H // 32), torch.uint8, "w2_scale")
    return T, D, H, E, k, path


def _ids32(topk_ids):
    return topk_ids if topk_ids.dtype == torch.int32 else topk_ids.to(torch.int32)


def _workspace(lib, p, m, dev, what, nbytes=None):
    if nbytes is None:
        nbytes = lib.moe_ffn_workspace_bytes(ctypes.byref(p), m)
    if nbytes == 0:
        raise MoeFfnError(lib.moe_ffn_validate(ctypes.byref(p), m) or MOE_FFN_EINVAL_SHAPE, what)
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _events(events):
    return (None, 0) if events is None else ((ctypes.c_void_p * 5)(*events), 5)


def moe_ffn_forward(x, w1, w2, topk_ids, topk_weights, out=None, mode="auto", x_scale=None,
                    w1_scale=None, w2_scale=None, workspace=None, stream=None, events=None):
    """out [T, D] bf16 = the routed MoE SwiGLU FFN forward pass.

    bf16 path: x [T, D], w1 [E, 2H, D], w2 [E, D, H] torch.bfloat16.
    MXFP8 path: x, w1, w2 are uint8 e4m3 codes and x_scale [T, D/32],
    w1_scale [E, 2H, D/32], w2_scale [E, D, H/32] uint8 e8m0 scales.
    MXFP4 path: as MXFP8, with w1 [E, 2H, D/2] and w2 [E, D, H/2] packed e2m1
    codes (moe_ffn_mxfp4_quantize); x stays e4m3.
    topk_ids int32 [T, k] (int64 is converted), topk_weights fp32 [T, k].
    stream: the torch stream to run on (default: the current one); the
    wrapper's temporaries are allocated on it.
    events: optional 5 hipEvent_t handles (ints) recorded at the stage
    boundaries (moe_ffn_forward_events).
    """
    T, D, H, E, k, path = _pass_shapes(x, w1, w2, topk_ids, topk_weights, out, x_scale, w1_scale, w2_scale)
    _check_cuda(x, w1, w2, topk_ids, topk_weights, out, x_scale, w1_scale, w2_scale, workspace)
    lib = library()
    m = _mode(mode)
    with _on(stream) as s:
        topk_ids = _ids32(topk_ids)
        if out is None:
            out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
        p = make_problem(T, D, H, E, k, path, x_scale, w1_scale, w2_scale)
        if workspace is None:
            workspace = _workspace(lib, p, m, x.device, "moe_ffn_forward")
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
        args = (ctypes.byref(p), x.data_ptr(), w1.data_ptr(), w2.data_ptr(), topk_ids.data_ptr(),
                topk_weights.data_ptr(), out.data_ptr(), m, _sp(s))
        if events is None:
            rc = lib.moe_ffn_forward(*args)
        else:
            rc = lib.moe_ffn_forward_events(*args, *_events(events))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_forward")
    return out


def moe_ffn_forward_noalloc(x, w1, w2, topk_ids, topk_weights, out, mode="auto", x_scale=None, w1_scale=None,
                            w2_scale=None, stream=None):
    """moe_ffn_forward on the library's static scratch array (moe_ffn_forward_noalloc):
    neither the library nor this wrapper allocates, so `out` must be given and
    topk_ids must already be int32. Raises MoeFfnError (MOE_FFN_ESCRATCH) for a
    problem whose workspace exceeds MOE_FFN_NOALLOC_SCRATCH_BYTES. Calls that
    overlap on one GPU share the array and race."""
    if out is None or topk_ids.dtype != torch.int32:
        raise ValueError("moe_ffn_forward_noalloc needs `out` and int32 topk_ids (it allocates nothing)")
    T, D, H, E, k, path = _pass_shapes(x, w1, w2, topk_ids, topk_weights, out, x_scale, w1_scale, w2_scale)
    _check_cuda(x, w1, w2, topk_ids, topk_weights, out, x_scale, w1_scale, w2_scale)
    p = make_problem(T, D, H, E, k, path, x_scale, w1_scale, w2_scale)
    s = torch.cuda.current_stream() if stream is None else stream
    rc = library().moe_ffn_forward_noalloc(ctypes.byref(p), x.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                                           topk_ids.data_ptr(), topk_weights.data_ptr(), out.data_ptr(),
                                           _mode(mode), _sp(s))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_forward_noalloc")
    return out


def moe_ffn_router(logits, k, stream=None):
    """(topk_ids int32 [T, k], topk_weights fp32 [T, k]) from fp32 logits [T, E] on the GPU:
    softmax, the k most probable experts (ties to the lower id), renormalized."""
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be float32 [T, E]")
    _check_cuda(logits)
    T, E = logits.shape
    with _on(stream) as s:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        wts = torch.empty((T, k), dtype=torch.float32, device=logits.device)
        rc = library().moe_ffn_router(logits.data_ptr(), T, E, k, ids.data_ptr(), wts.data_ptr(), _sp(s))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_router")
    return ids, wts


def moe_ffn_forward_logits(x, w1, w2, logits, k, out=None, mode="auto", x_scale=None, w1_scale=None,
                           w2_scale=None, workspace=None, topk_ids=None, topk_weights=None, stream=None,
                           events=None):
    """(out, topk_ids, topk_weights): the router on fp32 logits [T, E], then the pass
    (moe_ffn_forward_logits). Tensors as in moe_ffn_forward; ids/weights are
    written into `topk_ids` / `topk_weights` when given."""
    if logits.dtype != torch.float32:
        raise ValueError("logits must be float32")
    T, D = x.shape
    E = w1.shape[0]
    if tuple(logits.shape) != (T, E):
        raise ValueError("logits must be [T, E]")
    dev = x.device
    with _on(stream) as s:
        if topk_ids is None:
            topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        if topk_weights is None:
            topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
        if topk_ids.dtype != torch.int32:
            raise ValueError("topk_ids (an output here) must be int32")
        _T, _D, H, _E, _k, path = _pass_shapes(x, w1, w2, topk_ids, topk_weights, out, x_scale, w1_scale,
                                               w2_scale)
        if _k != k:
            raise ValueError("topk_ids must be [T, k]")
        _check_cuda(x, w1, w2, logits, topk_ids, topk_weights, out, x_scale, w1_scale, w2_scale, workspace)
        if out is None:
            out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        p = make_problem(T, D, H, E, k, path, x_scale, w1_scale, w2_scale)
        lib = library()
        m = _mode(mode)
        if workspace is None:
            workspace = _workspace(lib, p, m, dev, "moe_ffn_forward_logits")
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
        rc = lib.moe_ffn_forward_logits(ctypes.byref(p), x.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                                        logits.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(),
                                        out.data_ptr(), m, _sp(s), *_events(events))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_forward_logits")
    return out, topk_ids, topk_weights


def moe_ffn_forward_shared(x, w1, w2, topk_ids, topk_weights, shared_w1, shared_w2, out=None, mode="auto",
                           workspace=None, stream=None, events=None):
    """out [T, D] bf16 = the routed pass plus one shared expert on every token
    (shared_w1 [2Hs, D], shared_w2 [D, Hs] bf16), added with weight 1."""
    T, D, H, E, k, path = _pass_shapes(x, w1, w2, topk_ids, topk_weights, out)
    if path != "bf16":
        raise MoeFfnError(MOE_FFN_EUNSUPPORTED, "moe_ffn_forward_shared")
    Hs = shared_w1.shape[0] // 2
    _expect(shared_w1, (2 * Hs, D), torch.bfloat16, "shared_w1")
    _expect(shared_w2, (D, Hs), torch.bfloat16, "shared_w2")
    _check_cuda(x, w1, w2, topk_ids, topk_weights, shared_w1, shared_w2, out, workspace)
    lib = library()
    m = _mode(mode)
    with _on(stream) as s:
        topk_ids = _ids32(topk_ids)
        if out is None:
            out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
        p = make_problem(T, D, H, E, k, "bf16")
        if workspace is None:
            workspace = _workspace(lib, p, m, x.device, "moe_ffn_forward_shared",
                                   lib.moe_ffn_shared_workspace_bytes(ctypes.byref(p), Hs, m))
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
        rc = lib.moe_ffn_forward_shared(ctypes.byref(p), x.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                                        topk_ids.data_ptr(), topk_weights.data_ptr(), shared_w1.data_ptr(),
                                        shared_w2.data_ptr(), Hs, out.data_ptr(), m, _sp(s), *_events(events))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_forward_shared")
    return out


def moe_ffn_forward_act(x, w1, w2, topk_ids, topk_weights, kind="clamped_swiglu", limit=0.0, alpha=None,
                        weight_before_act=False, out=None, mode="split", workspace=None, stream=None, events=None):
    """out [T, D] bf16 = the pass with the activation variant (moe_ffn_forward_act):
    gate/up scaled by alpha [E] fp32 (or 1) and, with weight_before_act, by the
    routing weight; kind "clamped_swiglu" clamps gate from above and up on both
    sides at `limit`."""
    T, D, H, E, k, path = _pass_shapes(x, w1, w2, topk_ids, topk_weights, out)
    if path != "bf16":
        raise MoeFfnError(MOE_FFN_EUNSUPPORTED, "moe_ffn_forward_act")
    if alpha is not None:
        _expect(alpha, (E,), torch.float32, "alpha")
    _check_cuda(x, w1, w2, topk_ids, topk_weights, out, alpha, workspace)
    kinds = {"swiglu": MOE_FFN_ACT_SWIGLU, "clamped_swiglu": MOE_FFN_ACT_CLAMPED_SWIGLU}
    act = moe_ffn_activation(kinds.get(kind, kind) if isinstance(kind, str) else kind, float(limit),
                             alpha.data_ptr() if alpha is not None else None, 1 if weight_before_act else 0)
    lib = library()
    m = _mode(mode)
    with _on(stream) as s:
        topk_ids = _ids32(topk_ids)
        if out is None:
            out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
        p = make_problem(T, D, H, E, k, "bf16")
        if workspace is None:
            workspace = _workspace(lib, p, MOE_FFN_SPLIT, x.device, "moe_ffn_forward_act")
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
        rc = lib.moe_ffn_forward_act(ctypes.byref(p), x.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                                     topk_ids.data_ptr(), topk_weights.data_ptr(), ctypes.byref(act),
                                     out.data_ptr(), m, _sp(s), *_events(events))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_forward_act")
    return out


def moe_ffn_route(topk_ids, E, stream=None):
    """(counts [E], offsets [E+1], sorted_to_pair [P], pair_to_sorted [P]) int32 on the GPU."""
    if topk_ids.dim() != 2 or topk_ids.dtype not in (torch.int32, torch.int64):
        raise ValueError("topk_ids must be int32 (or int64) [T, k]")
    _check_cuda(topk_ids)
    T, k = topk_ids.shape
    P = T * k
    dev = topk_ids.device
    lib = library()
    nbytes = lib.moe_ffn_route_workspace_bytes(T, k, E)
    if nbytes == 0:
        raise MoeFfnError(MOE_FFN_EINVAL_SHAPE, "moe_ffn_route")
    with _on(stream) as s:
        topk_ids = _ids32(topk_ids)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        s2p = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
        p2s = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        rc = lib.moe_ffn_route(topk_ids.data_ptr(), T, k, E, counts.data_ptr(), offsets.data_ptr(),
                               s2p.data_ptr(), p2s.data_ptr(), ws.data_ptr(), nbytes, _sp(s))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, "moe_ffn_route")
    return counts, offsets, s2p[:P], p2s[:P]


def _quantize(fn, src, code_cols, what, stream):
    if src.dtype != torch.float32 or src.dim() < 1:
        raise ValueError("src must be float32")
    _check_cuda(src)
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    with _on(stream) as s:
        codes = torch.empty(src.shape[:-1] + (code_cols(K),), dtype=torch.uint8, device=src.device)
        scales = torch.empty(src.shape[:-1] + (K // 32,), dtype=torch.uint8, device=src.device)
        rc = fn(src.data_ptr(), rows, K, codes.data_ptr(), scales.data_ptr(), _sp(s))
    if rc != MOE_FFN_OK:
        raise MoeFfnError(rc, what)
    return codes, scales


def moe_ffn_mx_quantize(src, stream=None):
    """MX-fp8 quantization along the last dim: (codes uint8, scales uint8 [..., K/32])."""
    return _quantize(library().moe_ffn_mx_quantize, src, lambda K: K, "moe_ffn_mx_quantize", stream)


def moe_ffn_mxfp4_quantize(src, stream=None):
    """MXFP4 quantization along the last dim (expert weights): (packed e2m1 codes uint8 [..., K/2],
    even index in the low nibble; scales uint8 [..., K/32])."""
    return _quantize(library().moe_ffn_mxfp4_quantize, src, lambda K: K // 2, "moe_ffn_mxfp4_quantize", stream)
