"""CPU oracle for the routed MoE SwiGLU FFN forward pass (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the
``grouped_gemm_amd`` package and its HIP library) never does.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp32 accumulation, one
OpenMP loop over tokens). What each function follows is stated there and in
the docstrings below. Parity status of every function: pinned by the
``-m "not gpu"`` tests (brute-force dense fp64 loop, the E=1/k=1 dense
SwiGLU FFN, invariants, and the e4m3 format's own definition).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# The same source built for the host it runs on, for the CPU-baseline timing
# only (-O3 -march=native; still no fast-math and no FMA contraction, so the
# results are the checker's bit for bit).
_NATIVE_LIB = os.path.join(_HERE, "libmoe_oracle_native.so")
_FLAGS = ["-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
_lib = None
_native = None


def _compile(out: str, opt) -> str:
    tmp = out + ".tmp"
    subprocess.run(["gcc", *opt, *_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the checker build of the oracle with gcc (-O2, portable x86-64-v2,
    OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        _compile(_LIB, ["-O2", "-march=x86-64-v2"])
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def use_native_build() -> None:
    """Route the forward functions below through the -O3 -march=native build of
    the same source, compiled here for this host (the CPU-baseline timing)."""
    global _native, _lib
    if _native is None:
        _native = _bind(ctypes.CDLL(_compile(_NATIVE_LIB, ["-O3", "-march=native"])))
    _load()
    _lib = _native


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def _bind(lib):
    """Declare the C signatures on a loaded build of moe_oracle.c."""
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_route.argtypes = [P, i64, i32, i32, P, P, P, P]
    lib.oracle_router.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_forward_bf16.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, i64]
    lib.oracle_forward_bf16_act.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, i32, ctypes.c_float, P,
                                            i32, P, P, i64]
    lib.oracle_forward_bf16_shared.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, P, P,
                                               i64]
    lib.oracle_forward_mx.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                      P, i64, i32]
    lib.oracle_forward_mx4.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                       P, i64, i32]
    lib.oracle_mx_quantize.argtypes = [P, i64, i64, P, P]
    lib.oracle_mx4_quantize.argtypes = [P, i64, i64, P, P]
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_decode.restype = ctypes.c_float
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_float]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_mx4_scale_exp.argtypes = [P, ctypes.c_int]
    lib.oracle_mx4_scale_exp.restype = ctypes.c_int
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_float
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_mx_scale_exp.argtypes = [P, ctypes.c_int]
    lib.oracle_mx_scale_exp.restype = ctypes.c_int
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def route(topk_ids: np.ndarray, E: int):
    """Stable counting sort of pairs p = t*k + j by expert.

    Returns counts [E], offsets [E+1], sorted_to_pair [P] (-1 past
    offsets[E]), pair_to_sorted [P] (-1 for dropped routes), all int32.
    Prime Flash MoE, section 8: routing and sorting produce the per-expert
    row order the grouped GEMMs consume (its `offs` group offsets, section 1).
    """
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    P = T * k
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    s2p = np.zeros(max(P, 1), np.int32)
    p2s = np.zeros(max(P, 1), np.int32)
    _load().oracle_route(_p(ids), T, k, E, _p(counts), _p(offsets), _p(s2p), _p(p2s))
    return counts, offsets, s2p[:P], p2s[:P]


def router(logits: np.ndarray, k: int):
    """Softmax -> top-k -> renormalize: (topk_ids int32 [T, k], topk_weights fp32 [T, k]).

    Prime Flash MoE, section 1: the pass starts from each token's top-k
    experts and normalized routing weights. Order: largest logit first, ties
    to the lower expert id (softmax is increasing in the logit); weights are
    the selected softmax probabilities divided by their sum, in double,
    rounded once to fp32.
    """
    lg = _c(logits, np.float32)
    T, E = lg.shape
    assert 1 <= k <= E
    ids = np.zeros((T, k), np.int32)
    wts = np.zeros((T, k), np.float32)
    if T:
        _load().oracle_router(_p(lg), T, E, k, _p(ids), _p(wts))
    return ids, wts


def forward_bf16(x, w1, w2, topk_ids, topk_weights, tokens=None, shared=None):
    """bf16 forward: out bf16 bits [T, D] (rows not in `tokens` stay 0).

    x [T, D], w1 [E, 2H, D], w2 [E, D, H] as uint16 bf16 bits; ids int32
    [T, k]; weights fp32 [T, k]. Prime Flash MoE, section 1.
    shared = (ws1 [2Hs, D], ws2 [D, Hs]) adds one shared expert on every
    token with weight 1 ("GC-MoE on SM120", section 4.7).
    """
    x, w1, w2 = _c(x, np.uint16), _c(w1, np.uint16), _c(w2, np.uint16)
    ids, wts = _c(topk_ids, np.int32), _c(topk_weights, np.float32)
    T, D = x.shape
    E, H2, D1 = w1.shape
    H = H2 // 2
    k = ids.shape[1]
    assert D1 == D and w2.shape == (E, D, H) and ids.shape == wts.shape == (T, k)
    out = np.zeros((T, D), np.uint16)
    if tokens is None:
        tok_p, n = None, T
    else:
        tok = _c(tokens, np.int64)
        tok_p, n = _p(tok), tok.size
    if shared is None:
        _load().oracle_forward_bf16(T, D, H, E, k, _p(x), _p(w1), _p(w2), _p(ids), _p(wts), _p(out),
                                    tok_p, n)
    else:
        ws1, ws2 = _c(shared[0], np.uint16), _c(shared[1], np.uint16)
        Hs = ws1.shape[0] // 2
        assert ws1.shape == (2 * Hs, D) and ws2.shape == (D, Hs)
        _load().oracle_forward_bf16_shared(T, D, H, E, k, _p(x), _p(w1), _p(w2), _p(ids), _p(wts), _p(ws1),
                                           _p(ws2), Hs, _p(out), tok_p, n)
    return out


def forward_bf16_act(x, w1, w2, topk_ids, topk_weights, kind=0, limit=0.0, alpha=None,
                     weight_before_act=False, tokens=None):
    """bf16 forward with the activation variant: kind 0 = SwiGLU, 1 = SwiGLU on
    gate clamped from above and up clamped on both sides at `limit`; gate
    and up scaled first by alpha[e] (per expert, fp32) and, with
    weight_before_act, by the routing weight, which then does not scale the
    expert output ("Porting Block-Scaled GEMM Kernels from Blackwell to
    Rubin", section 5.3; "GC-MoE on SM120", section 4.8)."""
    x, w1, w2 = _c(x, np.uint16), _c(w1, np.uint16), _c(w2, np.uint16)
    ids, wts = _c(topk_ids, np.int32), _c(topk_weights, np.float32)
    T, D = x.shape
    E, H2, _ = w1.shape
    H = H2 // 2
    k = ids.shape[1]
    out = np.zeros((T, D), np.uint16)
    al = None if alpha is None else _c(alpha, np.float32)
    if tokens is None:
        tok_p, n = None, T
    else:
        tok = _c(tokens, np.int64)
        tok_p, n = _p(tok), tok.size
    _load().oracle_forward_bf16_act(T, D, H, E, k, _p(x), _p(w1), _p(w2), _p(ids), _p(wts), int(kind), float(limit),
                                    None if al is None else _p(al), 1 if weight_before_act else 0, _p(out), tok_p, n)
    return out


def mx_quantize(src: np.ndarray):
    """MXQ along the last dim: (codes uint8 same shape, scales uint8 [..., K/32])."""
    src = _c(src, np.float32)
    K = src.shape[-1]
    assert K % 32 == 0
    rows = src.size // K if K else 0
    codes = np.zeros(src.shape, np.uint8)
    scales = np.zeros(src.shape[:-1] + (K // 32,), np.uint8)
    _load().oracle_mx_quantize(_p(src), rows, K, _p(codes), _p(scales))
    return codes, scales


def forward_mx(xc, xs, w1c, w1s, w2c, w2s, topk_ids, topk_weights, tokens=None, requant=True):
    """MX-fp8 forward: out bf16 bits [T, D]. Prime Flash MoE, section 7."""
    arrs = [_c(a, np.uint8) for a in (xc, xs, w1c, w1s, w2c, w2s)]
    xc, xs, w1c, w1s, w2c, w2s = arrs
    ids, wts = _c(topk_ids, np.int32), _c(topk_weights, np.float32)
    T, D = xc.shape
    E, H2, _ = w1c.shape
    H = H2 // 2
    k = ids.shape[1]
    assert xs.shape == (T, D // 32) and w1s.shape == (E, H2, D // 32)
    assert w2c.shape == (E, D, H) and w2s.shape == (E, D, H // 32)
    out = np.zeros((T, D), np.uint16)
    if tokens is None:
        tok_p, n = None, T
    else:
        tok = _c(tokens, np.int64)
        tok_p, n = _p(tok), tok.size
    _load().oracle_forward_mx(T, D, H, E, k, _p(xc), _p(xs), _p(w1c), _p(w1s), _p(w2c), _p(w2s),
                              _p(ids), _p(wts), _p(out), tok_p, n, 1 if requant else 0)
    return out


def mx4_quantize(src: np.ndarray):
    """MXQ4 along the last dim: (packed e2m1 codes uint8 [..., K/2], even index in the low nibble;
    scales uint8 [..., K/32]). GC-MoE on SM120, scale formats; the rule is MXQ with 6 for 448."""
    src = _c(src, np.float32)
    K = src.shape[-1]
    assert K % 32 == 0
    rows = src.size // K if K else 0
    codes = np.zeros(src.shape[:-1] + (K // 2,), np.uint8)
    scales = np.zeros(src.shape[:-1] + (K // 32,), np.uint8)
    _load().oracle_mx4_quantize(_p(src), rows, K, _p(codes), _p(scales))
    return codes, scales


def forward_mx4(xc, xs, w1c, w1s, w2c, w2s, topk_ids, topk_weights, tokens=None, requant=True):
    """MXFP4-weight forward (e2m1 weights, e4m3 activations): out bf16 bits [T, D].
    w1c packed [E, 2H, D/2], w2c packed [E, D, H/2]; scales as for forward_mx."""
    arrs = [_c(a, np.uint8) for a in (xc, xs, w1c, w1s, w2c, w2s)]
    xc, xs, w1c, w1s, w2c, w2s = arrs
    ids, wts = _c(topk_ids, np.int32), _c(topk_weights, np.float32)
    T, D = xc.shape
    E, H2, _ = w1c.shape
    H = H2 // 2
    k = ids.shape[1]
    assert w1c.shape == (E, H2, D // 2) and xs.shape == (T, D // 32) and w1s.shape == (E, H2, D // 32)
    assert w2c.shape == (E, D, H // 2) and w2s.shape == (E, D, H // 32)
    out = np.zeros((T, D), np.uint16)
    if tokens is None:
        tok_p, n = None, T
    else:
        tok = _c(tokens, np.int64)
        tok_p, n = _p(tok), tok.size
    _load().oracle_forward_mx4(T, D, H, E, k, _p(xc), _p(xs), _p(w1c), _p(w1s), _p(w2c), _p(w2s),
                               _p(ids), _p(wts), _p(out), tok_p, n, 1 if requant else 0)
    return out


def e2m1_decode(code: int) -> float:
    return float(_load().oracle_e2m1_decode(int(code)))


def e2m1_encode(v: float) -> int:
    return int(_load().oracle_e2m1_encode(float(v)))


def mx4_scale_exp(block: np.ndarray) -> int:
    b = _c(block, np.float32)
    return int(_load().oracle_mx4_scale_exp(_p(b), b.size))


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code)))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def mx_scale_exp(block: np.ndarray) -> int:
    b = _c(block, np.float32)
    return int(_load().oracle_mx_scale_exp(_p(b), b.size))


def f32_to_bf16(v: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(v)))
