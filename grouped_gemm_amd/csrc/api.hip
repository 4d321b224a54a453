// Host side of the C ABI declared in include/moe_ffn.h: validation,
// workspace planning and kernel dispatch. No device memory is allocated
// here; every buffer comes from the caller.
#include "moe_ffn.h"

#include <climits>
#include <mutex>

#include "common.h"

// Scratch memory of moe_ffn_forward_noalloc: one array per device (each GPU
// the library runs on holds its own copy from module load until the process
// ends). In host code `scratch` names a host-side stand-in, not device
// memory: host code only ever uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_FFN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxExperts = 8192;
constexpr int kMaxTopk = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const moe_ffn_problem* p) {
    if (!p) return MOE_FFN_EINVAL_PTR;
    if (p->dtype != MOE_FFN_BF16 && p->dtype != MOE_FFN_MXFP8 && p->dtype != MOE_FFN_MXFP4)
        return MOE_FFN_EUNSUPPORTED;
    if (p->T < 0 || p->D < 1 || p->H < 1 || p->E < 1 || p->topk < 1) return MOE_FFN_EINVAL_SHAPE;
    // bf16: multiples of 64 (one 64-element K step of the generic kernels);
    // MX: multiples of 128 (the MX kernels stage K in 128-code steps)
    const int mult = p->dtype == MOE_FFN_BF16 ? 64 : 128;
    if (p->D % mult || p->H % mult) return MOE_FFN_EINVAL_SHAPE;
    if (p->E > kMaxExperts || p->topk > kMaxTopk || p->topk > p->E) return MOE_FFN_EINVAL_SHAPE;
    if (static_cast<int64_t>(p->T) * p->topk > INT_MAX) return MOE_FFN_EINVAL_SHAPE;
    return MOE_FFN_OK;
}

// AUTO resolves to the fused pipeline for bf16 passes bound by launch
// latency (moe::fused_preferred: a few MB of expert weights streamed, where
// its two kernels beat the split pipeline's four), for MX-fp8 passes whose
// fused blocks fit one round of the CUs (moe::mx_fused_preferred), and to
// the split pipeline otherwise: where the weights stream from HBM the split
// pipeline's decode kernels are as fast or faster, and at prefill sizes the
// fused pipeline's split-K partial rows cost fp32 atomic adds into the
// accumulator (P * H/slice * D of them, at about 330 G adds/s on MI355X's
// L2) and each expert's weights are streamed once per 32-row m-tile.
int resolve(const moe_ffn_problem* p, int mode) {
    if (mode != MOE_FFN_AUTO && mode != MOE_FFN_FUSED && mode != MOE_FFN_SPLIT) return MOE_FFN_EUNSUPPORTED;
    if (p->dtype == MOE_FFN_MXFP4) return mode == MOE_FFN_FUSED ? MOE_FFN_EUNSUPPORTED : MOE_FFN_SPLIT;
    if (mode == MOE_FFN_AUTO) {
        const bool fused = p->dtype == MOE_FFN_BF16 ? moe::fused_preferred(p->T, p->D, p->H, p->E, p->topk)
                                                    : moe::mx_fused_preferred(p->T, p->D, p->H, p->E, p->topk);
        return fused ? MOE_FFN_FUSED : MOE_FFN_SPLIT;
    }
    return mode;
}

struct RoutePlan {
    int64_t P;
    int32_t seg, S;
    size_t tile_prefix, seg_counts, end;  // byte offsets from the route base
};

RoutePlan plan_route(int64_t T, int32_t k, int32_t E, size_t base) {
    RoutePlan r;
    r.P = T * k;
    r.seg = 256;
    r.S = static_cast<int32_t>((r.P + r.seg - 1) / r.seg);
    while (static_cast<int64_t>(r.S) * E > (1 << 22)) {
        r.seg *= 2;
        r.S = static_cast<int32_t>((r.P + r.seg - 1) / r.seg);
    }
    size_t off = base;
    r.tile_prefix = off;
    off = align_up(off + sizeof(int32_t) * moe::kNumTileHeights * (E + 1));
    r.seg_counts = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(r.S) * E);
    r.end = off;
    return r;
}

struct Plan {
    int mode;
    RoutePlan route;
    size_t counts, offsets, s2p, p2s;
    size_t act, act_s, ypair, acc32, tcnt, clear_end, mtiles;
    size_t total;
};

Plan make_plan(const moe_ffn_problem* p, int mode) {
    Plan pl{};
    pl.mode = mode;
    const int64_t P = static_cast<int64_t>(p->T) * p->topk;
    size_t off = 0;
    pl.counts = off;
    off = align_up(off + sizeof(int32_t) * p->E);
    pl.offsets = off;
    off = align_up(off + sizeof(int32_t) * (p->E + 1));
    pl.s2p = off;
    off = align_up(off + sizeof(int32_t) * (P + moe::kRowMapPad));
    pl.p2s = off;
    off = align_up(off + sizeof(int32_t) * P);
    pl.route = plan_route(p->T, p->topk, p->E, off);
    off = pl.route.end;
    if (mode == MOE_FFN_SPLIT) {
        const size_t act_elem = p->dtype == MOE_FFN_BF16 ? 2 : 1;
        pl.act = off;
        off = align_up(off + act_elem * static_cast<size_t>(P) * p->H);
        if (p->dtype != MOE_FFN_BF16) {
            pl.act_s = off;
            off = align_up(off + static_cast<size_t>(P) * (p->H / 32));
        }
        pl.ypair = off;
        off = align_up(off + 2 * static_cast<size_t>(P) * p->D);
        pl.mtiles = off;
        off = align_up(off + static_cast<size_t>(moe::big_gemm_workspace_bytes(P, p->E)));
    } else {
        // the accumulator, then the per-token counters; the route step clears both
        pl.acc32 = off;
        off += 4 * static_cast<size_t>(p->T) * p->D;
        pl.tcnt = off;
        off += (4 * static_cast<size_t>(p->T) + 15) & ~size_t(15);
        pl.clear_end = off;
        off = align_up(off);
    }
    pl.total = off;
    return pl;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

MOE_FFN_API const char* moe_ffn_strerror(int code) {
    switch (code) {
        case MOE_FFN_OK: return "ok";
        case MOE_FFN_EINVAL_SHAPE: return "invalid shape";
        case MOE_FFN_EINVAL_PTR: return "invalid (null or misaligned) pointer";
        case MOE_FFN_EUNSUPPORTED: return "unsupported dtype or mode";
        case MOE_FFN_EWORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_FFN_EHIP: return "HIP launch error";
        case MOE_FFN_ESCRATCH: return "problem needs more scratch than the library's static buffer holds";
        default: return "unknown error";
    }
}

MOE_FFN_API int moe_ffn_validate(const moe_ffn_problem* p, int mode) {
    int rc = check_shape(p);
    if (rc != MOE_FFN_OK) return rc;
    rc = resolve(p, mode);
    return rc < 0 ? rc : MOE_FFN_OK;
}

MOE_FFN_API int moe_ffn_resolve_mode(const moe_ffn_problem* p, int mode) {
    int rc = check_shape(p);
    if (rc != MOE_FFN_OK) return rc;
    return resolve(p, mode);
}

MOE_FFN_API const char* moe_ffn_gemm_kernel(const moe_ffn_problem* p, int mode, int gemm) {
    if ((gemm != 1 && gemm != 2) || check_shape(p) != MOE_FFN_OK) return nullptr;
    const int m = resolve(p, mode);
    if (m < 0) return nullptr;
    if (p->T == 0) return "none";
    const bool g1 = gemm == 1;
    // the predicates below only test the m-tile table pointer for null; the
    // split pipeline's workspace always holds the table
    static int32_t table_stand_in;
    if (p->dtype == MOE_FFN_BF16) {
        moe::Bf16Args a{};
        a.T = p->T; a.D = p->D; a.H = p->H; a.E = p->E; a.k = p->topk;
        a.P = static_cast<int64_t>(p->T) * p->topk;
        if (m == MOE_FFN_FUSED) return moe::fused_decode_supported(a) ? "fused_dma_kernel" : "fused_bf16_kernel";
        a.mtiles = &table_stand_in;
        if (moe::bf16_uses_decode_kernels(a))
            return moe::decode_kernel_name(a, g1);
        if (moe::big_gemm_supported(a))
            return moe::big_gemm_tile_rows(a) == 256 ? "big_gemm_kernel<256>" : "big_gemm_kernel<128>";
        return g1 ? "gemm1_swiglu_kernel" : "gemm2_weight_kernel";
    }
    if (m == MOE_FFN_FUSED) {
        moe::MxArgs f{};
        f.T = p->T; f.D = p->D; f.H = p->H; f.E = p->E; f.k = p->topk;
        f.w4 = p->dtype == MOE_FFN_MXFP4;
        return moe::mx_fused_dma_supported(f) ? "mx_fused_dma_kernel" : "mx_fused_kernel";
    }
    moe::MxArgs a{};
    a.T = p->T; a.D = p->D; a.H = p->H; a.E = p->E; a.k = p->topk;
    a.P = static_cast<int64_t>(p->T) * p->topk;
    a.w4 = p->dtype == MOE_FFN_MXFP4;
    a.mtiles = &table_stand_in;
    if (moe::big_mx_supported(a)) return "big_gemm_kernel<256>";
    if (moe::skinny_mx_supported(a)) return moe::mx_decode_kernel_name(a, g1);
    return g1 ? "mx_gemm1_kernel" : "mx_gemm2_kernel";
}

MOE_FFN_API size_t moe_ffn_workspace_bytes(const moe_ffn_problem* p, int mode) {
    if (check_shape(p) != MOE_FFN_OK) return 0;
    const int m = resolve(p, mode);
    if (m < 0) return 0;
    return make_plan(p, m).total;
}

MOE_FFN_API size_t moe_ffn_route_workspace_bytes(int32_t T, int32_t topk, int32_t E) {
    if (T < 0 || topk < 1 || E < 1 || E > kMaxExperts || topk > kMaxTopk) return 0;
    if (static_cast<int64_t>(T) * topk > INT_MAX) return 0;
    return plan_route(T, topk, E, 0).end;
}

MOE_FFN_API int moe_ffn_route(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_to_pair, int32_t* pair_to_sorted,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0 || topk < 1 || E < 1 || E > kMaxExperts || topk > kMaxTopk) return MOE_FFN_EINVAL_SHAPE;
    if (static_cast<int64_t>(T) * topk > INT_MAX) return MOE_FFN_EINVAL_SHAPE;
    const int64_t P = static_cast<int64_t>(T) * topk;
    if (!counts || !offsets) return MOE_FFN_EINVAL_PTR;
    if (P > 0 && (!topk_ids || !sorted_to_pair || !pair_to_sorted)) return MOE_FFN_EINVAL_PTR;
    const RoutePlan rp = plan_route(T, topk, E, 0);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) || workspace_bytes < rp.end)
        return MOE_FFN_EWORKSPACE;
    moe::RouteBuffers b{topk_ids, P, E, rp.S, rp.seg, at<int32_t>(workspace, rp.seg_counts), counts, offsets,
                        at<int32_t>(workspace, rp.tile_prefix), sorted_to_pair, pair_to_sorted};
    return moe::launch_route(b, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_FFN_OK : MOE_FFN_EHIP;
}

MOE_FFN_API int moe_ffn_mx_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                                    void* stream) {
    if (rows < 0 || K < 32 || K % 32) return MOE_FFN_EINVAL_SHAPE;
    if (rows == 0) return MOE_FFN_OK;
    if (!src || !codes || !scales || !aligned16(src) || (reinterpret_cast<uintptr_t>(codes) & 3u))
        return MOE_FFN_EINVAL_PTR;
    return moe::launch_mx_quantize(src, rows, K, codes, scales, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_FFN_OK
               : MOE_FFN_EHIP;
}

MOE_FFN_API int moe_ffn_mxfp4_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                                       void* stream) {
    if (rows < 0 || K < 32 || K % 32) return MOE_FFN_EINVAL_SHAPE;
    if (rows == 0) return MOE_FFN_OK;
    if (!src || !codes || !scales || !aligned16(src) || (reinterpret_cast<uintptr_t>(codes) & 3u))
        return MOE_FFN_EINVAL_PTR;
    return moe::launch_mx4_quantize(src, rows, K, codes, scales, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_FFN_OK
               : MOE_FFN_EHIP;
}

MOE_FFN_API int moe_ffn_router(const float* logits, int32_t T, int32_t E, int32_t topk, int32_t* topk_ids,
                               float* topk_weights, void* stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || topk < 1 || topk > kMaxTopk || topk > E) return MOE_FFN_EINVAL_SHAPE;
    if (static_cast<int64_t>(T) * topk > INT_MAX) return MOE_FFN_EINVAL_SHAPE;
    if (T == 0) return MOE_FFN_OK;
    if (!logits || !topk_ids || !topk_weights || (reinterpret_cast<uintptr_t>(logits) & 3u) ||
        (reinterpret_cast<uintptr_t>(topk_ids) & 3u) || (reinterpret_cast<uintptr_t>(topk_weights) & 3u))
        return MOE_FFN_EINVAL_PTR;
    return moe::launch_router(logits, T, E, topk, topk_ids, topk_weights, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? MOE_FFN_OK
               : MOE_FFN_EHIP;
}

MOE_FFN_API int moe_ffn_forward(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2,
                                const int32_t* topk_ids, const float* topk_weights, void* out, int mode,
                                void* stream) {
    return moe_ffn_forward_events(p, x, w1, w2, topk_ids, topk_weights, out, mode, stream, nullptr, 0);
}

namespace {
struct SharedExpert {
    const void* w1;  // bf16 [2Hs, D]
    const void* w2;  // bf16 [D, Hs]
    int32_t Hs;
};
int forward_impl(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2, const float* logits,
                 const int32_t* topk_ids, const float* topk_weights, const SharedExpert* sh,
                 const moe_ffn_activation* act, void* out, int mode, void* stream, void* const* events, int n_events);

// The activation variant's own checks (bf16, the split pipeline).
int check_act(const moe_ffn_problem* p, const moe_ffn_activation* act, int mode) {
    if (act->kind != MOE_FFN_ACT_SWIGLU && act->kind != MOE_FFN_ACT_CLAMPED_SWIGLU) return MOE_FFN_EUNSUPPORTED;
    if (act->kind == MOE_FFN_ACT_CLAMPED_SWIGLU && !(act->limit > 0.0f && act->limit <= 3.0e38f))
        return MOE_FFN_EINVAL_SHAPE;
    if (act->weight_before_act != 0 && act->weight_before_act != 1) return MOE_FFN_EINVAL_SHAPE;
    if (act->alpha && (reinterpret_cast<uintptr_t>(act->alpha) & 3u)) return MOE_FFN_EINVAL_PTR;
    if (p->dtype != MOE_FFN_BF16 || mode == MOE_FFN_FUSED) return MOE_FFN_EUNSUPPORTED;
    return MOE_FFN_OK;
}

// The shared expert as its own split pass of one expert with k = 1.
moe_ffn_problem shared_problem(const moe_ffn_problem* p, int32_t Hs) {
    moe_ffn_problem q = *p;
    q.H = Hs;
    q.E = 1;
    q.topk = 1;
    q.dtype = MOE_FFN_BF16;
    q.x_scale = q.w1_scale = q.w2_scale = nullptr;
    return q;
}
// Workspace after the routed pass's plan: the shared pass's plan, then the
// unit weights of its identity routing.
size_t shared_bytes(const moe_ffn_problem* p, int32_t Hs) {
    const moe_ffn_problem q = shared_problem(p, Hs);
    return make_plan(&q, MOE_FFN_SPLIT).total + align_up(sizeof(float) * static_cast<size_t>(p->T));
}
int check_shared(const moe_ffn_problem* p, int32_t Hs) {
    if (p->dtype != MOE_FFN_BF16) return MOE_FFN_EUNSUPPORTED;  // an MX shared expert is not built
    if (Hs < 1 || Hs % 64) return MOE_FFN_EINVAL_SHAPE;
    return MOE_FFN_OK;
}
}  // namespace

MOE_FFN_API int moe_ffn_forward_events(const moe_ffn_problem* p, const void* x, const void* w1,
                                       const void* w2, const int32_t* topk_ids, const float* topk_weights,
                                       void* out, int mode, void* stream, void* const* events, int n_events) {
    return forward_impl(p, x, w1, w2, nullptr, topk_ids, topk_weights, nullptr, nullptr, out, mode, stream, events,
                        n_events);
}

MOE_FFN_API int moe_ffn_forward_act(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2,
                                    const int32_t* topk_ids, const float* topk_weights, const moe_ffn_activation* act,
                                    void* out, int mode, void* stream, void* const* events, int n_events) {
    if (!act) return MOE_FFN_EINVAL_PTR;
    return forward_impl(p, x, w1, w2, nullptr, topk_ids, topk_weights, nullptr, act, out, mode, stream, events,
                        n_events);
}

MOE_FFN_API size_t moe_ffn_shared_workspace_bytes(const moe_ffn_problem* p, int32_t Hs, int mode) {
    if (check_shape(p) != MOE_FFN_OK || check_shared(p, Hs) != MOE_FFN_OK) return 0;
    const int m = resolve(p, mode);
    if (m < 0) return 0;
    return make_plan(p, m).total + shared_bytes(p, Hs);
}

MOE_FFN_API int moe_ffn_forward_shared(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2,
                                       const int32_t* topk_ids, const float* topk_weights, const void* shared_w1,
                                       const void* shared_w2, int32_t Hs, void* out, int mode, void* stream,
                                       void* const* events, int n_events) {
    const SharedExpert sh{shared_w1, shared_w2, Hs};
    return forward_impl(p, x, w1, w2, nullptr, topk_ids, topk_weights, &sh, nullptr, out, mode, stream, events,
                        n_events);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL if the lookup failed.
static void* scratch_address() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

MOE_FFN_API int moe_ffn_forward_noalloc(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2,
                                        const int32_t* topk_ids, const float* topk_weights, void* out, int mode,
                                        void* stream) {
    int rc = check_shape(p);
    if (rc != MOE_FFN_OK) return rc;
    const int m = resolve(p, mode);
    if (m < 0) return m;
    if (make_plan(p, m).total > static_cast<size_t>(MOE_FFN_NOALLOC_SCRATCH_BYTES)) return MOE_FFN_ESCRATCH;
    if (p->T == 0) return MOE_FFN_OK;
    void* ws = scratch_address();
    if (!ws) return MOE_FFN_EHIP;
    moe_ffn_problem q = *p;
    q.workspace = ws;
    q.workspace_bytes = MOE_FFN_NOALLOC_SCRATCH_BYTES;
    return forward_impl(&q, x, w1, w2, nullptr, topk_ids, topk_weights, nullptr, nullptr, out, m, stream, nullptr,
                        0);
}

MOE_FFN_API int moe_ffn_forward_logits(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2,
                                       const float* logits, int32_t* topk_ids, float* topk_weights, void* out,
                                       int mode, void* stream, void* const* events, int n_events) {
    if (p && p->T > 0 && (!logits || (reinterpret_cast<uintptr_t>(logits) & 3u))) return MOE_FFN_EINVAL_PTR;
    return forward_impl(p, x, w1, w2, p && p->T > 0 ? logits : nullptr, topk_ids, topk_weights, nullptr, nullptr,
                        out, mode, stream, events, n_events);
}

}  // extern "C"

namespace {
// The pass from given routes (logits == NULL) or from router logits, which
// then fill topk_ids / topk_weights on the way; with `sh`, a shared expert
// runs first and its output joins the combine.
int forward_impl(const moe_ffn_problem* p, const void* x, const void* w1, const void* w2, const float* logits,
                 const int32_t* topk_ids, const float* topk_weights, const SharedExpert* sh,
                 const moe_ffn_activation* act, void* out, int mode, void* stream, void* const* events,
                 int n_events) {
    if (n_events != 0 && n_events != 5) return MOE_FFN_EINVAL_PTR;
    if (n_events == 5 && !events) return MOE_FFN_EINVAL_PTR;
    hipEvent_t ev[5];
    hipEvent_t* evp = nullptr;
    if (n_events == 5) {
        for (int i = 0; i < 5; ++i) {
            if (!events[i]) return MOE_FFN_EINVAL_PTR;
            ev[i] = static_cast<hipEvent_t>(events[i]);
        }
        evp = ev;
    }
    int rc = check_shape(p);
    if (rc != MOE_FFN_OK) return rc;
    if (sh && (rc = check_shared(p, sh->Hs)) != MOE_FFN_OK) return rc;
    if (act && (rc = check_act(p, act, mode)) != MOE_FFN_OK) return rc;
    int m = resolve(p, mode);
    if (m < 0) return m;
    if (act) m = MOE_FFN_SPLIT;  // AUTO: the variant runs on the split pipeline
    if (p->T == 0) return MOE_FFN_OK;
    const void* ptrs[] = {x, w1, w2, topk_ids, topk_weights, out};
    for (const void* q : ptrs)
        if (!q || !aligned16(q)) return MOE_FFN_EINVAL_PTR;
    if (sh && (!sh->w1 || !sh->w2 || !aligned16(sh->w1) || !aligned16(sh->w2))) return MOE_FFN_EINVAL_PTR;
    if (p->dtype != MOE_FFN_BF16) {
        const void* sp[] = {p->x_scale, p->w1_scale, p->w2_scale};
        for (const void* q : sp)
            if (!q || (reinterpret_cast<uintptr_t>(q) & 3u)) return MOE_FFN_EINVAL_PTR;
    }
    const Plan pl = make_plan(p, m);
    void* ws = p->workspace;
    const size_t need = pl.total + (sh ? shared_bytes(p, sh->Hs) : 0);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) || p->workspace_bytes < need)
        return MOE_FFN_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t P = static_cast<int64_t>(p->T) * p->topk;

    moe::record(evp, 0, st);
    const uint16_t* shared_y = nullptr;
    if (sh) {
        // the shared expert: one group of all T tokens through the split GEMMs
        const moe_ffn_problem q = shared_problem(p, sh->Hs);
        const Plan sp = make_plan(&q, MOE_FFN_SPLIT);
        void* sws = static_cast<char*>(ws) + pl.total;
        float* ones = at<float>(sws, sp.total);
        int32_t* tp = at<int32_t>(sws, sp.route.tile_prefix);
        if (moe::launch_identity_route(p->T, at<int32_t>(sws, sp.counts), at<int32_t>(sws, sp.offsets), tp,
                                       at<int32_t>(sws, sp.s2p), at<int32_t>(sws, sp.p2s), ones, st) != hipSuccess)
            return MOE_FFN_EHIP;
        moe::Bf16Args b{};
        b.T = p->T; b.D = p->D; b.H = sh->Hs; b.E = 1; b.k = 1; b.P = p->T;
        b.x = static_cast<const uint16_t*>(x);
        b.w1 = static_cast<const uint16_t*>(sh->w1);
        b.w2 = static_cast<const uint16_t*>(sh->w2);
        b.wts = ones;
        b.rv = moe::RouteView{at<int32_t>(sws, sp.counts), at<int32_t>(sws, sp.offsets), tp, at<int32_t>(sws, sp.s2p),
                              at<int32_t>(sws, sp.p2s)};
        b.act = at<uint16_t>(sws, sp.act);
        b.ypair = at<uint16_t>(sws, sp.ypair);
        b.mtiles = at<int32_t>(sws, sp.mtiles);
        if (moe::launch_gemms_bf16(b, st, nullptr) != hipSuccess) return MOE_FFN_EHIP;
        shared_y = b.ypair;  // [T, D]: pair t of the identity routing is token t
    }

    moe::RouteBuffers rb{topk_ids, P, p->E, pl.route.S, pl.route.seg, at<int32_t>(ws, pl.route.seg_counts),
                         at<int32_t>(ws, pl.counts), at<int32_t>(ws, pl.offsets),
                         at<int32_t>(ws, pl.route.tile_prefix), at<int32_t>(ws, pl.s2p), at<int32_t>(ws, pl.p2s)};
    if (m == MOE_FFN_FUSED) {
        rb.clear = at<float>(ws, pl.acc32);
        rb.clear_n = static_cast<int64_t>((pl.clear_end - pl.acc32) / 4);
    }
    const hipError_t re = logits ? moe::launch_router_route(logits, p->T, p->E, p->topk, const_cast<int32_t*>(topk_ids),
                                                            const_cast<float*>(topk_weights), rb, st)
                                 : moe::launch_route(rb, st);
    if (re != hipSuccess) return MOE_FFN_EHIP;
    moe::record(evp, 1, st);
    hipEvent_t* stage_ev = evp ? evp + 2 : nullptr;
    moe::RouteView rv{rb.counts, rb.offsets, rb.tile_prefix, rb.sorted_to_pair, rb.pair_to_sorted};

    hipError_t e;
    if (p->dtype == MOE_FFN_BF16) {
        moe::Bf16Args a{};
        a.T = p->T; a.D = p->D; a.H = p->H; a.E = p->E; a.k = p->topk; a.P = P;
        a.x = static_cast<const uint16_t*>(x);
        a.w1 = static_cast<const uint16_t*>(w1);
        a.w2 = static_cast<const uint16_t*>(w2);
        a.wts = topk_weights;
        a.rv = rv;
        a.out = static_cast<uint16_t*>(out);
        a.shared_y = shared_y;
        if (act) a.av = moe::ActVariant{act->kind, act->limit, act->alpha, act->weight_before_act};
        if (m == MOE_FFN_SPLIT) {
            a.act = at<uint16_t>(ws, pl.act);
            a.ypair = at<uint16_t>(ws, pl.ypair);
            a.mtiles = at<int32_t>(ws, pl.mtiles);
            e = moe::launch_split_bf16(a, st, stage_ev);
        } else {
            a.acc32 = at<float>(ws, pl.acc32);
            a.tcnt = at<int32_t>(ws, pl.tcnt);
            e = moe::launch_fused_bf16(a, st, stage_ev);
        }
    } else {
        moe::MxArgs a{};
        a.T = p->T; a.D = p->D; a.H = p->H; a.E = p->E; a.k = p->topk; a.P = P;
        a.x = static_cast<const uint8_t*>(x);
        a.xs = static_cast<const uint8_t*>(p->x_scale);
        a.w1 = static_cast<const uint8_t*>(w1);
        a.w1s = static_cast<const uint8_t*>(p->w1_scale);
        a.w2 = static_cast<const uint8_t*>(w2);
        a.w2s = static_cast<const uint8_t*>(p->w2_scale);
        a.wts = topk_weights;
        a.rv = rv;
        a.out = static_cast<uint16_t*>(out);
        a.w4 = p->dtype == MOE_FFN_MXFP4;
        if (m == MOE_FFN_SPLIT) {
            a.act = at<uint8_t>(ws, pl.act);
            a.act_s = at<uint8_t>(ws, pl.act_s);
            a.ypair = at<uint16_t>(ws, pl.ypair);
            a.mtiles = at<int32_t>(ws, pl.mtiles);
            e = moe::launch_split_mx(a, st, stage_ev);
        } else {
            a.acc32 = at<float>(ws, pl.acc32);
            a.tcnt = at<int32_t>(ws, pl.tcnt);
            e = moe::launch_fused_mx(a, st, stage_ev);
        }
    }
    return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_EHIP;
}
}  // namespace
