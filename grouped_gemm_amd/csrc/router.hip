// Router: logits [T, E] -> each token's top-k experts and routing weights.
//
// The pass starts from each token's top-k experts with normalized routing
// weights ("Prime Flash MoE", section 1 "The computation"): softmax over
// the E logits, the k most probable experts (most probable first, ties to
// the lower id), their probabilities renormalized to sum to 1. Softmax is
// strictly increasing in the logit, so the selection compares the fp32
// logits themselves (exact: the ids do not depend on how exp rounds), and
// the normalizer cancels: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over
// the k picks, l_0 the largest logit.
//
// G lanes serve one token (64/G tokens per wave), each lane holding V of
// its logits (expert gl + G*i). Each (logit, id) becomes one 64-bit key
// whose unsigned order is the router's order (the logit's bits made
// order-preserving above, the complemented id below), so a comparison is
// one 64-bit compare. Every lane keeps its best remaining key; round r
// takes the group's maximum (log2 G cross-lane steps, DPP within a row of
// 16 lanes) and the lane that held it moves on to its best key below it.
// Pick r is kept by lane r % G of the group. Rows of more than 2048
// experts (V > 32 keys would not fit in registers) use a scan of the
// lane's logits per round instead.
//
// Fused with the route step's first pass (the per-segment expert
// histogram): with COUNT, workgroup s handles the pairs [s*seg, (s+1)*seg)
// of p = t*k + j, writes their ids and weights, and counts them in LDS;
// tokens that straddle two segments are selected by both workgroups (the
// result is the same) and each writes only its own pairs.
#include <cfloat>
#include <climits>

#include "common.h"

namespace moe {

namespace {

struct Pick {
    float v;
    int id;
};

// 64-bit router keys: unsigned order = router order. The logit's bits are
// made order-preserving (negative: all bits flipped; positive: sign bit
// set) after folding -0 into +0 so that the two compare equal; a NaN gets
// the lowest logit rank. The low word is ~id (lower id = larger).
// Key 0 is below every real key and stands for "no candidate".
__device__ __forceinline__ uint64_t router_key(float v, int id) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    ord = v == v ? ord : 0u;
    return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~id);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t ord = static_cast<uint32_t>(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord ^ 0x80000000u) : ~ord);
}
__device__ __forceinline__ int key_id(uint64_t key) { return ~static_cast<int>(static_cast<uint32_t>(key)); }

// Cross-lane moves for the group reductions. Within a row of 16 lanes:
// DPP quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror (after
// each step every lane holds the reduction of its 2, 4, 8, 16 lanes);
// across rows: lane xor 16 and 32.
template <int STEP>
__device__ __forceinline__ int lane_move(int x) {
    if constexpr (STEP == 0) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
    else if constexpr (STEP == 1) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
    else if constexpr (STEP == 2) return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
    else if constexpr (STEP == 3) return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);
    else return __shfl_xor(x, STEP == 4 ? 16 : 32, 64);
}
template <int STEP>
__device__ __forceinline__ uint64_t lane_move64(uint64_t k) {
    const uint32_t lo = static_cast<uint32_t>(lane_move<STEP>(static_cast<int>(static_cast<uint32_t>(k))));
    const uint32_t hi = static_cast<uint32_t>(lane_move<STEP>(static_cast<int>(static_cast<uint32_t>(k >> 32))));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <int G, int STEP = 0>
__device__ __forceinline__ uint64_t group_max_key(uint64_t k) {
    if constexpr ((1 << STEP) < G) {
        const uint64_t o = lane_move64<STEP>(k);
        return group_max_key<G, STEP + 1>(o > k ? o : k);
    } else {
        return k;
    }
}
template <int G, int STEP = 0>
__device__ __forceinline__ float group_sum(float s) {
    if constexpr ((1 << STEP) < G) {
        return group_sum<G, STEP + 1>(s + __int_as_float(lane_move<STEP>(__float_as_int(s))));
    } else {
        return s;
    }
}

constexpr int kRouterThreads = 256;
constexpr int kNone = INT_MAX;  // id of "no candidate" (after every real id)

// Pick slots a lane keeps: picks r = G*i + gl for k <= 64.
template <int G, int V>
constexpr int router_slots() { return V < 64 / G ? V : 64 / G; }

// Select token t's top-k into the group's lanes: pick r lands in slot r / G
// of lane r % G. Returns the largest logit (pick 0). Lanes of a group whose
// token is past T compute on placeholders and store nothing. Key path
// (V <= 32 logits per lane).
template <int G, int V>
__device__ __forceinline__ float select_topk_keys(const float* __restrict__ row, bool live, int E, int k, int gl,
                                                  Pick (&mine)[router_slots<G, V>()]) {
    constexpr int NS = router_slots<G, V>();
    // every lane loads all V logits (clamped addresses), and the empty asm
    // makes each value needed unconditionally: the compiler would otherwise
    // move each load under its lane condition and wait for it there, one
    // memory latency per load
    float x[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = gl + G * i;
        x[i] = row[e < E ? e : E - 1];
    }
#pragma unroll
    for (int i = 0; i < V; ++i) asm volatile("" : "+v"(x[i]));
    uint64_t key[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = gl + G * i;
        key[i] = (live & (e < E)) ? router_key(x[i], e) : 0ull;
    }
    uint64_t cand = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) cand = key[i] > cand ? key[i] : cand;
    uint64_t slot[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) slot[i] = 0;
    uint64_t top = 0;
    for (int r = 0; r < k; ++r) {
        const uint64_t w = group_max_key<G>(cand);
        top = r == 0 ? w : top;
        const bool keeper = r % G == gl;
#pragma unroll
        for (int i = 0; i < NS; ++i) slot[i] = (keeper & (r / G == i)) ? w : slot[i];
        // the lane whose key was taken moves on to its best key below it
        uint64_t next = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) next = ((key[i] < w) & (key[i] > next)) ? key[i] : next;
        cand = cand == w ? next : cand;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
        mine[i] = slot[i] ? Pick{key_logit(slot[i]), key_id(slot[i])} : Pick{-INFINITY, kNone};
    return key_logit(top);
}

// Both paths order exactly like the key: a NaN logit after every other
// (NaNs by id), -0 equal to +0.
//
// Scan path (E > 2048, too many keys for registers): round r rescans the
// lane's logits (cache hits after the first round) for its best key below
// round r-1's pick, then takes the group's maximum.
template <int G, int V>
__device__ __forceinline__ float select_topk_scan(const float* __restrict__ row, bool live, int E, int k, int gl,
                                                  Pick (&mine)[router_slots<G, V>()]) {
    constexpr int NS = router_slots<G, V>();
    uint64_t slot[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) slot[i] = 0;
    uint64_t top = 0, w = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int i0 = 0; i0 < V; i0 += 8) {
            float x[8];  // eight loads in flight at a time (pinned as in select_topk_keys)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int e = gl + G * (i0 + j);
                x[j] = row[e < E ? e : E - 1];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(x[j]));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int e = gl + G * (i0 + j);
                const uint64_t key = (live & (e < E)) ? router_key(x[j], e) : 0ull;
                best = ((key < w) & (key > best)) ? key : best;
            }
        }
        w = group_max_key<G>(best);
        top = r == 0 ? w : top;
        const bool keeper = r % G == gl;
#pragma unroll
        for (int i = 0; i < NS; ++i) slot[i] = (keeper & (r / G == i)) ? w : slot[i];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
        mine[i] = slot[i] ? Pick{key_logit(slot[i]), key_id(slot[i])} : Pick{-INFINITY, kNone};
    return key_logit(top);
}

template <int G, int V>
__device__ __forceinline__ float select_topk(const float* __restrict__ row, bool live, int E, int k, int gl,
                                             Pick (&mine)[router_slots<G, V>()]) {
    if constexpr (V <= 32) return select_topk_keys<G, V>(row, live, E, k, gl, mine);
    else return select_topk_scan<G, V>(row, live, E, k, gl, mine);
}

// Weights of the group's picks and their stores. Pick r of token t is pair
// t*k + r; only pairs in [p_lo, p_hi) are stored (and counted in `hist`).
template <int G, int V>
__device__ __forceinline__ void store_picks(const Pick (&mine)[router_slots<G, V>()], float top, int64_t t, int k,
                                            int gl, int64_t p_lo, int64_t p_hi, int32_t* __restrict__ ids,
                                            float* __restrict__ wts, int* hist) {
    constexpr int NS = router_slots<G, V>();
    float ex[NS];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int r = G * i + gl;
        ex[i] = r < k && mine[i].id != kNone ? expf(mine[i].v - top) : 0.0f;
        s += ex[i];
    }
    s = group_sum<G>(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int r = G * i + gl;
        const int64_t p = t * k + r;
        if (r < k && p >= p_lo && p < p_hi) {
            const bool ok = mine[i].id != kNone;
            ids[p] = ok ? mine[i].id : -1;
            wts[p] = ok ? ex[i] * inv : 0.0f;
            if (hist && ok) atomicAdd(&hist[mine[i].id], 1);
        }
    }
}

// Plain router: tokens [0, T), grid-stride over groups of 64/G * 4 tokens.
template <int G, int V>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                                int k, int32_t* __restrict__ ids,
                                                                float* __restrict__ wts) {
    constexpr int TPW = 64 / G;  // tokens per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, gl = lane % G;
    const int64_t per_block = static_cast<int64_t>(TPW) * (kRouterThreads / 64);
    for (int64_t t0 = blockIdx.x * per_block; t0 < T; t0 += static_cast<int64_t>(gridDim.x) * per_block) {
        const int64_t t = t0 + wave * TPW + lane / G;
        const bool live = t < T;
        Pick mine[router_slots<G, V>()];
        const float top = select_topk<G, V>(logits + (live ? t : 0) * E, live, E, k, gl, mine);
        if (live) store_picks<G, V>(mine, top, t, k, gl, 0, T * k, ids, wts, nullptr);
    }
}

// Router fused with the route step's segment histogram: workgroup s owns the
// pairs [s*seg, min(P, (s+1)*seg)) and writes seg_counts[e*S + s].
template <int G, int V>
__global__ __launch_bounds__(kRouterThreads) void router_count_kernel(const float* __restrict__ logits, int64_t T,
                                                                      int E, int k, int32_t* __restrict__ ids,
                                                                      float* __restrict__ wts, int S, int seg,
                                                                      int32_t* __restrict__ seg_counts) {
    extern __shared__ int hist[];
    constexpr int TPW = 64 / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, gl = lane % G;
    const int s = blockIdx.x;
    const int64_t P = T * k;
    for (int e = threadIdx.x; e < E; e += kRouterThreads) hist[e] = 0;
    __syncthreads();
    const int64_t p0 = static_cast<int64_t>(s) * seg;
    const int64_t p1 = p0 + seg < P ? p0 + seg : P;
    const int64_t t_first = p0 / k, t_end = (p1 + k - 1) / k;
    constexpr int64_t per_block = static_cast<int64_t>(TPW) * (kRouterThreads / 64);
    for (int64_t t0 = t_first; t0 < t_end; t0 += per_block) {
        const int64_t t = t0 + wave * TPW + lane / G;
        const bool live = t < t_end;
        Pick mine[router_slots<G, V>()];
        const float top = select_topk<G, V>(logits + (live ? t : 0) * E, live, E, k, gl, mine);
        if (live) store_picks<G, V>(mine, top, t, k, gl, p0, p1, ids, wts, hist);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouterThreads) seg_counts[static_cast<int64_t>(e) * S + s] = hist[e];
}

// G lanes per token and V logits per lane. Base shape: V = 16 while a
// wave's 64 lanes suffice (E <= 1024); a round then costs log2(G) lane
// steps plus a 16-key scan by the lane that moves on. With few tokens the
// waves are few and each round's dependent chain is the time, so the plain
// router trades keys per lane for lanes per token (down to 1 key) until the
// batch fills about 256 waves.
struct RouterShape {
    int G, V;
};
RouterShape router_shape(int E, int64_t T, bool widen) {
    int G = 1;
    while (G < 64 && G * 16 < E) G *= 2;
    int V = 1;
    while (G * V < E) V *= 2;
    while (widen && G < 64 && V > 1 && T * G < 64 * 256) {
        G *= 2;
        V /= 2;
    }
    return {G, V};
}

template <int G, int V>
hipError_t launch_router_gv(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts,
                            const RouteBuffers* count, hipStream_t st) {
    if (count) {
        const size_t lds = sizeof(int) * static_cast<size_t>(E);
        router_count_kernel<G, V><<<count->S, kRouterThreads, lds, st>>>(logits, T, E, k, ids, wts, count->S,
                                                                         count->seg, count->seg_counts);
    } else {
        const int64_t per_block = (64 / G) * (kRouterThreads / 64);
        int64_t grid = (T + per_block - 1) / per_block;
        if (grid > 256 * 64) grid = 256 * 64;
        router_kernel<G, V><<<static_cast<int>(grid), kRouterThreads, 0, st>>>(logits, T, E, k, ids, wts);
    }
    return hipGetLastError();
}

template <int G>
hipError_t launch_router_g(int V, const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts,
                           const RouteBuffers* count, hipStream_t st) {
    switch (V) {
        case 1: return launch_router_gv<G, 1>(logits, T, E, k, ids, wts, count, st);
        case 2: return launch_router_gv<G, 2>(logits, T, E, k, ids, wts, count, st);
        case 4: return launch_router_gv<G, 4>(logits, T, E, k, ids, wts, count, st);
        case 8: return launch_router_gv<G, 8>(logits, T, E, k, ids, wts, count, st);
        case 16: return launch_router_gv<G, 16>(logits, T, E, k, ids, wts, count, st);
        default: break;
    }
    if constexpr (G == 64) {
        switch (V) {
            case 32: return launch_router_gv<64, 32>(logits, T, E, k, ids, wts, count, st);
            case 64: return launch_router_gv<64, 64>(logits, T, E, k, ids, wts, count, st);
            case 128: return launch_router_gv<64, 128>(logits, T, E, k, ids, wts, count, st);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

// Dispatch on router_shape() (E <= 8192: G * V covers E).
hipError_t launch_router_any(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts,
                             const RouteBuffers* count, hipStream_t st) {
    const RouterShape sh = router_shape(E, T, count == nullptr);
    switch (sh.G) {
        case 1: return launch_router_g<1>(sh.V, logits, T, E, k, ids, wts, count, st);
        case 2: return launch_router_g<2>(sh.V, logits, T, E, k, ids, wts, count, st);
        case 4: return launch_router_g<4>(sh.V, logits, T, E, k, ids, wts, count, st);
        case 8: return launch_router_g<8>(sh.V, logits, T, E, k, ids, wts, count, st);
        case 16: return launch_router_g<16>(sh.V, logits, T, E, k, ids, wts, count, st);
        case 32: return launch_router_g<32>(sh.V, logits, T, E, k, ids, wts, count, st);
        case 64: return launch_router_g<64>(sh.V, logits, T, E, k, ids, wts, count, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_router(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts, hipStream_t st) {
    if (T == 0) return hipSuccess;
    return launch_router_any(logits, T, E, k, ids, wts, nullptr, st);
}

hipError_t launch_router_route(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts,
                               const RouteBuffers& b, hipStream_t st) {
    if (T == 0) return hipSuccess;
    if (!route_counts_separately(b)) {
        const hipError_t e = launch_router_any(logits, T, E, k, ids, wts, nullptr, st);
        if (e != hipSuccess) return e;
        return launch_route(b, st);
    }
    // the router writes the ids and the segment histogram; the route step
    // continues from the histogram
    const hipError_t e = launch_router_any(logits, T, E, k, ids, wts, &b, st);
    if (e != hipSuccess) return e;
    return launch_route_after_count(b, st);
}

}  // namespace moe
