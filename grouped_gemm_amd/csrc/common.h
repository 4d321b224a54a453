// Internal declarations shared by the HIP translation units of libmoe_ffn.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
// 16-byte register chunk. A native vector type (not HIP's uint4 struct) so
// arrays of it stay in VGPRs instead of being copied through private memory.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// m-tile heights for which the route step writes tile prefix sums.
constexpr int kNumTileHeights = 5;  // 16, 32, 64, 128, 256
__host__ __device__ constexpr int tile_height_index(int bm) {
    return bm == 16 ? 0 : bm == 32 ? 1 : bm == 64 ? 2 : bm == 128 ? 3 : 4;
}

// bf16 <-> fp32. fp32 -> bf16 rounds to nearest even; gfx950 converts in
// hardware (v_cvt_pk_bf16_f32, two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Activation variant of the GEMM1 epilogues ("Porting Block-Scaled GEMM
// Kernels from Blackwell to Rubin", section 5.3; "GC-MoE on SM120", section
// 4.8): gate and up scaled by the expert's global scale alpha[e] and, with
// wba, by the pair's routing weight (which then does not scale y); kind 1
// clamps the gate from above and up on both sides at `limit`. All zero is
// the plain SwiGLU, which the kernels keep on their own code path.
struct ActVariant {
    int32_t kind;         // 0 SwiGLU, 1 clamped SwiGLU
    float limit;
    const float* alpha;   // [E] or null (1.0)
    int32_t wba;          // routing weight before the activation
    __host__ __device__ bool on() const { return kind != 0 || alpha != nullptr || wba != 0; }
};

// act of one (gate, up) pair under the variant; s = alpha[e] * (wba ? w : 1)
__device__ __forceinline__ float act_variant(float g, float u, float s, int kind, float limit) {
    g *= s;
    u *= s;
    if (kind == 1) {
        g = fminf(g, limit);
        u = fmaxf(fminf(u, limit), -limit);
    }
    return g / (1.0f + __expf(-g)) * u;
}

// Device view of the route step's outputs inside the workspace.
struct RouteView {
    const int32_t* counts;        // [E]
    const int32_t* offsets;       // [E+1]
    const int32_t* tile_prefix;   // [kNumTileHeights][E+1]
    const int32_t* sorted_to_pair;// [P]
    const int32_t* pair_to_sorted;// [P]
};

// Which expert / rows an m-tile covers. Returns false past the last tile.
struct MTile {
    int expert;
    int row0;   // first sorted row
    int rows;   // valid rows (1..BM)
    int m0;     // row offset inside the expert
};

template <int BM>
__device__ __forceinline__ bool find_mtile(const RouteView& rv, int E, int g, MTile& t) {
    const int32_t* tp = rv.tile_prefix + tile_height_index(BM) * (E + 1);
    if (g >= tp[E]) return false;
    int lo = 0, hi = E;  // tp[lo] <= g < tp[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tp[mid] <= g) lo = mid; else hi = mid;
    }
    t.expert = lo;
    t.m0 = (g - tp[lo]) * BM;
    int c = rv.counts[lo];
    t.rows = c - t.m0 < BM ? c - t.m0 : BM;
    t.row0 = rv.offsets[lo] + t.m0;
    return true;
}

// A pair index read back from the route maps, clamped into [0, P) so that a
// wrong map can only give wrong numbers, never an out-of-bounds access.
__device__ __forceinline__ int clamp_pair(int p, int64_t P) {
    return p < 0 ? 0 : (p >= P ? static_cast<int>(P - 1) : p);
}

// Compute units of the current device (queried once).
int device_cu_count();

// ---- launchers (each returns hipGetLastError() after enqueueing) ----

inline void record(hipEvent_t* ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

struct RouteBuffers {
    const int32_t* ids;
    int64_t P;
    int32_t E;
    int32_t S, seg;           // segments and pairs per segment
    int32_t* seg_counts;      // [E][S]
    int32_t* counts;
    int32_t* offsets;
    int32_t* tile_prefix;
    int32_t* sorted_to_pair;
    int32_t* pair_to_sorted;
    float* clear = nullptr;   // clear_n floats (a multiple of 4) the route step sets to zero, or null
    int64_t clear_n = 0;
};
hipError_t launch_route(const RouteBuffers& b, hipStream_t s);
// True when launch_route takes its multi-kernel path (segment histogram,
// scan, offsets, scatter); launch_route_after_count runs all but the first.
bool route_counts_separately(const RouteBuffers& b);
hipError_t launch_route_after_count(const RouteBuffers& b, hipStream_t s);
// Router: logits fp32 [T, E] -> ids int32 [T, k], weights fp32 [T, k].
hipError_t launch_router(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts, hipStream_t s);
// Router, then the route step on its ids (b.ids must be `ids`); on the
// multi-kernel path the router also builds the segment histogram.
hipError_t launch_router_route(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts,
                               const RouteBuffers& b, hipStream_t s);

struct Bf16Args {
    int32_t T, D, H, E, k;
    int64_t P;
    const uint16_t* x;
    const uint16_t* w1;
    const uint16_t* w2;
    const float* wts;
    RouteView rv;
    uint16_t* act;     // [P, H]   split only
    uint16_t* ypair;   // [P, D]   split only: weighted expert outputs in pair order
    int32_t* mtiles;   // split only: big_gemm_workspace_bytes for the prefill GEMMs
    float* acc32;      // [T, D]   fused only
    int32_t* tcnt;     // [T]      fused only: partial rows added per token (zero at entry)
    uint16_t* out;     // [T, D]
    const uint16_t* shared_y;  // [T, D] or null: a shared expert's output, added to each token's sum
    ActVariant av;             // zero: the plain SwiGLU
};
// `ev` (nullable) points at 3 events recorded after each of the launcher's
// three kernels.
hipError_t launch_split_bf16(const Bf16Args& a, hipStream_t s, hipEvent_t* ev);
// The split pipeline's two grouped GEMMs alone (ypair filled, no combine);
// `ev` (nullable) gets 2 events, after each GEMM.
hipError_t launch_gemms_bf16(const Bf16Args& a, hipStream_t s, hipEvent_t* ev);
// Route maps of T tokens each with one slot on expert 0 (the shared
// expert as a grouped GEMM of one group): counts, offsets, tile prefix
// sums, the identity maps, and `ones` [T] = 1.0f as the routing weights.
hipError_t launch_identity_route(int64_t T, int32_t* counts, int32_t* offsets, int32_t* tile_prefix,
                                 int32_t* sorted_to_pair, int32_t* pair_to_sorted, float* ones, hipStream_t s);
// Decode-shaped GEMM1 / GEMM2 (weights streamed on the MFMA's wide side).
// Whether the bf16 split pipeline runs the decode-shaped GEMMs (host only).
bool bf16_uses_decode_kernels(const Bf16Args& a);
// Token rows per tile of the bf16 prefill GEMMs (128 or 256).
int big_gemm_tile_rows(const Bf16Args& a);
// Name of the decode kernel launch_skinny_gemm1 (gemm1) / 2 runs for `a`.
const char* decode_kernel_name(const Bf16Args& a, bool gemm1);
hipError_t launch_skinny_gemm1(const Bf16Args& a, hipStream_t s);
hipError_t launch_skinny_gemm2(const Bf16Args& a, hipStream_t s);
// Prefill-shaped GEMM1 / GEMM2 (256-feature tiles, 128 or 256 token rows).
bool big_gemm_supported(const Bf16Args& a);
// Entries (int4 each) the m-tile table needs for P routed pairs and E experts.
int64_t big_gemm_mtile_capacity(int64_t P, int E);
// Workspace bytes at `mtiles` the prefill GEMMs use: the m-tile table, then
// a 1 MB sink for the result stores of rows past an expert's count.
int64_t big_gemm_workspace_bytes(int64_t P, int E);
// Entries past P that sorted_to_pair in the workspace must hold (a tile's
// row-map window may run past the last routed row; the extra entries are
// read and clamped, never written).
constexpr int64_t kRowMapPad = 256;
hipError_t launch_big_gemm(const Bf16Args& a, bool gemm1, hipStream_t s);
// Whether the decode-shaped kernels suit a batch of T tokens with k routes
// each over E experts. They take 32-row m-tiles and about one block per CU
// (the row groups per block are chosen for that), so every expert past 32
// rows adds a second m-tile, and the blocks past one per CU run as a second
// round. They are used while, with routes spread uniformly (each token's k
// experts distinct), fewer than 0.5 experts are expected past 32 rows:
// E * P(Binomial(T, k/E) > 32) < 0.5. Measured against the prefill or
// generic kernels: 21% faster at 20-24 rows per expert with 32 experts,
// 19% at 18 with 64; 20-26% slower at 24 with 64 or 128 experts and at 32
// with 32 or 64.
bool decode_kernels_fit(int64_t T, int k, int E);
hipError_t launch_fused_bf16(const Bf16Args& a, hipStream_t s, hipEvent_t* ev);
// The fused pass on the decode kernels' rings (32-row m-tiles, 256-wide
// slices of the intermediate dimension); D and H multiples of 256, no
// activation variant. Adds into a.acc32, which must hold zeros.
bool fused_decode_supported(const Bf16Args& a);
// Whether AUTO runs a bf16 pass (no activation variant) on the fused pipeline.
bool fused_preferred(int64_t T, int D, int H, int E, int k);
bool mx_fused_preferred(int64_t T, int D, int H, int E, int k);
hipError_t launch_fused_decode(const Bf16Args& a, hipStream_t s);

struct MxArgs {
    int32_t T, D, H, E, k;
    int64_t P;
    const uint8_t* x;   const uint8_t* xs;
    const uint8_t* w1;  const uint8_t* w1s;
    const uint8_t* w2;  const uint8_t* w2s;
    const float* wts;
    RouteView rv;
    uint8_t* act;       // [P, H] e4m3 codes
    uint8_t* act_s;     // [P, H/32] e8m0
    uint16_t* ypair;    // [P, D]
    uint16_t* out;      // [T, D]
    int32_t* mtiles;    // big_gemm_workspace_bytes for the prefill GEMMs
    float* acc32;       // [T, D] fused only
    int32_t* tcnt;      // [T]    fused only: partial rows added per token (zero at entry)
    bool w4;            // MXFP4 weights: w1, w2 packed e2m1 [E, 2H, D/2], [E, D, H/2]
};
hipError_t launch_split_mx(const MxArgs& a, hipStream_t s, hipEvent_t* ev);
// Decode-shaped MX GEMM1 / GEMM2, e2m1 or e4m3 weights (streamed on the MFMA's row side).
bool skinny_mx_supported(const MxArgs& a);
hipError_t launch_skinny_mx(const MxArgs& a, bool gemm1, hipStream_t s);
// Name of the MX decode kernel launch_skinny_mx runs for `a` (gemm1: GEMM1).
const char* mx_decode_kernel_name(const MxArgs& a, bool gemm1);
// MXQ4: fp32 [rows, K] -> packed e2m1 codes [rows, K/2] + e8m0 [rows, K/32].
hipError_t launch_mx4_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t s);
// Fused MX pipeline: GEMM1, SwiGLU and the act requantization in LDS, then a
// split-K down projection over each 64-wide H slice into acc32 (fp32
// atomics), then the conversion to bf16; `ev` (nullable) gets 3 events.
hipError_t launch_fused_mx(const MxArgs& a, hipStream_t s, hipEvent_t* ev);
// The fused MX pass on the decode kernels' rings (mx_fused_dma_kernel): e4m3
// weights, D a multiple of 512, H of 128. Adds into a.acc32 (zero on entry)
// and converts each token's row itself (a.tcnt zero on entry).
bool mx_fused_dma_supported(const MxArgs& a);
hipError_t launch_mx_fused_dma(const MxArgs& a, hipStream_t s);
// Prefill-shaped MX GEMM1 / GEMM2 (the bf16 prefill kernels' ring on the scaled MFMA).
bool big_mx_supported(const MxArgs& a);
hipError_t launch_big_mx(const MxArgs& a, bool gemm1, hipStream_t s);

hipError_t launch_combine(const uint16_t* ypair, const int32_t* pair_to_sorted, int32_t T, int32_t k,
                          int32_t D, uint16_t* out, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
hipError_t launch_mx_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);

}  // namespace moe
