// Route step: permute routed (token, expert) pairs by expert.
//
// The grouped GEMMs read the pairs of each expert as one contiguous group
// of rows ("Prime Flash MoE", section 1: the grouped-GEMM formulation with
// sorted rows and group offsets; section 8: routing and sorting). Here the
// pairs p = t*k + j are sorted stably by expert id with a counting sort
// (up to 256 pairs: route_wave does all of it in one wave; up to 16384
// pairs: route_small in one workgroup; otherwise):
//   1. route_count   : one workgroup per segment of `seg` pairs builds that
//                      segment's per-expert histogram in LDS.
//   2. route_scan    : one workgroup per expert turns its row of segment
//                      counts into an exclusive prefix and writes counts[e].
//   3. route_offsets : one workgroup scans counts into offsets[E+1] and the
//                      m-tile prefix sums for the GEMMs' tile heights.
//   4. route_scatter : one wave per segment walks its pairs in order, 64 at a
//                      time; lanes holding the same expert find each other
//                      with ballots over the bits of the id, so the rank of a
//                      pair among equal ids is the popcount of lower lanes in
//                      its group. The result does not depend on scheduling.
#include "common.h"

namespace moe {

namespace {

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Exclusive scan across a block of NW waves; `sh` holds NW ints of LDS.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int& total, int* sh) {
    const int incl = wave_incl_scan(v);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    int wbase = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        int t = sh[i];
        wbase += i < w ? t : 0;
        total += t;
    }
    __syncthreads();
    return wbase + incl - v;
}

// Extra blocks of a route kernel (blockIdx.x >= first) store zeros over n
// floats at p (n a multiple of 4): the fused pipeline's accumulator and its
// token counters are cleared alongside the route step, with no kernel of
// their own.
__device__ __forceinline__ void clear_blocks(float* p, int64_t n, int first) {
    float4* q = reinterpret_cast<float4*>(p);
    const int64_t n4 = n / 4, stride = static_cast<int64_t>(gridDim.x - first) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x - first) * blockDim.x + threadIdx.x; i < n4; i += stride)
        q[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// Blocks of `threads` that clear n floats at about four float4 stores per thread.
inline int clear_block_count(int64_t n, int threads) {
    if (n <= 0) return 0;
    const int64_t b = (n / 4 + 4 * threads - 1) / (4 * threads);
    return static_cast<int>(b < 2048 ? b : 2048);
}

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                          int E, int S, int seg,
                                                          int32_t* __restrict__ seg_counts) {
    extern __shared__ int32_t hist[];
    const int s = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    const int64_t p0 = static_cast<int64_t>(s) * seg;
    const int64_t p1 = p0 + seg < P ? p0 + seg : P;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
        int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) seg_counts[static_cast<int64_t>(e) * S + s] = hist[e];
}

// Exclusive prefix over segments for expert blockIdx.x, in place.
__global__ __launch_bounds__(256) void route_scan_kernel(int32_t* __restrict__ seg_counts, int S, int E,
                                                         int32_t* __restrict__ counts, float* clear,
                                                         int64_t clear_n) {
    if (static_cast<int>(blockIdx.x) >= E) {
        clear_blocks(clear, clear_n, E);
        return;
    }
    __shared__ int sh[4];
    int32_t* row = seg_counts + static_cast<int64_t>(blockIdx.x) * S;
    int carry = 0;
    for (int base = 0; base < S; base += 256 * 4) {
        int v[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int idx = base + threadIdx.x * 4 + i;
            v[i] = idx < S ? row[idx] : 0;
            local += v[i];
        }
        int total;
        int ex = block_excl_scan<4>(local, total, sh) + carry;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int idx = base + threadIdx.x * 4 + i;
            if (idx < S) row[idx] = ex;
            ex += v[i];
        }
        carry += total;
    }
    if (threadIdx.x == 0) counts[blockIdx.x] = carry;
}

// offsets[E+1] and, for each tile height BM in {16..256}, the prefix sums of
// ceil(counts/BM) (the m-tile index of each expert's first tile).
__global__ __launch_bounds__(1024) void route_offsets_kernel(const int32_t* __restrict__ counts,
                                                             int E, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tile_prefix) {
    __shared__ int sh[16];
    constexpr int PER = 8;  // experts per thread: E <= 8192
    const int e0 = threadIdx.x * PER;
    int c[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) c[i] = e0 + i < E ? counts[e0 + i] : 0;
    for (int b = -1; b < kNumTileHeights; ++b) {
        const int bm = 16 << (b < 0 ? 0 : b);
        int v[PER], local = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            v[i] = b < 0 ? c[i] : (c[i] + bm - 1) / bm;
            local += v[i];
        }
        int total;
        int ex = block_excl_scan<16>(local, total, sh);
        int32_t* dst = b < 0 ? offsets : tile_prefix + b * (E + 1);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (e0 + i < E) dst[e0 + i] = ex;
            ex += v[i];
        }
        if (threadIdx.x == 0) dst[E] = total;
    }
}

__global__ __launch_bounds__(64) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int S, int seg, int nbits,
    const int32_t* __restrict__ seg_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_to_pair, int32_t* __restrict__ pair_to_sorted) {
    extern __shared__ int32_t run[];
    const int s = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) run[e] = offsets[e] + seg_base[static_cast<int64_t>(e) * S + s];
    const int64_t valid_total = offsets[E];
    __syncthreads();
    const int64_t p0 = static_cast<int64_t>(s) * seg;
    const int64_t p1 = p0 + seg < P ? p0 + seg : P;
    // sorted positions past the valid pairs hold -1; this segment's index
    // range [p0, p1) takes its share of them.
    for (int64_t i = p0 + lane; i < p1; i += 64)
        if (i >= valid_total) sorted_to_pair[i] = -1;
    const uint64_t lower = (1ull << lane) - 1ull;
    for (int64_t base = p0; base < p1; base += 64) {
        const int64_t p = base + lane;
        const bool in = p < p1;
        const int e = in ? ids[p] : -1;
        const bool valid = in && e >= 0 && e < E;
        const int key = valid ? e : E;
        uint64_t same = ~0ull;
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (key >> b) & 1;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        const int rank = __popcll(same & lower);
        const int cnt = __popcll(same);
        const bool leader = (same >> lane) == 1ull;  // highest lane of its group
        int pos = valid ? run[e] + rank : 0;
        __syncthreads();
        if (valid && leader) run[e] += cnt;
        __syncthreads();
        if (valid && pos >= 0 && pos < P) {
            sorted_to_pair[pos] = static_cast<int32_t>(p);
            pair_to_sorted[p] = pos;
        } else if (in) {
            pair_to_sorted[p] = -1;
        }
    }
}

// The whole route step in one workgroup of 16 waves, for small problems
// (one launch instead of four). Wave w owns the contiguous pair segment
// [w*seg, (w+1)*seg): it counts its segment into its own LDS row cnt[w][.],
// one scan turns the rows into per-(wave, expert) start positions, and each
// wave then places its pairs in order with the same ballot ranking as
// route_scatter_kernel, so the result is the same stable order.
// The lanes of this wave whose key equals this lane's (keys < 2^nbits).
__device__ __forceinline__ uint64_t lanes_with_key(int key, int nbits) {
    uint64_t same = ~0ull;
    for (int bb = 0; bb < nbits; ++bb) {
        const bool bit = (key >> bb) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    return same;
}

// One wave routes a small batch (at most 256 pairs, 64 experts) with no
// workgroup barrier (measured: faster than one 1024-thread workgroup up to a
// few hundred pairs, slower beyond): lane e holds expert e for the prefix sums, and
// the histogram and the scatter walk the pairs 64 at a time with the same
// ballot ranks as route_scatter (one leader lane per expert per chunk
// updates that expert's counter, so no atomics are needed).
constexpr int kWaveMaxExperts = 64;
constexpr int64_t kWaveMaxPairs = 256;

__global__ __launch_bounds__(64) void route_wave_kernel(const int32_t* __restrict__ ids, int P, int E, int nbits,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ tile_prefix,
                                                        int32_t* __restrict__ sorted_to_pair,
                                                        int32_t* __restrict__ pair_to_sorted, float* clear,
                                                        int64_t clear_n) {
    if (blockIdx.x > 0) {
        clear_blocks(clear, clear_n, 1);
        return;
    }
    __shared__ int32_t run[kWaveMaxExperts + 1];  // [E] collects the dropped pairs
    const int lane = threadIdx.x;
    run[lane] = 0;
    if (lane == 0) run[kWaveMaxExperts] = 0;
    __builtin_amdgcn_wave_barrier();
    const uint64_t lower = (1ull << lane) - 1ull;
    // all of this lane's ids at once (one memory latency, not one per chunk)
    constexpr int NC = kWaveMaxPairs / 64;
    int myid[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) myid[c] = 64 * c + lane < P ? ids[64 * c + lane] : -1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int base = 64 * c;
        if (base >= P) break;
        const int e = myid[c];
        const bool valid = e >= 0 && e < E;
        const uint64_t same = lanes_with_key(valid ? e : E, nbits);
        if (valid && (same & lower) == 0) run[e] += __popcll(same);
        __builtin_amdgcn_wave_barrier();
    }
    const int n_e = lane < E ? run[lane] : 0;  // pairs of expert `lane`
    int valid_total = 0;
    for (int b = -1; b < kNumTileHeights; ++b) {
        const int bm = 16 << (b < 0 ? 0 : b);
        const int v = b < 0 ? n_e : (n_e + bm - 1) / bm;
        const int incl = wave_incl_scan(v);
        const int total = __shfl(incl, 63, 64);
        int32_t* dst = b < 0 ? offsets : tile_prefix + b * (E + 1);
        if (lane < E) dst[lane] = incl - v;
        if (lane == 0) dst[E] = total;
        if (b < 0) {
            valid_total = total;
            if (lane < E) {
                counts[lane] = n_e;
                run[lane] = incl - v;  // next free sorted row of expert `lane`
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int base = 64 * c;
        if (base >= P) break;
        const int p = base + lane;
        const bool in = p < P;
        const int e = myid[c];
        const bool valid = e >= 0 && e < E;
        const uint64_t same = lanes_with_key(valid ? e : E, nbits);
        const int pos = valid ? run[e] + __popcll(same & lower) : -1;
        __builtin_amdgcn_wave_barrier();
        if (valid && (same & lower) == 0) run[e] += __popcll(same);
        __builtin_amdgcn_wave_barrier();
        if (in) pair_to_sorted[p] = pos;
        if (valid && pos < P) sorted_to_pair[pos] = p;
    }
    for (int i = valid_total + lane; i < P; i += 64) sorted_to_pair[i] = -1;
}

constexpr int kSmallWaves = 16;
constexpr int kSmallMaxExperts = 1024;
constexpr int64_t kSmallMaxPairs = 16384;

__global__ __launch_bounds__(1024) void route_small_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                           int nbits, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tile_prefix,
                                                           int32_t* __restrict__ sorted_to_pair,
                                                           int32_t* __restrict__ pair_to_sorted, float* clear,
                                                           int64_t clear_n) {
    if (blockIdx.x > 0) {
        clear_blocks(clear, clear_n, 1);
        return;
    }
    extern __shared__ int32_t cnt[];  // [kSmallWaves][E]
    __shared__ int sh[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kSmallWaves * E; i += 1024) cnt[i] = 0;
    __syncthreads();
    const int64_t seg = (P + kSmallWaves - 1) / kSmallWaves;
    const int64_t p0 = w * seg, p1 = p0 + seg < P ? p0 + seg : P;
    for (int64_t p = p0 + lane; p < p1; p += 64) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[w * E + e], 1);
    }
    __syncthreads();
    // per-expert totals -> offsets and tile prefix sums; thread t owns expert t, so
    // the scan in thread order is the scan in expert order
    constexpr int PER = kSmallMaxExperts / 1024;
    static_assert(PER == 1, "one expert per thread");
    __shared__ int s_valid_total;
    int c[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + 1024 * i;
        int tot = 0;
        if (e < E)
            for (int v = 0; v < kSmallWaves; ++v) tot += cnt[v * E + e];
        c[i] = tot;
    }
    for (int b = -1; b < kNumTileHeights; ++b) {
        const int bm = 16 << (b < 0 ? 0 : b);
        int v[PER], local = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            v[i] = b < 0 ? c[i] : (c[i] + bm - 1) / bm;
            local += v[i];
        }
        int total;
        int ex = block_excl_scan<16>(local, total, sh);
        int32_t* dst = b < 0 ? offsets : tile_prefix + b * (E + 1);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + 1024 * i;
            if (e < E) dst[e] = ex;
            ex += v[i];
        }
        if (tid == 0) dst[E] = total;
        if (b < 0) {
            if (tid == 0) s_valid_total = total;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int e = tid + 1024 * i;
                if (e < E) {
                    counts[e] = c[i];
                    // start of each wave's pairs of expert e
                    int run = dst[e];
                    for (int v2 = 0; v2 < kSmallWaves; ++v2) {
                        const int t2 = cnt[v2 * E + e];
                        cnt[v2 * E + e] = run;
                        run += t2;
                    }
                }
            }
        }
        __syncthreads();
    }
    const int64_t valid_total = s_valid_total;
    for (int64_t i = tid; i < P; i += 1024)
        if (i >= valid_total) sorted_to_pair[i] = -1;
    const uint64_t lower = (1ull << lane) - 1ull;
    int32_t* run = cnt + w * E;
    for (int64_t base = p0; base < p1; base += 64) {
        const int64_t p = base + lane;
        const bool in = p < p1;
        const int e = in ? ids[p] : -1;
        const bool valid = in && e >= 0 && e < E;
        const int key = valid ? e : E;
        uint64_t same = ~0ull;
        for (int bb = 0; bb < nbits; ++bb) {
            const bool bit = (key >> bb) & 1;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        const int rank = __popcll(same & lower);
        const int n = __popcll(same);
        const bool leader = (same >> lane) == 1ull;
        const int pos = valid ? run[e] + rank : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid && leader) run[e] += n;
        __builtin_amdgcn_wave_barrier();
        if (valid && pos >= 0 && pos < P) {
            sorted_to_pair[pos] = static_cast<int32_t>(p);
            pair_to_sorted[p] = pos;
        } else if (in) {
            pair_to_sorted[p] = -1;
        }
    }
}

}  // namespace

bool route_counts_separately(const RouteBuffers& b) {
    return !(b.P <= kWaveMaxPairs && b.E <= kWaveMaxExperts) && !(b.P <= kSmallMaxPairs && b.E <= kSmallMaxExperts);
}

// Steps 2..4 of the multi-kernel route, from the segment histogram.
hipError_t launch_route_after_count(const RouteBuffers& b, hipStream_t st) {
    const size_t lds = sizeof(int32_t) * static_cast<size_t>(b.E);
    int nbits = 0;
    while ((1 << nbits) <= b.E) ++nbits;  // enough bits for ids 0..E (E = sentinel)
    route_scan_kernel<<<b.E + clear_block_count(b.clear_n, 256), 256, 0, st>>>(b.seg_counts, b.S, b.E, b.counts,
                                                                              b.clear, b.clear_n);
    route_offsets_kernel<<<1, 1024, 0, st>>>(b.counts, b.E, b.offsets, b.tile_prefix);
    if (b.S > 0) {
        route_scatter_kernel<<<b.S, 64, lds, st>>>(b.ids, b.P, b.E, b.S, b.seg, nbits, b.seg_counts,
                                                   b.offsets, b.sorted_to_pair, b.pair_to_sorted);
    }
    return hipGetLastError();
}

hipError_t launch_route(const RouteBuffers& b, hipStream_t st) {
    if (b.P <= kWaveMaxPairs && b.E <= kWaveMaxExperts) {
        int nbits = 0;
        while ((1 << nbits) <= b.E) ++nbits;
        route_wave_kernel<<<1 + clear_block_count(b.clear_n, 64), 64, 0, st>>>(
            b.ids, static_cast<int>(b.P), b.E, nbits, b.counts, b.offsets, b.tile_prefix, b.sorted_to_pair,
            b.pair_to_sorted, b.clear, b.clear_n);
        return hipGetLastError();
    }
    if (b.P <= kSmallMaxPairs && b.E <= kSmallMaxExperts) {
        int nbits = 0;
        while ((1 << nbits) <= b.E) ++nbits;
        const size_t lds = sizeof(int32_t) * kSmallWaves * static_cast<size_t>(b.E);
        route_small_kernel<<<1 + clear_block_count(b.clear_n, 1024), 1024, lds, st>>>(
            b.ids, b.P, b.E, nbits, b.counts, b.offsets, b.tile_prefix, b.sorted_to_pair, b.pair_to_sorted,
            b.clear, b.clear_n);
        return hipGetLastError();
    }
    if (b.S > 0) {
        const size_t lds = sizeof(int32_t) * static_cast<size_t>(b.E);
        route_count_kernel<<<b.S, 256, lds, st>>>(b.ids, b.P, b.E, b.S, b.seg, b.seg_counts);
    }
    return launch_route_after_count(b, st);
}

}  // namespace moe
