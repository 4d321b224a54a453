// The fused pass for few rows per expert: one kernel for GEMM1, SwiGLU and
// GEMM2 on the decode kernels' DMA rings.
//
// The fused pipeline of "Prime Flash MoE" (section 2, "Trick 2": the down
// projection split over slices of the intermediate dimension, each slice's
// partial added into a global accumulator). A block owns one 32-row m-tile
// and a slice of BH act columns h0 .. h0 + BH - 1:
//   phase 1 streams the slice's gate and up rows of W1 in k-major order, as
//     dma_kmajor_kernel does: per 256-value K chunk, the chunk's token rows
//     once and then the slice's BH/32 row groups (32 act columns: their gate
//     and up rows, interleaved 8 + 8 per 16-row block), each wave owning 16
//     rows over the whole chunk; after the last chunk silu(gate) * up goes
//     into an act tile in LDS as bf16;
//   phase 2 streams the slice's columns of every W2 row (groups of R2 output
//     features, one 32 KB stage each) against that act tile and adds
//     weight * partial into acc32 [T, D] (fp32) with atomics.
// The weight waves (0-1) run one continuous ring through both phases, so
// phase 2's first W2 stages are in flight while phase 1 drains; the token
// waves (2-3) fetch the token chunks in phase 1 and, in phase 2, where they
// move nothing, do all of the down projection: each owns half of a stage's
// output rows over the whole slice and adds its partials straight from the
// MFMA results, so the weight waves' vmcnt budgets count their DMAs alone
// and a stage needs one barrier. A slice is 64, 128 or 256 act columns (the
// pages' CPC knob: two 128-wide column groups per block halve the number of
// partial rows to reduce; 64 doubles the blocks for small batches). A
// token's row is converted to bf16 by the block that adds its last partial
// (per-token counters), so the pass is two launches: the route step (whose
// extra blocks clear the accumulator) and this kernel. The blocks of one
// m-tile's slices are consecutive in the grid, so they run side by side and
// the m-tile's token rows come from L2.
#include <algorithm>
#include <cmath>

#include "dma_ring.h"
#include "mxq.h"

namespace moe {

namespace {

template <int BH>
struct FusedTile {
    static constexpr int G1 = BH / 32;       // GEMM1 row groups per slice
    static constexpr int RB2 = 2 * BH;       // bytes of a W2 row per stage (the slice)
    static constexpr int R2 = 32768 / RB2;   // W2 rows per stage (32 KB)
    static constexpr int CPR2 = RB2 / 16;    // 16-byte chunks per W2 (and act) row
    static constexpr int RPI2 = 1024 / RB2;  // W2 rows per DMA instruction
    static constexpr int KS2 = BH / 16;      // 32 x 32 x 16 MFMA k-steps over the slice
    static constexpr int FB2 = R2 / 64;      // 32-feature blocks of a token wave per stage
    static constexpr int ACT = 32 * RB2;     // act tile [32 tokens][BH] bf16
    static_assert(BH == 64 || BH == 128 || BH == 256, "64-, 128- or 256-wide slices");
};





// What the fused kernels' completion steps need of a pass.
struct FusedOut {
    int T, D, k;
    const int32_t* pair_to_sorted;
    float* acc32;               // [T, D] fp32, the partial rows' sum
    int32_t* tcnt;              // [T] partial rows added per token
    uint16_t* out;              // [T, D] bf16
    const uint16_t* shared_y;   // [T, D] bf16 or null: a shared expert's rows
};

// Tokens none of whose routes reach an expert get no partial rows: their
// output is the shared expert's row, or zeros. One wave of block b takes
// tokens b, b + gridDim.x, ... (k <= 64: a lane per route).
__device__ void fused_write_unrouted(const FusedOut& o, int lane) {
    for (int t = blockIdx.x; t < o.T; t += gridDim.x) {
        const bool routed = lane < o.k && o.pair_to_sorted[static_cast<int64_t>(t) * o.k + lane] >= 0;
        if (__ballot(routed)) continue;
        const int64_t row = static_cast<int64_t>(t) * o.D;
        for (int c = lane; c < o.D / 8; c += 64)
            *reinterpret_cast<u32x4_t*>(o.out + row + 8 * c) =
                o.shared_y ? *reinterpret_cast<const u32x4_t*>(o.shared_y + row + 8 * c) : u32x4_t{0, 0, 0, 0};
    }
}

// The partial rows a token needs, H / BH per routed pair (prologue of the
// fused kernels, by the threads of the m-tile's rows): unconditional loads
// (indexes clamped to the token's k pairs), so they go out together with
// the other per-row loads.
__device__ __forceinline__ int fused_target(const FusedOut& o, int token, int nslices) {
    const int64_t t0 = static_cast<int64_t>(token) * o.k;
    int nv = 0;
    for (int j0 = 0; j0 < o.k; j0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = o.pair_to_sorted[t0 + (j0 + u < o.k ? j0 + u : o.k - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) nv += (j0 + u < o.k && v[u] >= 0) ? 1 : 0;
    }
    return nv * nslices;
}

// The end of a fused block. A token's row is complete once each of its
// routed pairs has had all H / BH slices' partials added. The token waves
// (the ones that issued the adds) count this block's partial rows per token
// once their adds are acknowledged (the adds and the counts are
// device-scope atomics, performed where every XCD sees them); the block
// whose count completes a row reads it back with device-scope loads and
// converts it to bf16, plus the shared expert's row, into `out`. No block
// waits on another, and no cache is written back or invalidated. sDone has
// 33 entries; sDone[32] must be zero on entry.
__device__ __forceinline__ void fused_finish(const FusedOut& o, int rows, bool adder, int wave, int lane,
                                             const int* sTok, const int* sTgt, int* sDone) {
    if (adder) wait_vm<0>();
    __syncthreads();
    if (wave == 2 && lane < rows) {
        const int t = sTok[lane];
        if (atomicAdd(o.tcnt + t, 1) + 1 == sTgt[lane]) sDone[atomicAdd(&sDone[32], 1)] = t;
    }
    __syncthreads();
    const int ndone = sDone[32];
    // The completed rows, four floats per item and U items per thread in
    // flight: the loads (device scope, so they bypass caches that may hold
    // stale lines) go out together from clamped, always valid indexes, and
    // only the stores are predicated.
    constexpr int U = 16;
    const int per = o.D / 4, total = ndone * per;
    for (int b0 = 0; b0 < total; b0 += U * kThreads) {
        uint64_t lo[U], hi[U];
        uint2 sy[U];
        int64_t off[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int idx = b0 + u * kThreads + static_cast<int>(threadIdx.x);
            idx = idx < total ? idx : total - 1;
            const int i = idx / per;
            off[u] = static_cast<int64_t>(sDone[i]) * o.D + 4 * (idx - i * per);
            const uint64_t* src = reinterpret_cast<const uint64_t*>(o.acc32 + off[u]);
            lo[u] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            hi[u] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sy[u] = o.shared_y ? *reinterpret_cast<const uint2*>(o.shared_y + off[u]) : uint2{0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (b0 + u * kThreads + static_cast<int>(threadIdx.x) >= total) continue;
            const float v0 = __uint_as_float(static_cast<uint32_t>(lo[u])) + bf16_to_f32(static_cast<uint16_t>(sy[u].x & 0xffffu));
            const float v1 = __uint_as_float(static_cast<uint32_t>(lo[u] >> 32)) + bf16_to_f32(static_cast<uint16_t>(sy[u].x >> 16));
            const float v2 = __uint_as_float(static_cast<uint32_t>(hi[u])) + bf16_to_f32(static_cast<uint16_t>(sy[u].y & 0xffffu));
            const float v3 = __uint_as_float(static_cast<uint32_t>(hi[u] >> 32)) + bf16_to_f32(static_cast<uint16_t>(sy[u].y >> 16));
            *reinterpret_cast<uint2*>(o.out + off[u]) = uint2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
    }
}

// Logical block of block b among the grid's first G blocks, XCD-major:
// block b runs on XCD b % 8 (8 XCDs, each with its own L2), and XCD x takes
// logical blocks S_x .. S_x + n_x - 1 in order, n_x = |{b < G : b % 8 = x}|.
// The m-tiles of one expert are consecutive logical blocks, so they run side
// by side on one XCD and its L2 serves the expert's weights to all of them.
__device__ __forceinline__ int xcd_major(int b, int G) {
    const int x = b & 7, q = G >> 3, r = G & 7;
    return x * q + (x < r ? x : r) + (b >> 3);
}

// Logical grid: (m-tiles x slices), the slices of one m-tile consecutive.
template <int BH, int SW>
__global__ __launch_bounds__(kThreads) void fused_dma_kernel(Bf16Args a) {
    using T = DmaTile<2, 256, 2>;  // phase 1: 512-byte row segments, KC = 256 values per stage
    using F = FusedTile<BH>;
    constexpr int NT = 2;
    static_assert(F::G1 >= 2, "a token chunk's slot is refilled at the chunk's second stage");
    constexpr int W_INS = 2 * T::W_INS, T_INS = 2 * T::T_INS;  // per wave of the pair that moves them
    static_assert(W_INS * 1024 * 2 == T::W_BYTES, "a stage is the two weight waves' DMAs");
    static_assert(SW * T::W_BYTES + 2 * T::T_BYTES + F::ACT <= 160 * 1024 - 512, "LDS of a CU");
    static_assert((SW - 1) * W_INS < 64, "vmcnt range");
    static_assert(2 * T::T_BYTES == T::W_BYTES, "the token ring holds one weight stage in phase 2");
    __shared__ __attribute__((aligned(16))) uint8_t lds[SW * T::W_BYTES + 2 * T::T_BYTES + F::ACT];
    __shared__ int64_t sRow[32];  // acc32 row offset (token * D) of each m-tile row
    __shared__ float sW[32];      // its routing weight (0 past the tile's rows)
    __shared__ int sTok[32];      // its token
    __shared__ int sTgt[32];      // partial rows that complete its token's row: H / BH per routed pair
    __shared__ int sDone[33];     // [32]: count of the tokens whose rows this block completes, then the tokens
    uint8_t* const tring = lds + SW * T::W_BYTES;
    uint8_t* const act = tring + 2 * T::T_BYTES;
    const int nslices = a.H / BH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const FusedOut fo{a.T, a.D, a.k, a.rv.pair_to_sorted, a.acc32, a.tcnt, a.out, a.shared_y};
    if (wave == 1) fused_write_unrouted(fo, lane);  // overlaps wave 0's m-tile lookup
    MTile mt;
    int lb = blockIdx.x;  // logical block
    if (a.E > kWaveLookupMaxExperts) {
        if (!find_mtile<32>(a.rv, a.E, lb / nslices, mt)) return;
    } else {
        const TileSamples ts = tile_samples(a.rv, a.E, lane);
        const int G = ts.M * nslices;
        if (static_cast<int>(blockIdx.x) >= G) return;
        lb = xcd_major(blockIdx.x, G);
        find_mtile_wave(a.rv, a.E, ts, lb / nslices, lane, mt);
    }
    const int slice = lb % nslices;
    const bool wmover = wave < 2;
    const int mw = wave & 1;
    const int h0 = slice * BH;
    const int r = lane & 15, kg = lane >> 4;
    const int KIT1 = a.D / 256, NIT1 = F::G1 * KIT1, NG2 = a.D / F::R2, NIT = NIT1 + NG2;
    // the blocks of one (expert, slice) walk K and the W2 row groups in the
    // same order, so one XCD's L2 serves their common weights; each (expert,
    // slice) starts at its own chunk and row group, so the reads of different
    // weights spread over the HBM channels instead of crowding a few
    const int es = mt.expert * nslices + slice;
    const int kc0 = es % KIT1;
    const int rot = es % NG2;
    if (threadIdx.x < 32) {
        const int m = threadIdx.x;
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (m < mt.rows ? m : 0)], a.P);
        sRow[m] = static_cast<int64_t>(p / a.k) * a.D;
        sW[m] = m < mt.rows ? a.wts[p] : 0.0f;
        sTok[m] = p / a.k;
        const int tg = fused_target(fo, p / a.k, nslices);
        sTgt[m] = m < mt.rows ? tg : 0;
        if (m == 0) sDone[32] = 0;
    }
    const char* src[W_INS];
    if (wmover) {
        // W1 rows in the slot as dma_kmajor_kernel lays them out: each 16-row
        // block holds 8 gate rows and the 8 up rows of the same act columns
        const int pc = lane % T::CPR;
#pragma unroll
        for (int j = 0; j < W_INS; ++j) {
            const int row = (mw * W_INS + j) * T::RPI + lane / T::CPR;  // slot row 0..63
            const int c = pc ^ (row & (T::CPR - 1));
            const int jj = row & 15, h = h0 + 8 * (row >> 4) + (jj & 7);
            const int64_t grow = static_cast<int64_t>(mt.expert) * 2 * a.H + (jj < 8 ? h : a.H + h);
            src[j] = reinterpret_cast<const char*>(a.w1) + grow * a.D * 2 + c * 16;
        }
    } else {
        const int pc = lane % T::CPR;
#pragma unroll
        for (int j = 0; j < W_INS; ++j) {
            const int m = (mw * T_INS + (j < T_INS ? j : 0)) * T::RPI + lane / T::CPR;
            const int c = pc ^ (m & (T::CPR - 1));
            const int mm = m < mt.rows ? m : 0;
            const int64_t tok = clamp_pair(a.rv.sorted_to_pair[mt.row0 + mm], a.P) / a.k;
            src[j] = reinterpret_cast<const char*>(a.x) + tok * a.D * 2 + c * 16;
        }
    }
    __syncthreads();  // sRow / sW, and every wave's index loads done before the ring starts
    const int64_t gstride1 = static_cast<int64_t>(32) * a.D * 2, gstride2 = static_cast<int64_t>(F::R2) * a.H * 2;
    // LDS slot of weight stage `it`: phase 1 cycles over the SW weight slots;
    // phase 2, which no longer needs the token ring, cycles over SW + 1 slots
    // (the next SW weight slots in order, then the token ring's 32 KB), so it
    // keeps SW - 1 stages in flight instead of SW - 2
    auto wslot_of = [&](int it) -> uint8_t* {
        if (it < NIT1) return lds + (it % SW) * T::W_BYTES;
        const int i2 = (it - NIT1) % (SW + 1);
        return i2 == SW ? tring : lds + ((NIT1 + i2) % SW) * T::W_BYTES;
    };
    // weight stage `it`: phase 1 (group it % G1 of K chunk it / G1, the chunks
    // walked from the block's own chunk kc0) or phase 2 (R2 W2 rows of group
    // (it - NIT1 + rot) % NG2, the slice's columns)
    auto issue_w = [&](int it) {
        if (it == NIT1) {
            const int pc = lane % F::CPR2;
#pragma unroll
            for (int j = 0; j < W_INS; ++j) {
                const int row = (mw * W_INS + j) * F::RPI2 + lane / F::CPR2;
                const int c = pc ^ (row & (F::CPR2 - 1));
                src[j] = reinterpret_cast<const char*>(a.w2) +
                         ((static_cast<int64_t>(mt.expert) * a.D + row) * a.H + h0) * 2 + c * 16;
            }
        }
        const int64_t off = it < NIT1
            ? static_cast<int64_t>((it / F::G1 + kc0) % KIT1) * T::RB + (it % F::G1) * gstride1
            : ((it - NIT1 + rot) % NG2) * gstride2;
        uint8_t* slot = wslot_of(it);
#pragma unroll
        for (int j = 0; j < W_INS; ++j)
            __builtin_amdgcn_global_load_lds(src[j] + off, (lds_ptr_t)(slot + (mw * W_INS + j) * 1024), 16, 0,
                                             kWeightDmaAux);
    };
    // the 32 token rows' K chunk kc, into token slot kc & 1
    auto issue_t = [&](int kc) {
        const int64_t off = static_cast<int64_t>((kc + kc0) % KIT1) * T::RB;
        uint8_t* slot = tring + (kc & 1) * T::T_BYTES;
#pragma unroll
        for (int j = 0; j < T_INS; ++j)
            __builtin_amdgcn_global_load_lds(src[j] + off, (lds_ptr_t)(slot + (mw * T_INS + j) * 1024), 16, 0, 0);
    };
    // Stage `it` of the ring: each wave waits for its own DMAs of the stage
    // (the weight waves: later stages keep W_INS each in flight; the token
    // waves: the chunk's tokens, their only DMAs), one barrier, then the
    // weight waves issue the stage SW - 1 ahead (SW ahead in phase 2) and the
    // token waves, at a chunk's second stage, the next chunk's tokens (chunk
    // kc + 1's slot was last read at chunk kc - 1's first stage).
    auto ring_step = [&](int it) {
        if (wmover) {
            const int ahead = (it > NIT1 ? it + SW - 1 : it + SW - 2) - it;
            const int left = NIT - 1 - it;
            const int n = ahead < left ? ahead : left;
            if (n >= SW - 1) wait_vm<(SW - 1) * W_INS>();
            else if (n == SW - 2) wait_vm<(SW - 2) * W_INS>();
            else wait_vm<0>();
        } else if (it < NIT1 && it % F::G1 == 0) {
            wait_vm<0>();
        }
        if (it == NIT1) lds_barrier();  // the act tile's last LDS writes are complete
        else ring_barrier();
        if (wmover) {
            if (it < NIT1) {
                if (it + SW - 1 < NIT) issue_w(it + SW - 1);
            } else {
                if (it == NIT1 && it + SW - 1 < NIT) issue_w(it + SW - 1);  // the token ring is free from here
                if (it + SW < NIT) issue_w(it + SW);
            }
        } else if (it < NIT1 && it % F::G1 == 1 && it / F::G1 + 1 < KIT1) {
            issue_t(it / F::G1 + 1);
        }
    };
    if (wmover) {
#pragma unroll
        for (int j = 0; j < SW - 1; ++j) issue_w(j);
    } else {
        issue_t(0);
    }
    // Phase 1, k-major as dma_kmajor_kernel: each wave owns 16 of a stage's 64
    // W1 rows over the whole K chunk (no cross-wave reduction) against the
    // chunk's token fragments, read once per chunk and kept in registers
    // across its G1 groups; after the last chunk, silu(gate) * up of each
    // group (the up rows 32 lanes away) goes into the act tile.
    int it = 0;
    {
        f32x4_t acc[F::G1][NT];
#pragma unroll
        for (int g = 0; g < F::G1; ++g)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[g][t] = f32x4_t{};
        for (int kc = 0; kc < KIT1; ++kc) {
            bf16x8_t tk0[T::NS], tk1[T::NS];
#pragma unroll
            for (int g = 0; g < F::G1; ++g, ++it) {
                ring_step(it);
                if (g == 0) {
                    const uint8_t* ts = tring + (kc & 1) * T::T_BYTES;
                    uint32_t p0[T::NS], p1[T::NS];
#pragma unroll
                    for (int ks = 0; ks < T::NS; ++ks) {
                        const int c = 4 * ks + kg;
                        p0[ks] = lds_addr(ts + r * T::RB + ((c ^ r) << 4));
                        p1[ks] = lds_addr(ts + (16 + r) * T::RB + ((c ^ (16 + r)) << 4));
                    }
                    lds_read8(tk0, p0);
                    lds_read8(tk1, p1);
                }
                const uint8_t* slot = wslot_of(it);
                const int row = 16 * wave + r;
                uint32_t pw[T::NS];
#pragma unroll
                for (int ks = 0; ks < T::NS; ++ks)
                    pw[ks] = lds_addr(slot + row * T::RB + (((4 * ks + kg) ^ (row & 31)) << 4));
                bf16x8_t w[T::NS];
                lds_read8(w, pw);
#pragma unroll
                for (int ks = 0; ks < T::NS; ++ks) {
                    acc[g][0] = mfma16(w[ks], tk0[ks], acc[g][0]);
                    acc[g][1] = mfma16(w[ks], tk1[ks], acc[g][1]);
                }
                if (kc != KIT1 - 1) continue;
                // acc[g][t][q]: slot row 16 wave + 4 kg + q, token 16 t + r; lanes
                // kg < 2 hold gate rows, kg >= 2 the matching up rows
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    float up[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) up[q] = __shfl_xor(acc[g][t][q], 32);
                    if (kg >= 2) continue;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float gt = acc[g][t][q];
                        v[q] = gt / (1.0f + __expf(-gt)) * up[q];
                    }
                    const int m = 16 * t + r, h = 32 * g + 8 * wave + 4 * kg;  // act columns h .. h + 3
                    lds_write_b64(lds_addr(act + m * F::RB2 + (((h >> 3) ^ (m & (F::CPR2 - 1))) << 4) + (h & 7) * 2),
                                  pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        }
    }
    for (; it < NIT; ++it) {
        ring_step(it);
        uint8_t* wslot = wslot_of(it);
        // phase 2, token waves only: act tile x the stage's R2 W2 rows, each
        // wave half of the rows in 32-feature blocks, on the 32 x 32 MFMA with
        // the tokens as its rows. A register of its result then holds 32
        // consecutive output features of two token rows, so weight * partial
        // goes straight from the accumulators to the atomics, each instruction
        // covering two whole 128-byte lines (MI355X's L2 atomics cost per line).
        if (wmover) continue;
        f32x16_t y[F::FB2];
#pragma unroll
        for (int fb = 0; fb < F::FB2; ++fb) y[fb] = f32x16_t{};
        const int f0 = (wave - 2) * (F::R2 / 2) + (lane & 31);  // this lane's feature in block 0
        const int tm = lane & 31;                                 // this lane's token row (A operand)
#pragma unroll
        for (int k0 = 0; k0 < F::KS2; k0 += 4) {
            uint32_t pa[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = 2 * (k0 + u) + (lane >> 5);
                pa[u] = lds_addr(act + tm * F::RB2 + ((c ^ (tm & (F::CPR2 - 1))) << 4));
            }
            bf16x8_t af[4];
            lds_read4(af, pa);
#pragma unroll
            for (int fb = 0; fb < F::FB2; ++fb) {
                const int row = f0 + 32 * fb;
                uint32_t pw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = 2 * (k0 + u) + (lane >> 5);
                    pw[u] = lds_addr(wslot + row * F::RB2 + ((c ^ (row & (F::CPR2 - 1))) << 4));
                }
                bf16x8_t wf[4];
                lds_read4(wf, pw);
#pragma unroll
                for (int u = 0; u < 4; ++u) y[fb] = mfma32(af[u], wf[u], y[fb]);
            }
        }
        const int d0 = ((it - NIT1 + rot) % NG2) * F::R2;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int mlo = ((v >> 2) << 3) + (v & 3);  // lanes 0-31: token row mlo, lanes 32-63: mlo + 4
            if (mlo >= mt.rows) continue;
            const int m = mlo + ((lane >> 5) << 2);
            if (m < mt.rows) {
                float* dst = a.acc32 + sRow[m] + d0 + f0;
                const float w = sW[m];
#pragma unroll
                for (int fb = 0; fb < F::FB2; ++fb) unsafeAtomicAdd(dst + 32 * fb, w * y[fb][v]);
            }
        }
    }
    fused_finish(fo, mt.rows, !wmover, wave, lane, sTok, sTgt, sDone);
}

// ---------------- the fused MX-fp8 pass on the rings ----------------
// The same pass with MX-fp8 operands ("Prime Flash MoE", section 7: e4m3
// codes with an e8m0 scale per 32 along K; the act requantized on chip).
// Phase 1 is mx_kmajor_kernel's GEMM1 on the slice's row groups: a stage is
// one group's 64 W1 rows (32 act columns, gate and up rows interleaved
// 4 + 4 per 8 rows) x 512 codes with their scale bytes, the m-tile's token
// chunk of 512 codes rides with a chunk's first stage, and the four waves
// are two 32-row blocks x two halves of the chunk's K (the halves meet in
// LDS after the last chunk). After the last chunk each group's silu(gate)
// * up is requantized by MXQ (one scale per token and group: the group's
// 32 act columns are one MX block) into an act tile of e4m3 codes and
// scale bytes in LDS. Phase 2 streams the slice's codes of every W2 row
// (32 KB stages of R2 rows) with their scale bytes; the token waves run
// the scaled 32 x 32 x 64 MFMA with the tokens as its rows and add the
// results straight to the accumulator, as in fused_dma_kernel.
template <int BH>
struct MxFusedTile {
    static constexpr int G1 = BH / 32;       // GEMM1 row groups per slice
    static constexpr int R2 = 32768 / BH;    // W2 rows per stage (32 KB of codes)
    static constexpr int CPR2 = BH / 16;     // 16-byte chunks per W2 (and act) row
    static constexpr int RPI2 = 1024 / BH;   // W2 rows per DMA instruction
    static constexpr int SB2 = BH / 32;      // scale bytes of a W2 (and act) row in the slice
    static constexpr int KS2 = BH / 64;      // scaled-MFMA k-steps over the slice
    static constexpr int FB2 = R2 / 64;      // 32-feature blocks of a token wave per stage
    static constexpr int ACT = 32 * BH;      // act codes [32 tokens][BH]
    static constexpr int ACTS = 32 * SB2;    // act scale bytes [32 tokens][BH / 32]
    static_assert(BH == 128, "128-wide slices");
    static_assert(R2 * SB2 == 1024, "a stage's W2 scales fill the slot's 1 KB scale area");
};

__device__ __forceinline__ void lds_write_b128(uint32_t addr, u32x4_t v) {
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_write_b8(uint32_t addr, uint32_t v) {
    asm volatile("ds_write_b8 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// grid: (m-tiles x slices), the slices of one m-tile consecutive.
template <int BH, int SW>
__global__ __launch_bounds__(kThreads) void mx_fused_dma_kernel(MxArgs a, int one_round) {
    using C = Mx4<64, false>;  // phase 1: 64 e4m3 weight rows x 512 codes per stage, 16 KB token chunks
    using F = MxFusedTile<BH>;
    constexpr int WSLOT = C::WB + 64 * 16;        // codes, then 64 scale rows of 16 bytes
    constexpr int TSLOT = C::TB + 64 * 16;        // token codes, then 32 scale rows (and a 512-byte pad)
    constexpr int W_INS = 2 * C::WINS, T_INS = 2 * C::TINS;  // per wave of the pair that moves them
    constexpr int NSK = 4;                        // 64-code k-steps of a wave's half of a stage
    static_assert(C::WB == 32768 && C::TB == 16384 && C::WRB == 512 && C::WCH == 32 && C::WRPI == 2, "geometry");
    static_assert(W_INS * 1024 * 2 == C::WB && T_INS * 1024 * 2 == C::TB, "the pairs' DMAs");
    static_assert(SW * WSLOT + TSLOT + F::ACT + F::ACTS <= 160 * 1024 - 1536, "LDS of a CU");
    static_assert((SW - 2) * W_INS < 64, "vmcnt range");
    static_assert(F::G1 >= 2, "a token chunk's slot is refilled at the chunk's second stage");
    __shared__ __attribute__((aligned(16))) uint8_t lds[SW * WSLOT + TSLOT + F::ACT + F::ACTS];
    __shared__ float xamax[2][2][32];  // per group parity, row block and token: the act maximum of 16 columns
    __shared__ int64_t sRow[32];
    __shared__ float sW[32];
    __shared__ int sTok[32];
    __shared__ int sTgt[32];
    __shared__ int sDone[33];
    uint8_t* const tslot = lds + SW * WSLOT;
    uint8_t* const act = tslot + TSLOT;
    uint8_t* const acts = act + F::ACT;
    const int nslices = a.H / BH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const FusedOut fo{a.T, a.D, a.k, a.rv.pair_to_sorted, a.acc32, a.tcnt, a.out, nullptr};
    if (wave == 1) fused_write_unrouted(fo, lane);
    MTile mt;
    // Block order: XCD-major as in fused_dma_kernel while the blocks fit one
    // round of the CUs (`one_round`, from the expected m-tile count: the
    // slices of an m-tile then share its token rows in one L2); the plain
    // grid order (m-tile-major, slices consecutive) otherwise, measured
    // faster here from 1024 tokens of the MX workload's dims on, where the
    // twelve 128-wide slices' atomic adds bound the kernel.
    int lb = blockIdx.x;  // logical block
    if (a.E > kWaveLookupMaxExperts) {
        if (!find_mtile<32>(a.rv, a.E, lb / nslices, mt)) return;
    } else {
        const TileSamples ts = tile_samples(a.rv, a.E, lane);
        const int G = ts.M * nslices;
        if (static_cast<int>(blockIdx.x) >= G) return;
        if (one_round) lb = xcd_major(blockIdx.x, G);
        find_mtile_wave(a.rv, a.E, ts, lb / nslices, lane, mt);
    }
    const int slice = lb % nslices;
    const bool wmover = wave < 2;
    const int mw = wave & 1;
    const int rb = wave & 1, kp = wave >> 1;  // phase 1: row block and K half of this wave
    const int lr = lane & 31, g = lane >> 5;
    const int h0 = slice * BH;
    const int DB = a.D / 32, HB = a.H / 32;   // scale bytes per W1 / W2 row
    const int KIT1 = a.D / kMx4KC, NIT1 = F::G1 * KIT1, NG2 = a.D / F::R2, NIT = NIT1 + NG2;
    const int kc0 = lb % KIT1;
    const int rot = (lb / nslices + slice) % NG2;
    if (threadIdx.x < 32) {
        const int m = threadIdx.x;
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (m < mt.rows ? m : 0)], a.P);
        sRow[m] = static_cast<int64_t>(p / a.k) * a.D;
        sW[m] = m < mt.rows ? a.wts[p] : 0.0f;
        sTok[m] = p / a.k;
        const int tg = fused_target(fo, p / a.k, nslices);
        sTgt[m] = m < mt.rows ? tg : 0;
        if (m == 0) sDone[32] = 0;
    }
    // DMA sources. Weight waves: W1 code rows of group 0 (slot row r: act
    // column h0 + 16 (r >> 5) + 4 ((r & 31) >> 3) + (r & 3), gate rows where
    // r & 4 is clear, up rows where it is set), wave 0 also lane r's scale
    // row. Token waves: the m-tile's token code rows, wave 2 also the token
    // scale rows (lanes 32..63 repeat rows 0..31 into the slot's pad).
    const char* src[W_INS];
    const char* ssrc = nullptr;
    auto w1row = [&](int r) -> int64_t {
        const int col = h0 + 16 * (r >> 5) + 4 * ((r & 31) >> 3) + (r & 3);
        return static_cast<int64_t>(mt.expert) * 2 * a.H + ((r & 4) ? a.H + col : col);
    };
    auto trow = [&](int m) -> int64_t {
        return clamp_pair(a.rv.sorted_to_pair[mt.row0 + (m < mt.rows ? m : 0)], a.P) / a.k;
    };
    if (wmover) {
#pragma unroll
        for (int j = 0; j < W_INS; ++j) {
            const int row = (mw * W_INS + j) * C::WRPI + lane / C::WCH;
            const int c = (lane & (C::WCH - 1)) ^ (row & (C::WCH - 1));
            src[j] = reinterpret_cast<const char*>(a.w1) + w1row(row) * a.D + c * 16;
        }
        if (mw == 0) ssrc = reinterpret_cast<const char*>(a.w1s) + w1row(lane) * DB;
    } else {
#pragma unroll
        for (int j = 0; j < W_INS; ++j) {
            const int m = (mw * T_INS + (j < T_INS ? j : 0)) * 2 + lane / 32;
            const int c = (lane & 31) ^ (m & 31);
            src[j] = reinterpret_cast<const char*>(a.x) + trow(m) * a.D + c * 16;
        }
        if (mw == 0) ssrc = reinterpret_cast<const char*>(a.xs) + trow(lane & 31) * DB;
    }
    __syncthreads();  // sRow / sW / sTgt, and every wave's index loads done before the ring starts
    const int64_t gcode1 = static_cast<int64_t>(32) * a.D, gscale1 = static_cast<int64_t>(32) * DB;
    const int64_t gcode2 = static_cast<int64_t>(F::R2) * a.H, gscale2 = static_cast<int64_t>(F::R2) * HB;
    auto wslot_of = [&](int it) -> uint8_t* { return lds + (it % SW) * WSLOT; };
    // weight stage `it`: phase 1 (group it % G1 of K chunk it / G1, the chunks
    // walked from kc0) or phase 2 (R2 W2 rows of group (it - NIT1 + rot) %
    // NG2, the slice's codes; their scale bytes as dwords, 2 x 2 DMAs)
    auto issue_w = [&](int it) {
        if (it == NIT1) {
#pragma unroll
            for (int j = 0; j < W_INS; ++j) {
                const int row = (mw * W_INS + j) * F::RPI2 + lane / F::CPR2;
                const int c = (lane & (F::CPR2 - 1)) ^ (row & (F::CPR2 - 1));
                src[j] = reinterpret_cast<const char*>(a.w2) + (static_cast<int64_t>(mt.expert) * a.D + row) * a.H + h0 +
                         c * 16;
            }
        }
        uint8_t* slot = wslot_of(it);
        if (it < NIT1) {
            const int kr = (it / F::G1 + kc0) % KIT1, gr = it % F::G1;
            const int64_t off = static_cast<int64_t>(kr) * kMx4KC + gr * gcode1;
#pragma unroll
            for (int j = 0; j < W_INS; ++j)
                __builtin_amdgcn_global_load_lds(src[j] + off, (lds_ptr_t)(slot + (mw * W_INS + j) * 1024), 16, 0,
                                                 kWeightDmaAux);
            if (mw == 0)
                __builtin_amdgcn_global_load_lds(ssrc + static_cast<int64_t>(kr) * 16 + gr * gscale1,
                                                 (lds_ptr_t)(slot + C::WB), 16, 0, 0);
        } else {
            const int gr = (it - NIT1 + rot) % NG2;
            const int64_t off = gr * gcode2;
#pragma unroll
            for (int j = 0; j < W_INS; ++j)
                __builtin_amdgcn_global_load_lds(src[j] + off, (lds_ptr_t)(slot + (mw * W_INS + j) * 1024), 16, 0,
                                                 kWeightDmaAux);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = (2 * mw + i) * 64 + lane;  // dword q of the stage's 1 KB of scales
                const int row = q / (F::SB2 / 4), part = q % (F::SB2 / 4);
                const char* sp = reinterpret_cast<const char*>(a.w2s) +
                                 (static_cast<int64_t>(mt.expert) * a.D + gr * F::R2 + row) * HB + h0 / 32 + 4 * part;
                __builtin_amdgcn_global_load_lds(sp, (lds_ptr_t)(slot + C::WB + (2 * mw + i) * 256), 4, 0, 0);
            }
        }
    };
    // the token rows' K chunk kc (codes and scale bytes) into the token slot
    auto issue_t = [&](int kc) {
        const int kr = (kc + kc0) % KIT1;
#pragma unroll
        for (int j = 0; j < T_INS; ++j)
            __builtin_amdgcn_global_load_lds(src[j] + static_cast<int64_t>(kr) * kMx4KC,
                                             (lds_ptr_t)(tslot + (mw * T_INS + j) * 1024), 16, 0, 0);
        if (mw == 0)
            __builtin_amdgcn_global_load_lds(ssrc + static_cast<int64_t>(kr) * 16, (lds_ptr_t)(tslot + C::TB), 16, 0,
                                             0);
    };
    // Stage `it` of the ring: each wave waits for its own DMAs of the stage
    // (the weight waves: later stages keep at least W_INS each in flight;
    // the token waves: the chunk's tokens, their only DMAs), one barrier,
    // then the weight waves issue the stage SW - 1 ahead and the token waves,
    // at a chunk's second stage, the next chunk (every wave read the token
    // slot at the chunk's first stage).
    auto ring_step = [&](int it) {
        if (wmover) {
            const int left = NIT - 1 - it;
            const int n = SW - 2 < left ? SW - 2 : left;
            if (n == SW - 2) wait_vm<(SW - 2) * W_INS>();
            else if (n >= 1) wait_vm<W_INS>();
            else wait_vm<0>();
        } else if (it < NIT1 && it % F::G1 == 0) {
            wait_vm<0>();
        }
        if (it == NIT1) lds_barrier();  // the act tile's last LDS writes are complete
        else ring_barrier();
        if (wmover) {
            if (it + SW - 1 < NIT) issue_w(it + SW - 1);
        } else if (it < NIT1 && it % F::G1 == 1 && it / F::G1 + 1 < KIT1) {
            issue_t(it / F::G1 + 1);
        }
    };
    if (wmover) {
#pragma unroll
        for (int j = 0; j < SW - 1; ++j) issue_w(j);
    } else {
        issue_t(0);
    }
    int it = 0;
    {
        f32x16_t acc[F::G1];
#pragma unroll
        for (int gi = 0; gi < F::G1; ++gi) acc[gi] = f32x16_t{};
        const int row = 32 * rb + lr;  // this lane's weight row in the slot
        for (int kc = 0; kc < KIT1; ++kc) {
            u32x4_t tlo[NSK], thi[NSK];
            uint32_t tsc[NSK];
#pragma unroll
            for (int gi = 0; gi < F::G1; ++gi, ++it) {
                ring_step(it);
                if (gi == 0) {
                    uint32_t alo[4], ahi[4], as[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ks = kp * NSK + i, ct = 4 * ks + g;
                        alo[i] = lds_addr(tslot + lr * C::TRB + ((ct ^ lr) << 4));
                        ahi[i] = lds_addr(tslot + lr * C::TRB + (((ct + 2) ^ lr) << 4));
                        as[i] = lds_addr(tslot + C::TB + lr * 16 + 2 * ks + g);
                    }
                    mxk_read4x2(tlo, thi, tsc, alo, ahi, as);
                }
                const uint8_t* slot = wslot_of(it);
                uint32_t alo[4], ahi[4], as[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ks = kp * NSK + i, ct = 4 * ks + g;
                    alo[i] = lds_addr(slot + row * C::WRB + ((ct ^ (row & (C::WCH - 1))) << 4));
                    ahi[i] = lds_addr(slot + row * C::WRB + (((ct + 2) ^ (row & (C::WCH - 1))) << 4));
                    as[i] = lds_addr(slot + C::WB + row * 16 + 2 * ks + g);
                }
                u32x4_t wl[4], wh[4];
                uint32_t wsc[4];
                mxk_read4x2(wl, wh, wsc, alo, ahi, as);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x8_t aa{(int)wl[i].x, (int)wl[i].y, (int)wl[i].z, (int)wl[i].w,
                                     (int)wh[i].x, (int)wh[i].y, (int)wh[i].z, (int)wh[i].w};
                    const i32x8_t bt{(int)tlo[i].x, (int)tlo[i].y, (int)tlo[i].z, (int)tlo[i].w,
                                     (int)thi[i].x, (int)thi[i].y, (int)thi[i].z, (int)thi[i].w};
                    acc[gi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aa, bt, acc[gi], 0, 0, 0, (int)wsc[i],
                                                                             0, (int)tsc[i]);
                }
                if (kc != KIT1 - 1) continue;
                // group gi complete: the K halves meet in the slot just consumed
                // (free until the next stage's barrier); acc[gi][v]: slot row
                // 32 rb + 8 (v / 4) + 4 g + v % 4, token lr
                f32x16_t v = acc[gi];
                const uint32_t red = lds_addr(slot);
                lds_barrier();
                if (kp == 1) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) lds_store_f32(red + ((rb * 16 + q) * 64 + lane) * 4, v[q]);
                }
                lds_barrier();
                float amax = 0.0f, actv[16];
                if (kp == 0) {
#pragma unroll
                    for (int q0 = 0; q0 < 16; q0 += 4) {
                        uint32_t pq[4];
                        float o[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) pq[i] = red + ((rb * 16 + q0 + i) * 64 + lane) * 4;
                        lds_load4_f32(o, pq);
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[q0 + i] += o[i];
                    }
                }
                // gate rows in lanes g = 0, the matching up rows 32 lanes away
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const float up = __shfl_xor(v[q], 32);
                    actv[q] = v[q] / (1.0f + __expf(-v[q])) * up;
                    amax = fmaxf(amax, fabsf(actv[q]));
                }
                const int buf = gi & 1;
                if (kp == 0 && g == 0) xamax[buf][rb][lr] = amax;
                lds_barrier();
                if (kp == 0 && g == 0) {
                    // MXQ of the group's 32 act columns for token lr: this lane
                    // holds 16 of them (columns 32 gi + 16 rb + q), the other
                    // row block's wave the rest
                    const int sc = mx_scale_exp(fmaxf(amax, xamax[buf][rb ^ 1][lr]));
                    const float inv = pow2f(-sc);
                    uint32_t code[4];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        code[q4] = e4m3_encode(actv[4 * q4] * inv, actv[4 * q4]) |
                                   (e4m3_encode(actv[4 * q4 + 1] * inv, actv[4 * q4 + 1]) << 8) |
                                   (e4m3_encode(actv[4 * q4 + 2] * inv, actv[4 * q4 + 2]) << 16) |
                                   (e4m3_encode(actv[4 * q4 + 3] * inv, actv[4 * q4 + 3]) << 24);
                    const int c = 2 * gi + rb;  // the 16-byte chunk of the act row
                    lds_write_b128(lds_addr(act + lr * BH + ((c ^ (lr & (F::CPR2 - 1))) << 4)),
                                   u32x4_t{code[0], code[1], code[2], code[3]});
                    if (rb == 0) lds_write_b8(lds_addr(acts + lr * F::SB2 + gi), static_cast<uint32_t>(sc + 127));
                }
            }
        }
    }
    for (; it < NIT; ++it) {
        ring_step(it);
        if (wmover) continue;
        // phase 2, token waves only: act tile x the stage's R2 W2 rows, each
        // wave half of the rows in 32-feature blocks, on the scaled 32 x 32 x
        // 64 MFMA with the tokens as its rows (act the A operand)
        const uint8_t* slot = wslot_of(it);
        f32x16_t y[F::FB2];
#pragma unroll
        for (int fb = 0; fb < F::FB2; ++fb) y[fb] = f32x16_t{};
        const int fl = (wave - 2) * (F::R2 / 2) + lr;  // this lane's feature row in block 0
#pragma unroll
        for (int s0 = 0; s0 < F::KS2; s0 += 2) {
            // two k-steps at a time (mxk_read4x2 takes four operands: act and W2 of steps s0, s0 + 1)
            uint32_t alo[4], ahi[4], as[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ct = 4 * (s0 + i) + g;
                alo[i] = lds_addr(act + lr * BH + ((ct ^ (lr & (F::CPR2 - 1))) << 4));
                ahi[i] = lds_addr(act + lr * BH + (((ct + 2) ^ (lr & (F::CPR2 - 1))) << 4));
                as[i] = lds_addr(acts + lr * F::SB2 + 2 * (s0 + i) + g);
            }
#pragma unroll
            for (int fb = 0; fb < F::FB2; ++fb) {
                const int f = fl + 32 * fb;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int ct = 4 * (s0 + i) + g;
                    alo[2 + i] = lds_addr(slot + f * BH + ((ct ^ (f & (F::CPR2 - 1))) << 4));
                    ahi[2 + i] = lds_addr(slot + f * BH + (((ct + 2) ^ (f & (F::CPR2 - 1))) << 4));
                    as[2 + i] = lds_addr(slot + C::WB + f * F::SB2 + 2 * (s0 + i) + g);
                }
                u32x4_t lo[4], hi[4];
                uint32_t sc[4];
                mxk_read4x2(lo, hi, sc, alo, ahi, as);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const i32x8_t av{(int)lo[i].x, (int)lo[i].y, (int)lo[i].z, (int)lo[i].w,
                                     (int)hi[i].x, (int)hi[i].y, (int)hi[i].z, (int)hi[i].w};
                    const i32x8_t bw{(int)lo[2 + i].x, (int)lo[2 + i].y, (int)lo[2 + i].z, (int)lo[2 + i].w,
                                     (int)hi[2 + i].x, (int)hi[2 + i].y, (int)hi[2 + i].z, (int)hi[2 + i].w};
                    y[fb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bw, y[fb], 0, 0, 0, (int)sc[i], 0,
                                                                           (int)sc[2 + i]);
                }
            }
        }
        const int d0 = ((it - NIT1 + rot) % NG2) * F::R2;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int mlo = ((v >> 2) << 3) + (v & 3);  // lanes 0-31: token row mlo, lanes 32-63: mlo + 4
            if (mlo >= mt.rows) continue;
            const int m = mlo + (g << 2);
            if (m < mt.rows) {
                float* dst = a.acc32 + sRow[m] + d0 + fl;
                const float w = sW[m];
#pragma unroll
                for (int fb = 0; fb < F::FB2; ++fb) unsafeAtomicAdd(dst + 32 * fb, w * y[fb][v]);
            }
        }
    }
    fused_finish(fo, mt.rows, !wmover, wave, lane, sTok, sTgt, sDone);
}

inline int mtiles_upper(int64_t P, int E, int bm) { return static_cast<int>((P + bm - 1) / bm + E); }

}  // namespace

// AUTO's pipeline for a bf16 pass: the fused one where the pass is bound by
// launch latency, which is where its two kernels (route, fused) beat the
// split pipeline's four. Measured on MI355X (graph replay, ms, fused against
// split): D=256, H=512, E=8, k=2 at 16 to 256 tokens 0.021-0.027 against
// 0.028-0.034, at 1024 tokens (each expert's weights streamed once per
// 32-row m-tile, eight times) 0.045 against 0.045, at 4096 0.087 against
// 0.055; where the weights streamed run to hundreds of MB (D=2048 to 6144)
// the two are within a few percent at up to 16 tokens and the split pass
// is ahead from 32 on. So fused while the weights the fused kernel streams,
// 3 H D bf16 per expected m-tile, stay within 16 MB.
bool fused_preferred(int64_t T, int D, int H, int E, int k) {
    if (D % 256 || H % 128) return false;  // the fused decode-ring kernel's shapes
    return expected_mtiles32(T, k, E) * 3.0 * H * D * 2.0 <= 16e6;
}

// AUTO's pipeline for an MX-fp8 pass: the fused ring kernel streams the
// same weights as the split decode kernels in one launch instead of three,
// and wins while its (m-tile, slice) blocks fit one round of the CUs; past
// that each further round pays a block start and a ring fill again.
// Measured (graph replay, fused / split) at D=4096, H=1536, E=64, k=6: 0.93,
// 0.99, 0.95 at 1, 2 and 4 tokens (72, 138 and 250 expected blocks), 1.04
// at 8 (419 blocks), 1.15 at 16.
bool mx_fused_preferred(int64_t T, int D, int H, int E, int k) {
    if (D % 512 || H % 128) return false;  // the MX fused ring kernel's shapes
    return expected_mtiles32(T, k, E) * (H / 128) <= device_cu_count();
}

bool fused_decode_supported(const Bf16Args& a) {
    return a.D % 256 == 0 && a.H % 128 == 0 && !a.av.on();
}

// Slice width of the fused kernel: a block (m-tile, slice) is the unit of
// work, and the blocks run about one per CU, so the width whose block count
// fills whole rounds of the CUs best wins, the widest of those within 5%
// of the best fill (wider slices: fewer partial rows to add, longer W2 row
// segments, fewer blocks to start). Measured (graph replay, ms, widths
// 64 / 128 / 256): D=2048, H=768, E=128, k=8 at 4 tokens 0.083 / 0.077 /
// 0.125, at 16 tokens 0.162 / 0.151 / 0.143, at 64 tokens 0.245 / 0.226 /
// 0.257; D=6144, H=2048, E=32, k=8 at 8 tokens 0.420 / 0.381 / 0.366;
// D=256, H=512, E=8, k=2 at 16 tokens 0.023 / 0.028 / 0.039.
int fused_slice(const Bf16Args& a) {
    const double mt = expected_mtiles32(a.T, a.k, a.E), cus = device_cu_count();
    auto fill = [&](int bh) {
        if (a.H % bh) return 0.0;
        const double units = mt * (a.H / bh);
        return units / (std::ceil(units / cus) * cus);
    };
    const double best = std::max(fill(256), std::max(fill(128), fill(64)));
    for (int bh : {256, 128})
        if (fill(bh) >= 0.95 * best) return bh;
    return 64;
}

bool mx_fused_dma_supported(const MxArgs& a) {
    return !a.w4 && a.D % kMx4KC == 0 && a.H % 128 == 0;
}

// The MX kernel runs 128-wide slices: with 256 its eight groups'
// accumulators, the token and weight fragments and the requantization
// would not fit the registers (the compiler spills).
hipError_t launch_mx_fused_dma(const MxArgs& a, hipStream_t s) {
    constexpr int BH = 128;
    const int64_t blocks = static_cast<int64_t>(mtiles_upper(a.P, a.E, 32)) * (a.H / BH);
    const int one_round = expected_mtiles32(a.T, a.k, a.E) * (a.H / BH) <= device_cu_count();
    mx_fused_dma_kernel<BH, 4><<<static_cast<unsigned>(blocks), kThreads, 0, s>>>(a, one_round);
    return hipGetLastError();
}

hipError_t launch_fused_decode(const Bf16Args& a, hipStream_t s) {
    const int bh = fused_slice(a);
    const int64_t blocks = static_cast<int64_t>(mtiles_upper(a.P, a.E, 32)) * (a.H / bh);
    if (bh == 256) fused_dma_kernel<256, 3><<<static_cast<unsigned>(blocks), kThreads, 0, s>>>(a);
    else if (bh == 128) fused_dma_kernel<128, 3><<<static_cast<unsigned>(blocks), kThreads, 0, s>>>(a);
    else fused_dma_kernel<64, 3><<<static_cast<unsigned>(blocks), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
