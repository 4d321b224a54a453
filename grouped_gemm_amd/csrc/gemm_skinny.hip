// Decode-shaped bf16 grouped GEMMs: few routed tokens per expert.
//
// When an expert holds only a few rows (decode: ~16 tokens per expert, as in
// the 64-token, 32-local-expert, top-8 example of "Optimizing Grouped GEMM for
// MoE on Blackwell"), the pass is bound by reading every expert weight once
// from HBM. As in the swap-AB idea of "Porting Block-Scaled GEMM Kernels from
// Blackwell to Rubin" (section 5), the weights go on the MFMA's 16-row side
// and the tokens (up to 16*NT per m-tile) on the other (16x16x32 bf16 MFMA),
// so each weight byte is read once and used against every token of its
// expert.
//
// Getting close to the HBM roofline on gfx950 takes three things, each
// measured on MI355X:
//  * whole contiguous row segments per load instruction. The MFMA operand
//    layout alone would fetch 16 rows x 64 bytes per instruction (every
//    128-byte line in two halves); instead global->LDS DMA instructions
//    (global_load_lds_dwordx4: lane i's 16 bytes land at base + 16*i) fetch
//    512 contiguous bytes of a row per 32 lanes into a row-major LDS tile,
//    and the fragments are read back from it;
//  * the nontemporal policy on the weight DMA (streamed once);
//  * a multi-stage LDS ring whose waits are explicit: a fence-free barrier
//    and per-wave vmcnt budgets keep the later stages in flight (the
//    __syncthreads() fence, or a compiler-inserted wait before an LDS read
//    it cannot tell apart from the slots being filled, would drain it).
//
// GEMM1: a block owns 32 act columns h..h+31 of one expert per row group:
// gate rows h..h+31 and up rows H+h..H+h+31 of W1 (the gate/up pairing of
// "Prime Flash MoE", section 2, Trick 1), so silu(gate)*up is elementwise
// on the accumulators. GEMM2: a block owns 64 output features per row
// group; the epilogue scales by the routing weight and writes the pair's
// row for the segmented combine.
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// wait until at most n vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] at bits 3:0, vmcnt[5:4] at bits 15:14, expcnt 6:4, lgkmcnt 11:8
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every outstanding DMA (vmcnt(0)), draining the ring. Each
// wave has already waited for its own DMAs of the stage (wait_vm), and its
// LDS reads of the previous stage were consumed by MFMAs before it arrives,
// so the bare s_barrier orders everything the ring needs; the empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier after this wave's own LDS writes have completed (lgkmcnt(0)),
// leaving its in-flight global->LDS DMAs (vmcnt) running.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt max, expcnt max, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------- tile, DMA and fragment reads ----------------
// Global->LDS DMA instructions fetch
// whole row segments (RB = 2*KC bytes of one row per CPR = RB/16 lanes), into
// a row-major LDS tile whose 16-byte chunks are XOR-swizzled by the row
// (physical chunk = logical ^ (row mod CPR)), and the MFMA fragments are
// read from the tile; 16 rows reading one logical chunk hit 16 distinct bank
// groups. Per stage a block fetches 64 weight rows x RB bytes plus the
// 16*NT token rows x RB bytes; the four waves split the stage's k-steps and
// the partial sums meet in LDS at the end. Ring of S stages, one barrier per
// stage, each wave waits only for its own DMAs of the stage it consumes.
#ifndef MOE_DMA_AUX
#define MOE_DMA_AUX 2   // cache policy bits of the weight DMA: 2 = nontemporal (streamed once)
#endif

template <int NT, int KC, int S>
struct DmaTile {
    static constexpr int R = 64;                 // weight rows per block
    static constexpr int BM = 16 * NT;           // token rows per block
    static constexpr int RB = 2 * KC;            // bytes per row per stage
    static constexpr int CPR = RB / 16;          // 16-byte chunks per row per stage
    static constexpr int RPI = 64 / CPR;         // rows per DMA instruction
    static constexpr int W_INS = R / RPI / 4;    // weight DMA instructions per wave per stage
    static constexpr int T_INS = BM / RPI / 4;   // token DMA instructions per wave per stage
    static constexpr int W_BYTES = R * RB, T_BYTES = BM * RB, STAGE = W_BYTES + T_BYTES;
    static constexpr int NS = KC / 32;           // MFMA k-steps per stage
    static_assert(CPR >= 16 && CPR <= 64, "16..64 chunks per row keep the 16-row fragment reads conflict free");
    static_assert(W_INS * RPI * 4 == R && T_INS * RPI * 4 == BM, "DMA instructions must split evenly over waves");
    static_assert(S * STAGE <= 160 * 1024 && S >= 2, "ring must fit the LDS of a CU");
};

// Issue this wave's DMA instructions for ring stage `it` (row group `grp`
// relative to the block's first, K step `kit`) into slot it % S.
template <int NT, int KC, int S>
__device__ __forceinline__ void dma_issue(uint8_t* ring, int it, int grp, int kit, int64_t group_stride,
                                          const char* const* wsrc, const char* const* tsrc) {
    using T = DmaTile<NT, KC, S>;
    const int wave = threadIdx.x >> 6;
    uint8_t* slot = ring + (it % S) * T::STAGE;
    const int64_t kb = static_cast<int64_t>(kit) * T::RB;
    const int64_t wb = kb + grp * group_stride;
#pragma unroll
    for (int j = 0; j < T::W_INS; ++j)
        __builtin_amdgcn_global_load_lds(wsrc[j] + wb, (lds_ptr_t)(slot + (wave * T::W_INS + j) * 1024), 16, 0,
                                         MOE_DMA_AUX);
#pragma unroll
    for (int j = 0; j < T::T_INS; ++j)
        __builtin_amdgcn_global_load_lds(tsrc[j] + kb, (lds_ptr_t)(slot + T::W_BYTES + (wave * T::T_INS + j) * 1024),
                                         16, 0, 0);
}

// Six 16-byte LDS reads (4 weight fragments, 2 token fragments) and a wait
// for them, in one asm statement. Written as asm so that the compiler, which
// cannot tell the ring slot being read from the slots its DMAs are filling,
// does not insert vmcnt(0) before the reads (that would drain the ring every
// stage); the ring's own vmcnt waits and barriers already order these reads
// after the DMA that filled the slot.
__device__ __forceinline__ void lds_read6(bf16x8_t (&w)[4], bf16x8_t (&t)[2], const uint32_t (&pw)[4],
                                          const uint32_t (&pt)[2]) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(t[0]), "=&v"(t[1])
        : "v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]), "v"(pt[0]), "v"(pt[1])
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// grid: (m-tiles of 16*NT rows, row groups / G). A block walks G consecutive
// 64-row weight groups (GEMM1: 32 act columns = gate rows h..h+31 and up
// rows H+h..H+h+31; GEMM2: 64 output features) through one continuous ring,
// so the ring's fill and drain are paid once per block. The four waves split
// each stage's k-steps (8 independent accumulators per wave: 4 row blocks x
// 2 token tiles); at the end of a group the partials meet in the ring slot
// just consumed (LDS-only barriers, the DMAs in flight keep running).
template <int NT, int KC, int S, bool GEMM1>
__global__ __launch_bounds__(kThreads) void dma_skinny_kernel(Bf16Args a, int G) {
    using T = DmaTile<NT, KC, S>;
    constexpr int NB = 4, NV = NB * NT * 4;
    static_assert(NT == 2, "written for two token tiles");
    static_assert(T::NS % 4 == 0, "k-steps must split evenly over the four waves");
    // the group reduction reuses one ring slot, PB row blocks at a time
    constexpr int PB = (4 * NV * 64 * 4 <= T::STAGE) ? NB : (4 * (NV / 2) * 64 * 4 <= T::STAGE ? NB / 2 : 1);
    static_assert(4 * PB * NT * 4 * 64 * 4 <= T::STAGE, "reduction pass must fit one ring slot");
    __shared__ __attribute__((aligned(16))) uint8_t ring[S * T::STAGE];
    MTile mt;
    if (!find_mtile<T::BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = GEMM1 ? a.D : a.H;
    const int grp0 = blockIdx.y * G;  // first row group of this block
    const char* wsrc[T::W_INS];
    const char* tsrc[T::T_INS];
    const int pc = lane % T::CPR;
#pragma unroll
    for (int j = 0; j < T::W_INS; ++j) {
        const int row = (wave * T::W_INS + j) * T::RPI + lane / T::CPR;
        const int c = pc ^ (row & (T::CPR - 1));
        int64_t grow;
        if (GEMM1) {
            const int h0 = grp0 * 32;
            grow = static_cast<int64_t>(mt.expert) * 2 * a.H + (row < 32 ? h0 + row : a.H + h0 + row - 32);
        } else {
            grow = static_cast<int64_t>(mt.expert) * a.D + grp0 * 64 + row;
        }
        wsrc[j] = reinterpret_cast<const char*>(GEMM1 ? a.w1 : a.w2) + grow * K * 2 + c * 16;
    }
    const int64_t group_stride = static_cast<int64_t>(GEMM1 ? 32 : 64) * K * 2;
#pragma unroll
    for (int j = 0; j < T::T_INS; ++j) {
        const int m = (wave * T::T_INS + j) * T::RPI + lane / T::CPR;
        const int c = pc ^ (m & (T::CPR - 1));
        const int mm = m < mt.rows ? m : 0;
        int64_t grow;
        if (GEMM1) grow = clamp_pair(a.rv.sorted_to_pair[mt.row0 + mm], a.P) / a.k;
        else grow = mt.row0 + mm;
        tsrc[j] = reinterpret_cast<const char*>(GEMM1 ? a.x : a.act) + grow * K * 2 + c * 16;
    }
    const int r = lane & 15, kg = lane >> 4;
    const int KIT = K / KC, NIT = G * KIT;
    // GEMM2: each block walks its G groups starting at a different one.
    // Groups are 64 rows apart, so if every block visited them in the same
    // order, all blocks would read rows at the same offsets mod 64 rows at the
    // same time and, with rows a power of two of bytes apart (GEMM2's K = H:
    // 4 KB), pile onto the same subset of HBM channels; counters showed 18x
    // the DRAM credit stalls of GEMM1, and the rotation takes GEMM2 from 161
    // to 152 us on the decode workload. (GEMM1's 12 KB rows already spread
    // over the channels; rotating them measured 2% slower.)
    const int rot = GEMM1 ? 0 : (blockIdx.x + blockIdx.y) % G;
    f32x4_t acc[NB][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[b][t] = f32x4_t{};
#pragma unroll
    for (int j = 0; j < S - 1; ++j)
        if (j < NIT) dma_issue<NT, KC, S>(ring, j, (j / KIT + rot) % G, j % KIT, group_stride, wsrc, tsrc);
    for (int it = 0; it < NIT; ++it) {
        if (it + S - 2 < NIT) wait_vm<(S - 2) * (T::W_INS + T::T_INS)>();
        else wait_vm<0>();
        ring_barrier();
        if (it + S - 1 < NIT) {
            const int nx = it + S - 1;
            dma_issue<NT, KC, S>(ring, nx, (nx / KIT + rot) % G, nx % KIT, group_stride, wsrc, tsrc);
        }
        uint8_t* slot = ring + (it % S) * T::STAGE;
#pragma unroll
        for (int q = 0; q < T::NS / 4; ++q) {
            const int c = 4 * (wave * (T::NS / 4) + q) + kg;  // logical chunk of this lane's k-group
            uint32_t pw[4], pt[2];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int row = 16 * b + r;
                pw[b] = lds_addr(slot + row * T::RB + ((c ^ (row & (T::CPR - 1))) << 4));
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int m = 16 * t + r;
                pt[t] = lds_addr(slot + T::W_BYTES + m * T::RB + ((c ^ (m & (T::CPR - 1))) << 4));
            }
            bf16x8_t w[NB], tk[NT];
            lds_read6(w, tk, pw, pt);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[b][t] = mfma16(w[b], tk[t], acc[b][t]);
        }
        if (it % KIT != KIT - 1) continue;
        // group finished: sum the four waves' partials in this slot, PB row blocks per pass
        float* red = reinterpret_cast<float*>(slot);
        constexpr int PV = PB * NT * 4;  // floats per lane per pass
#pragma unroll
        for (int b0 = 0; b0 < NB; b0 += PB) {
            lds_barrier();
#pragma unroll
            for (int b = 0; b < PB; ++b)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[((wave * PV) + (b * NT + t) * 4 + v) * 64 + lane] = acc[b0 + b][t][v];
            lds_barrier();
#pragma unroll
            for (int b = 0; b < PB; ++b)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int i = ((b * NT + t) * 4 + v) * 64 + lane;
                        acc[b0 + b][t][v] =
                            (red[i] + red[PV * 64 + i]) + (red[2 * PV * 64 + i] + red[3 * PV * 64 + i]);
                    }
        }
        // epilogue: wave w stores token tile w (acc[b][t][v]: row 16b + 4kg + v, token 16t + r)
        const int g = grp0 + (it / KIT + rot) % G;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int m = 16 * t + r;
            if (t != wave || m >= mt.rows) continue;
            if (GEMM1) {
                uint16_t* dst = a.act + static_cast<int64_t>(mt.row0 + m) * a.H + g * 32 + 4 * kg;
                if (a.av.on()) {
                    const float al = a.av.alpha ? a.av.alpha[mt.expert] : 1.0f;
                    const float sc =
                        a.av.wba ? al * a.wts[clamp_pair(a.rv.sorted_to_pair[mt.row0 + m], a.P)] : al;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float v[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = act_variant(acc[j][t][q], acc[j + 2][t][q], sc, a.av.kind, a.av.limit);
                        *reinterpret_cast<uint2*>(dst + 16 * j) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    }
                    continue;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float gt = acc[j][t][q], u = acc[j + 2][t][q];
                        v[q] = gt / (1.0f + __expf(-gt)) * u;
                    }
                    *reinterpret_cast<uint2*>(dst + 16 * j) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                }
            } else {
                const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + m], a.P);
                const float wt = a.av.wba ? 1.0f : a.wts[p];
                uint16_t* dst = a.ypair + static_cast<int64_t>(p) * a.D + g * 64 + 4 * kg;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const f32x4_t& cc = acc[b][t];
                    *reinterpret_cast<uint2*>(dst + 16 * b) =
                        uint2{pack_bf16x2(cc[0] * wt, cc[1] * wt), pack_bf16x2(cc[2] * wt, cc[3] * wt)};
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[b][t] = f32x4_t{};
    }
}

inline int mtiles_upper(int64_t P, int E, int bm) { return static_cast<int>((P + bm - 1) / bm + E); }


#ifndef MOE_DMA_KC
#define MOE_DMA_KC 256
#endif

// Row groups per block: as many as leave about one block per CU, so that
// every CU fills its ring once and no second round of blocks runs on half the
// chip. The m-tile count is estimated from the average rows per expert (the
// real one is known only on the device).
int groups_per_block(int groups, int64_t P, int E) {
    const int64_t per_expert = (P / E + 31) / 32;
    const int64_t mtiles = static_cast<int64_t>(E) * (per_expert > 0 ? per_expert : 1);
    int64_t G = groups * mtiles / device_cu_count();
    if (G < 1) G = 1;
    if (G > groups) G = groups;
    while (groups % G) --G;
    return static_cast<int>(G);
}

hipError_t launch_dma(const Bf16Args& a, bool gemm1, hipStream_t s) {
    constexpr int NT = 2;  // m-tiles of 32 tokens
    const int K = gemm1 ? a.D : a.H;
    const int groups = gemm1 ? a.H / 32 : a.D / 64;
    const int G = groups_per_block(groups, a.P, a.E);
    dim3 g(mtiles_upper(a.P, a.E, 16 * NT), groups / G);
    const bool wide = MOE_DMA_KC == 256 && K % 256 == 0;
    if (gemm1) {
        if (wide) dma_skinny_kernel<NT, 256, 3, true><<<g, kThreads, 0, s>>>(a, G);
        else dma_skinny_kernel<NT, 128, 6, true><<<g, kThreads, 0, s>>>(a, G);
    } else {
        if (wide) dma_skinny_kernel<NT, 256, 3, false><<<g, kThreads, 0, s>>>(a, G);
        else dma_skinny_kernel<NT, 128, 6, false><<<g, kThreads, 0, s>>>(a, G);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny_gemm1(const Bf16Args& a, hipStream_t s) { return launch_dma(a, true, s); }

hipError_t launch_skinny_gemm2(const Bf16Args& a, hipStream_t s) { return launch_dma(a, false, s); }

}  // namespace moe
