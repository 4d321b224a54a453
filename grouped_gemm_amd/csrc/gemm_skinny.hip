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
//    it cannot tell apart from the slots being filled, would drain it);
//  * k-major order (dma_kmajor_kernel): each token chunk fetched once per K
//    chunk and kept in registers across a block's row groups, and each
//    block's K walk started at its own chunk.
//
// GEMM1: a block owns 32 act columns h..h+31 of one expert per row group:
// gate rows h..h+31 and up rows H+h..H+h+31 of W1 (the gate/up pairing of
// "Prime Flash MoE", section 2, Trick 1), so silu(gate)*up is elementwise
// on the accumulators. GEMM2: a block owns 64 output features per row
// group; the epilogue scales by the routing weight and writes the pair's
// row for the segmented combine.
#include <cmath>

#include "dma_ring.h"
#include "mxq.h"

namespace moe {

namespace {


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
                                         kWeightDmaAux);
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


// The epilogue's per-token values for token 16 * (wave & 1) + (lane & 15) of
// the m-tile (the token tile waves 0-1 store): its pair index and its scale
// (GEMM2: the routing weight, or 1 when it was applied before the
// activation; GEMM1: the activation variant's scale). Loaded once, before
// the ring starts, and waited for here: a global load in the loop would come
// with a vmcnt(0) wait that drains the wave's DMAs in flight.
template <bool GEMM1>
__device__ __forceinline__ void dma_epilogue_token(const Bf16Args& a, const MTile& mt, int wave, int lane, int& ep,
                                                   float& esc) {
    const int m = 16 * (wave & 1) + (lane & 15);
    ep = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (m < mt.rows ? m : 0)], a.P);
    if (GEMM1)
        esc = a.av.on() ? (a.av.alpha ? a.av.alpha[mt.expert] : 1.0f) * (a.av.wba ? a.wts[ep] : 1.0f) : 1.0f;
    else
        esc = a.av.wba ? 1.0f : a.wts[ep];
    asm volatile("" : "+v"(ep), "+v"(esc));
}

// End of a row group: the four waves' partials (acc[b][t][v]: row 16b +
// 4kg + v, token 16t + r) meet in `red` (a just-consumed ring slot of SLOT
// bytes, PB row blocks per pass, LDS-only barriers so the DMAs in flight
// keep running); wave t (t < 2) is left holding the sums of token tile t.
template <int SLOT>
__device__ __forceinline__ void group_reduce(f32x4_t (&acc)[4][2], float* red, int wave, int lane) {
    constexpr int NB = 4, NT = 2, NV = NB * NT * 4;
    constexpr int PB = (4 * NV * 64 * 4 <= SLOT) ? NB : (4 * (NV / 2) * 64 * 4 <= SLOT ? NB / 2 : 1);
    static_assert(4 * PB * NT * 4 * 64 * 4 <= SLOT, "reduction pass must fit one ring slot");
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
        // only wave t stores token tile t, so only it sums that tile
        if (wave < NT) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t != wave) continue;
#pragma unroll
                for (int b = 0; b < PB; ++b)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int i = ((b * NT + t) * 4 + v) * 64 + lane;
                        acc[b0 + b][t][v] =
                            (red[i] + red[PV * 64 + i]) + (red[2 * PV * 64 + i] + red[3 * PV * 64 + i]);
                    }
            }
        }
    }
}

// The split pipeline's group end: wave t stores token tile t of group g:
// GEMM1 the act columns g*32.. (silu(gate) * up, or the activation variant),
// GEMM2 the weighted outputs g*64.. of the pair's ypair row.
template <int SLOT, bool GEMM1>
__device__ __forceinline__ void dma_group_end(const Bf16Args& a, f32x4_t (&acc)[4][2], float* red, const MTile& mt,
                                              int g, int wave, int lane, int ep, float esc) {
    constexpr int NB = 4, NT = 2;
    const int r = lane & 15, kg = lane >> 4;
    group_reduce<SLOT>(acc, red, wave, lane);
    // epilogue: wave w stores token tile w (acc[b][t][v]: row 16b + 4kg + v, token 16t + r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int m = 16 * t + r;
        if (t != wave || m >= mt.rows) continue;
        if (GEMM1) {
            uint16_t* dst = a.act + static_cast<int64_t>(mt.row0 + m) * a.H + g * 32 + 4 * kg;
            if (a.av.on()) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = act_variant(acc[j][t][q], acc[j + 2][t][q], esc, a.av.kind, a.av.limit);
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
            uint16_t* dst = a.ypair + static_cast<int64_t>(ep) * a.D + g * 64 + 4 * kg;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4_t& cc = acc[b][t];
                *reinterpret_cast<uint2*>(dst + 16 * b) =
                    uint2{pack_bf16x2(cc[0] * esc, cc[1] * esc), pack_bf16x2(cc[2] * esc, cc[3] * esc)};
            }
        }
    }
}

// A decode kernel's block index: the row-group chunks of one m-tile are
// consecutive (1-D grid, chunk fastest), so the blocks of the m-tiles that
// exist, which come first, are dispatched before the ones past the m-tile
// count (the grid is sized for the most m-tiles the routes could produce;
// those blocks exit at once).
struct BlockPos {
    int mtile, chunk;
};
__device__ __forceinline__ BlockPos block_pos(int nchunks) {
    return BlockPos{static_cast<int>(blockIdx.x) / nchunks, static_cast<int>(blockIdx.x) % nchunks};
}

// grid: m-tiles of 16*NT rows x (row groups / G) chunks, 1-D (block_pos). A block walks G consecutive
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
    __shared__ __attribute__((aligned(16))) uint8_t ring[S * T::STAGE];
    MTile mt;
    const BlockPos bp = block_pos((GEMM1 ? a.H / 32 : a.D / 64) / G);
    if (!find_mtile<T::BM>(a.rv, a.E, bp.mtile, mt)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = GEMM1 ? a.D : a.H;
    const int grp0 = bp.chunk * G;  // first row group of this block
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
    const int rot = GEMM1 ? 0 : (bp.mtile + bp.chunk) % G;
    f32x4_t acc[NB][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[b][t] = f32x4_t{};
    int ep;
    float esc;
    dma_epilogue_token<GEMM1>(a, mt, wave, lane, ep, esc);
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
        dma_group_end<T::STAGE, GEMM1>(a, acc, reinterpret_cast<float*>(slot), mt, grp0 + (it / KIT + rot) % G, wave,
                                       lane, ep, esc);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[b][t] = f32x4_t{};
    }
}


// Most row groups a k-major block keeps accumulators for at once.
constexpr int kKmajorGroups = 12;

// A k-major block's G row groups cut into nsg super-groups of `base` or
// base + 1 groups (the first `rem` get one more); each super-group walks
// its K in 256-value chunks, and each chunk its groups: stage s is group gi
// of super-group sg at chunk kc.
struct KmajorPlan {
    int base, rem, kit;
    __device__ int first(int sg) const { return sg * base + (sg < rem ? sg : rem); }
    __device__ int size(int sg) const { return base + (sg < rem ? 1 : 0); }
    __device__ void locate(int s, int& sg, int& kc, int& gi) const {
        const int big = rem * (base + 1) * kit;
        int r;
        if (s < big) {
            sg = s / ((base + 1) * kit);
            r = s - sg * (base + 1) * kit;
        } else {
            const int q = (s - big) / (base * kit);
            sg = rem + q;
            r = s - big - q * base * kit;
        }
        const int gs = size(sg);
        kc = r / gs;
        gi = r - kc * gs;
    }
};

// A decode block's work: m-tile `mtile`, its row groups g0 .. g0 + n - 1.
struct DecodeWork {
    int mtile, g0, n;
};

// The k-major kernels' work, split on the device, where the m-tile count M
// (32-row tiles of the route just run) is known: the grid's B blocks (one
// per CU) are dealt out over the M m-tiles as evenly as they go (B mod M of
// them get one block more), and each m-tile's row groups as evenly over its
// blocks, at least MIN groups to a block (the fewest a super-group of the
// kernel holds; an m-tile takes no more blocks than that allows). A batch
// with an expert past 32 rows then spreads its extra m-tile over the chip
// instead of running a second round of blocks after the first. With M >= B
// (many experts hit), block b takes m-tile b whole (the grid holds at least
// M blocks).
template <int MIN>
__device__ __forceinline__ bool decode_work_m(int M, int groups, DecodeWork& w) {
    const int B = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
    if (M <= 0) return false;
    if (M >= B) {
        if (b >= M) return false;
        w = DecodeWork{b, 0, groups};
        return true;
    }
    const int base = B / M, extra = B % M, cap = groups / MIN;
    int j, q, nb;
    if (b < extra * (base + 1)) {
        j = b / (base + 1);
        q = b - j * (base + 1);
        nb = base + 1;
    } else {
        const int b2 = b - extra * (base + 1);
        j = extra + b2 / base;
        q = b2 - (j - extra) * base;
        nb = base;
    }
    if (nb > cap) {
        if (q >= cap) return false;
        nb = cap;
    }
    const int g0 = q * groups / nb, g1 = (q + 1) * groups / nb;
    w = DecodeWork{j, g0, g1 - g0};
    return true;
}

// A decode block's work and its m-tile (the m-tile count and the lookup from
// one wave-parallel read of the tile prefix sums, find_mtile_wave; a binary
// search past kWaveLookupMaxExperts experts).
template <int MIN>
__device__ __forceinline__ bool decode_lookup(const RouteView& rv, int E, int groups, DecodeWork& w, MTile& mt) {
    if (E > kWaveLookupMaxExperts) {
        const int M = rv.tile_prefix[tile_height_index(32) * (E + 1) + E];
        return decode_work_m<MIN>(M, groups, w) && find_mtile<32>(rv, E, w.mtile, mt);
    }
    const int lane = threadIdx.x & 63;
    const TileSamples s = tile_samples(rv, E, lane);
    if (!decode_work_m<MIN>(s.M, groups, w)) return false;
    find_mtile_wave(rv, E, s, w.mtile, lane, mt);
    return true;
}

// The decode GEMMs, k-major: a block (m-tile, G row groups: decode_work) walks K in
// 256-value chunks and, within a chunk, up to kKmajorGroups groups, so each
// chunk of the m-tile's 32 token rows (16 KB) is fetched once per chunk
// instead of once per group (with the token rows fetched per group, their
// L2 traffic was half the weights' and held HBM streaming about 10% below
// what the weights alone reach). A stage is one group's 64 weight rows x
// 512 bytes (32 KB, a 4-slot ring); the token chunk rides with the first
// stage of its chunk into a 2-slot token ring (the next chunk's tokens
// overwrite a slot only after two stages, so every super-group has at
// least two groups). Each wave owns 16 of a group's 64 rows for every
// k-step (no split-K, no cross-wave reduction) and keeps its fragments of
// the token chunk in registers across the chunk's groups. GEMM1's rows are
// laid out in the slot so that each 16-row block holds 8 gate rows and the
// 8 up rows of the same act columns: an MFMA lane holding gate rows finds
// the matching up rows 32 lanes away.
template <bool GEMM1>
__global__ __launch_bounds__(kThreads) void dma_kmajor_kernel(Bf16Args a) {
    using T = DmaTile<2, 256, 2>;  // 512-byte row segments: 32 KB weight stages, 16 KB token chunks
    constexpr int SW = 4, NT = 2, NS = T::NS, GSM = kKmajorGroups;
    constexpr int W_INS = T::W_INS, T_INS = T::T_INS;  // per wave per stage / per chunk
    static_assert(NS == 8 && T::CPR == 32 && T::RPI * T::RB == 1024, "512-byte segments, 8 k-steps per stage");
    static_assert(SW * T::W_BYTES + 2 * T::T_BYTES <= 160 * 1024, "rings must fit the LDS of a CU");
    static_assert((SW - 2) * W_INS < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) uint8_t lds[SW * T::W_BYTES + 2 * T::T_BYTES];
    uint8_t* const tring = lds + SW * T::W_BYTES;
    static_assert(T::BM == 32, "32-row m-tiles");
    DecodeWork wk;
    MTile mt;
    if (!decode_lookup<2>(a.rv, a.E, GEMM1 ? a.H / 32 : a.D / 64, wk, mt)) return;
    const int G = wk.n, nsg = (G + GSM - 1) / GSM;  // every super-group holds at least two groups
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, kg = lane >> 4;
    const int K = GEMM1 ? a.D : a.H;
    const int grp0 = wk.g0;
    const int pc = lane % T::CPR;
    const char* wsrc[W_INS];
#pragma unroll
    for (int j = 0; j < W_INS; ++j) {
        const int row = (wave * W_INS + j) * T::RPI + lane / T::CPR;  // slot row 0..63
        const int c = pc ^ (row & (T::CPR - 1));
        int64_t grow;
        if (GEMM1) {
            const int jj = row & 15, h = grp0 * 32 + 8 * (row >> 4) + (jj & 7);
            grow = static_cast<int64_t>(mt.expert) * 2 * a.H + (jj < 8 ? h : a.H + h);
        } else {
            grow = static_cast<int64_t>(mt.expert) * a.D + grp0 * 64 + row;
        }
        wsrc[j] = reinterpret_cast<const char*>(GEMM1 ? a.w1 : a.w2) + grow * K * 2 + c * 16;
    }
    const char* tsrc[T_INS];
#pragma unroll
    for (int j = 0; j < T_INS; ++j) {
        const int m = (wave * T_INS + j) * T::RPI + lane / T::CPR;  // token row 0..31
        const int c = pc ^ (m & (T::CPR - 1));
        const int mm = m < mt.rows ? m : 0;
        const int64_t grow = GEMM1 ? clamp_pair(a.rv.sorted_to_pair[mt.row0 + mm], a.P) / a.k : mt.row0 + mm;
        tsrc[j] = reinterpret_cast<const char*>(GEMM1 ? a.x : a.act) + grow * K * 2 + c * 16;
    }
    const int64_t group_stride = static_cast<int64_t>(GEMM1 ? 32 : 64) * K * 2;
    const int KIT = K / 256, NIT = G * KIT;
    const int rot = GEMM1 ? 0 : static_cast<int>(blockIdx.x + blockIdx.x / 8) % G;  // as in dma_skinny_kernel
    // The K chunks are walked from chunk kc0 on, wrapping: the blocks run in
    // near lockstep, and if every block read the same 512-byte column of its
    // rows at once, the reads would crowd a few HBM channels. Block b runs on
    // XCD b % 8, so the start also moves with b / 8: with b % KIT alone the
    // blocks of one XCD took only KIT / gcd(KIT, 8) distinct starts (one for
    // GEMM2's 8 chunks at the decode dims), and the XCDs' blocks finished up
    // to 14% apart; the same for GEMM2's row-group rotation.
    const int kc0 = static_cast<int>(blockIdx.x + blockIdx.x / 8) % KIT;
    const KmajorPlan pl{G / nsg, G % nsg, KIT};
    // epilogue values of tokens r and 16 + r (every wave stores both tiles)
    int ep[NT];
    float esc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int m = 16 * t + r;
        ep[t] = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (m < mt.rows ? m : 0)], a.P);
        if (GEMM1)
            esc[t] = a.av.on() ? (a.av.alpha ? a.av.alpha[mt.expert] : 1.0f) * (a.av.wba ? a.wts[ep[t]] : 1.0f) : 1.0f;
        else
            esc[t] = a.av.wba ? 1.0f : a.wts[ep[t]];
    }
    asm volatile("" : "+v"(ep[0]), "+v"(ep[1]), "+v"(esc[0]), "+v"(esc[1]));
    auto issue = [&](int st) {
        int sg, kc, gi;
        pl.locate(st, sg, kc, gi);
        const int g = (pl.first(sg) + gi + rot) % G;
        const int kr = (kc + kc0) % KIT;
        const int64_t off = static_cast<int64_t>(kr) * T::RB + g * group_stride;
        uint8_t* slot = lds + (st % SW) * T::W_BYTES;
#pragma unroll
        for (int j = 0; j < W_INS; ++j)
            __builtin_amdgcn_global_load_lds(wsrc[j] + off, (lds_ptr_t)(slot + (wave * W_INS + j) * 1024), 16, 0,
                                             kWeightDmaAux);
        if (gi == 0) {
            uint8_t* ts = tring + ((sg * KIT + kc) & 1) * T::T_BYTES;
#pragma unroll
            for (int j = 0; j < T_INS; ++j)
                __builtin_amdgcn_global_load_lds(tsrc[j] + static_cast<int64_t>(kr) * T::RB,
                                                 (lds_ptr_t)(ts + (wave * T_INS + j) * 1024), 16, 0, 0);
        }
    };
#pragma unroll
    for (int j = 0; j < SW - 1; ++j)
        if (j < NIT) issue(j);
    int s = 0;
    for (int sg = 0; sg < nsg; ++sg) {
        const int gs = pl.size(sg), gfirst = pl.first(sg);
        f32x4_t acc[GSM][NT];
#pragma unroll
        for (int gi = 0; gi < GSM; ++gi)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[gi][t] = f32x4_t{};
        for (int kc = 0; kc < KIT; ++kc) {
            bf16x8_t tk0[NS], tk1[NS];
#pragma unroll
            for (int gi = 0; gi < GSM; ++gi) {
                if (gi >= gs) continue;
                // the stage's DMAs (and, at gi = 0, the chunk's token DMAs issued with them) are this
                // wave's oldest; later stages hold at least W_INS each
                if (s + SW - 2 < NIT) wait_vm<(SW - 2) * W_INS>();
                else wait_vm<0>();
                ring_barrier();
                if (s + SW - 1 < NIT) issue(s + SW - 1);
                if (gi == 0) {
                    const uint8_t* ts = tring + ((sg * KIT + kc) & 1) * T::T_BYTES;
                    uint32_t p0[NS], p1[NS];
#pragma unroll
                    for (int ks = 0; ks < NS; ++ks) {
                        const int c = 4 * ks + kg;
                        p0[ks] = lds_addr(ts + r * T::RB + ((c ^ r) << 4));
                        p1[ks] = lds_addr(ts + (16 + r) * T::RB + ((c ^ (16 + r)) << 4));
                    }
                    lds_read8(tk0, p0);
                    lds_read8(tk1, p1);
                }
                const uint8_t* slot = lds + (s % SW) * T::W_BYTES;
                const int row = 16 * wave + r;
                uint32_t pw[NS];
#pragma unroll
                for (int ks = 0; ks < NS; ++ks) pw[ks] = lds_addr(slot + row * T::RB + (((4 * ks + kg) ^ (row & 31)) << 4));
                bf16x8_t w[NS];
                lds_read8(w, pw);
#pragma unroll
                for (int ks = 0; ks < NS; ++ks) {
                    acc[gi][0] = mfma16(w[ks], tk0[ks], acc[gi][0]);
                    acc[gi][1] = mfma16(w[ks], tk1[ks], acc[gi][1]);
                }
                ++s;
            }
        }
        // epilogue (acc[gi][t][v]: slot row 16 * wave + 4kg + v, token 16t + r)
#pragma unroll
        for (int gi = 0; gi < GSM; ++gi) {
            if (gi >= gs) continue;
            const int g = grp0 + (gfirst + gi + rot) % G;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int m = 16 * t + r;
                if (GEMM1) {
                    float up[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) up[q] = __shfl_xor(acc[gi][t][q], 32);
                    if (kg >= 2 || m >= mt.rows) continue;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float gt = acc[gi][t][q];
                        v[q] = a.av.on() ? act_variant(gt, up[q], esc[t], a.av.kind, a.av.limit)
                                         : gt / (1.0f + __expf(-gt)) * up[q];
                    }
                    uint16_t* dst = a.act + static_cast<int64_t>(mt.row0 + m) * a.H + g * 32 + 8 * wave + 4 * kg;
                    *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else {
                    if (m >= mt.rows) continue;
                    const f32x4_t& cc = acc[gi][t];
                    uint16_t* dst = a.ypair + static_cast<int64_t>(ep[t]) * a.D + g * 64 + 16 * wave + 4 * kg;
                    *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(cc[0] * esc[t], cc[1] * esc[t]),
                                                           pack_bf16x2(cc[2] * esc[t], cc[3] * esc[t])};
                }
            }
        }
    }
}

inline int mtiles_upper(int64_t P, int E, int bm) { return static_cast<int>((P + bm - 1) / bm + E); }




// Row groups per block: as many as leave about one block per CU, so that
// every CU fills its ring once and no second round of blocks runs on half the
// chip. The m-tile count is estimated from the routes spread uniformly (the
// real one is known only on the device): with fewer tokens than experts,
// only the experts hit hold m-tiles.
// G is the smallest divisor of the group count whose blocks fit in one round.
int groups_per_block(int groups, int64_t T, int k, int E) {
    const double mtiles = std::ceil(expected_mtiles32(T, k, E));
    for (int G = 1; G < groups; ++G)
        if (groups % G == 0 && mtiles * (groups / G) <= device_cu_count()) return G;
    return groups;
}

// Which decode kernel a GEMM runs: dma_kmajor_kernel when K is a multiple
// of 256, else dma_skinny_kernel (128-value stages). (The decode kernels run
// only with D and H multiples of 128, so a GEMM has at least two row groups,
// the pair dma_kmajor_kernel's blocks take them in.)
bool decode_kmajor(const Bf16Args& a, bool gemm1) { return (gemm1 ? a.D : a.H) % 256 == 0; }

hipError_t launch_dma(const Bf16Args& a, bool gemm1, hipStream_t s) {
    constexpr int NT = 2;  // m-tiles of 32 tokens
    const int groups = gemm1 ? a.H / 32 : a.D / 64;
    if (decode_kmajor(a, gemm1)) {  // one block per CU, or one per m-tile when they can be more (decode_work)
        const unsigned gk = static_cast<unsigned>(std::max(device_cu_count(), mtiles_upper(a.P, a.E, 16 * NT)));
        if (gemm1) dma_kmajor_kernel<true><<<gk, kThreads, 0, s>>>(a);
        else dma_kmajor_kernel<false><<<gk, kThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    const int G = groups_per_block(groups, a.T, a.k, a.E);
    const unsigned g = static_cast<unsigned>(mtiles_upper(a.P, a.E, 16 * NT)) * (groups / G);
    if (gemm1) dma_skinny_kernel<NT, 128, 6, true><<<g, kThreads, 0, s>>>(a, G);
    else dma_skinny_kernel<NT, 128, 6, false><<<g, kThreads, 0, s>>>(a, G);
    return hipGetLastError();
}

}  // namespace

const char* decode_kernel_name(const Bf16Args& a, bool gemm1) {
    return decode_kmajor(a, gemm1) ? "dma_kmajor_kernel" : "dma_skinny_kernel";
}

hipError_t launch_skinny_gemm1(const Bf16Args& a, hipStream_t s) { return launch_dma(a, true, s); }

hipError_t launch_skinny_gemm2(const Bf16Args& a, hipStream_t s) { return launch_dma(a, false, s); }

// ---------------------------------------------------------------------------
// Decode-shaped MX GEMMs: MX-fp8 activations ("Prime Flash MoE", section
// 7) against e2m1 weights ("GC-MoE on SM120", scale formats: a UE8M0
// exponent per 32 along K) or e4m3 weights. The same streaming design as
// above: weights on the MFMA's row side, a ring of stages filled by
// global->LDS DMA of whole row segments, one barrier per stage, k-major
// over a block's row groups (mx_kmajor_kernel). MFMA:
// v_mfma_scale_f32_32x32x64_f8f6f4 with the weights as A
// (e2m1: 16 contiguous bytes per lane, K values 32g..32g+31 of the 64-wide
// step, g = lane >> 5; e4m3: 16-byte chunks g and 2 + g of the step) and the
// e4m3 tokens as B (chunks g and 2 + g); lane group g supplies the scale of
// 32-block g (layouts measured on gfx950 with in-bounds probes).
//
// Stage (K step of KC = 512 values): R weight rows x 256 (e2m1) or 512
// (e4m3) bytes and each row's 16 scale bytes; R = 128 e2m1 rows or 64 e4m3
// rows make 32 KB of weights per stage. A token chunk is 32 rows x 512
// bytes and their scale bytes.
// Chunks are XOR-swizzled by the row over the row's chunks (^ (row & 15) or
// ^ (row & 31)), so the rows a fragment read touches hit distinct bank
// groups. Waves 0 .. R/64 - 1 also move the weight rows' scales, wave R/64
// the tokens'.
namespace {

// The same with one 16-byte chunk per k-step (e2m1 weights).
__device__ __forceinline__ void mxk_read4x1(u32x4_t (&w)[4], uint32_t (&sc)[4], const uint32_t (&aw)[4],
                                            const uint32_t (&as)[4]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_u8 %4, %12\n\t"
        "ds_read_u8 %5, %13\n\t"
        "ds_read_u8 %6, %14\n\t"
        "ds_read_u8 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]),
          "=&v"(sc[3])
        : "v"(aw[0]), "v"(aw[1]), "v"(aw[2]), "v"(aw[3]), "v"(as[0]), "v"(as[1]), "v"(as[2]), "v"(as[3])
        : "memory");
}


// Most row groups an MX k-major block keeps accumulators for at once (e2m1
// weights hold twice the token fragments, eight k-steps per wave). With at
// least four groups to a block, cutting them into super-groups of at most 7
// or 8 leaves at least four in each.
constexpr int mx_kmajor_groups(bool w4) { return w4 ? 7 : 8; }

// The MX decode GEMMs, k-major (the order of dma_kmajor_kernel): a block
// (m-tile, G row groups, G >= 4) walks K in 512-value chunks and, within a
// chunk, up to mx_kmajor_groups groups; a stage is one group's R weight rows
// (32 KB of e4m3 or e2m1 codes) and their scale bytes, in a 4-slot ring.
// The m-tile's token chunk (32 rows x 512 e4m3 codes and their scales) rides
// with the first stage of its chunk into one token slot, which the next
// chunk's DMA overwrites only four stages later (so every super-group has at
// least four groups). Each wave owns one 32-row block of a group (e2m1: R =
// 128, four blocks, all eight 64-value k-steps of a stage; e4m3: R = 64, two
// blocks, each wave half the k-steps, the halves summed in LDS at the end of
// a super-group) and keeps its token fragments in registers across the
// chunk's groups. GEMM1's group is R/2 act columns; within each 8 rows the
// first 4 are gate rows and the next 4 the up rows of the same columns, so an
// MFMA lane holding gate sums finds the up sums 32 lanes away, and each
// 32-row block yields 16 act columns (half an MX scale block: the two waves
// of a scale block swap their row maxima through LDS).
template <int R, bool W4, bool GEMM1>
__global__ __launch_bounds__(kThreads) void mx_kmajor_kernel(MxArgs a) {
    using C = Mx4<R, W4>;
    constexpr int SW = 4, NB = R / 32, KP = 4 / NB, NSK = 8 / KP;  // k-steps per wave per stage
    constexpr int GSM = mx_kmajor_groups(W4);
    constexpr int WSLOT = C::WB + R * 16;   // weight codes, then R scale rows of 16 bytes
    constexpr int TSLOT = C::TB + 64 * 16;  // token codes, then 32 scale rows (and a 512-byte pad)
    static_assert(NB * KP == 4 && NSK % 4 == 0, "four waves: row blocks x K parts");
    static_assert(SW * WSLOT + TSLOT + 2 * 4 * 32 * 4 <= 160 * 1024, "LDS of a CU");
    static_assert((SW - 2) * C::WINS < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) uint8_t lds[SW * WSLOT + TSLOT];
    __shared__ float xamax[2][4][32];  // GEMM1: per token, the act maximum of each wave's 16 columns
    uint8_t* const tslot = lds + SW * WSLOT;
    static_assert(kMx4BM == 32, "32-row m-tiles");
    DecodeWork wk;  // at least four row groups: every super-group then holds at least four
    MTile mt;
    if (!decode_lookup<4>(a.rv, a.E, GEMM1 ? a.H / (R / 2) : a.D / R, wk, mt)) return;
    const int G = wk.n, nsg = (G + GSM - 1) / GSM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rb = wave % NB, kp = wave / NB;
    const int lr = lane & 31, g = lane >> 5;
    const int K = GEMM1 ? a.D : a.H;
    const int KB = K / 32;  // scale bytes per row
    const int grp0 = wk.g0;
    const uint8_t* wbase = GEMM1 ? a.w1 : a.w2;
    const uint8_t* wsbase = GEMM1 ? a.w1s : a.w2s;
    auto wrow = [&](int r) -> int64_t {  // expert weight row of slot row r in group grp0
        if (GEMM1) {
            const int col = grp0 * (R / 2) + 16 * (r >> 5) + 4 * ((r & 31) >> 3) + (r & 3);
            return static_cast<int64_t>(mt.expert) * 2 * a.H + ((r & 4) ? a.H + col : col);
        }
        return static_cast<int64_t>(mt.expert) * a.D + grp0 * R + r;
    };
    const int64_t rowb = W4 ? K / 2 : K;  // weight row bytes
    // (arrays of a size that does not depend on the template arguments: the
    // host pass drops the kernel's launch stub when a lambda captures one
    // whose size does)
    constexpr int WINS = 8, TINS = 4;
    static_assert(C::WINS == WINS && C::TINS == TINS, "32 KB weight stages, 16 KB token chunks");
    const char* wsrc[WINS];
#pragma unroll
    for (int j = 0; j < C::WINS; ++j) {
        const int row = (wave * C::WINS + j) * C::WRPI + lane / C::WCH;
        const int c = (lane & (C::WCH - 1)) ^ (row & (C::WCH - 1));
        wsrc[j] = reinterpret_cast<const char*>(wbase) + wrow(row) * rowb + c * 16;
    }
    auto trow = [&](int m) -> int64_t {
        const int mm = m < mt.rows ? m : 0;
        if (GEMM1) return clamp_pair(a.rv.sorted_to_pair[mt.row0 + mm], a.P) / a.k;
        return mt.row0 + mm;
    };
    const uint8_t* tbase = GEMM1 ? a.x : a.act;
    const uint8_t* tsbase = GEMM1 ? a.xs : a.act_s;
    const char* tsrc[TINS];
#pragma unroll
    for (int j = 0; j < C::TINS; ++j) {
        const int m = (wave * C::TINS + j) * 2 + lane / 32;
        const int c = (lane & 31) ^ (m & 31);
        tsrc[j] = reinterpret_cast<const char*>(tbase) + trow(m) * K + c * 16;
    }
    // scale DMA: wave w < SWAVES lane i -> scale row of slot row 64w + i; wave SWAVES -> token row i & 31
    const char* ssrc = wave < C::SWAVES ? reinterpret_cast<const char*>(wsbase) + wrow(64 * wave + lane) * KB
                                        : reinterpret_cast<const char*>(tsbase) + trow(lane & 31) * KB;
    const int64_t wgroup_stride = static_cast<int64_t>(GEMM1 ? R / 2 : R) * rowb;
    const int64_t sgroup_stride = static_cast<int64_t>(GEMM1 ? R / 2 : R) * KB;
    const int KIT = K / kMx4KC, NIT = G * KIT;
    const int rot = GEMM1 ? 0 : static_cast<int>(blockIdx.x) % G;  // as in dma_skinny_kernel
    const int kc0 = static_cast<int>(blockIdx.x) % KIT;               // as in dma_kmajor_kernel
    const KmajorPlan pl{G / nsg, G % nsg, KIT};
    int ep = 0;
    float wt = 1.0f;
    if (!GEMM1) {
        ep = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (lr < mt.rows ? lr : 0)], a.P);
        wt = a.wts[ep];
        asm volatile("" : "+v"(ep), "+v"(wt));
    }
    auto issue = [&](int st) {
        int sg, kc, gi;
        pl.locate(st, sg, kc, gi);
        const int gr = (pl.first(sg) + gi + rot) % G;
        const int kr = (kc + kc0) % KIT;
        uint8_t* slot = lds + (st % SW) * WSLOT;
        const int64_t wb = static_cast<int64_t>(kr) * C::WRB + gr * wgroup_stride;
#pragma unroll
        for (int j = 0; j < C::WINS; ++j)
            __builtin_amdgcn_global_load_lds(wsrc[j] + wb, (lds_ptr_t)(slot + (wave * C::WINS + j) * 1024), 16, 0,
                                             kWeightDmaAux);
        if (wave < C::SWAVES)
            __builtin_amdgcn_global_load_lds(ssrc + static_cast<int64_t>(kr) * 16 + gr * sgroup_stride,
                                             (lds_ptr_t)(slot + C::WB + wave * 1024), 16, 0, 0);
        if (gi == 0) {
            const int64_t tb = static_cast<int64_t>(kr) * C::TRB;
#pragma unroll
            for (int j = 0; j < C::TINS; ++j)
                __builtin_amdgcn_global_load_lds(tsrc[j] + tb, (lds_ptr_t)(tslot + (wave * C::TINS + j) * 1024), 16,
                                                 0, 0);
            if (wave == C::SWAVES)
                __builtin_amdgcn_global_load_lds(ssrc + static_cast<int64_t>(kr) * 16, (lds_ptr_t)(tslot + C::TB), 16,
                                                 0, 0);
        }
    };
#pragma unroll
    for (int j = 0; j < SW - 1; ++j)
        if (j < NIT) issue(j);
    const int row = 32 * rb + lr;  // this lane's weight row in the slot
    int s = 0;
    for (int sg = 0; sg < nsg; ++sg) {
        const int gs = pl.size(sg), gfirst = pl.first(sg);
        f32x16_t acc[GSM];
#pragma unroll
        for (int gi = 0; gi < GSM; ++gi) acc[gi] = f32x16_t{};
        for (int kc = 0; kc < KIT; ++kc) {
            u32x4_t tlo[NSK], thi[NSK];
            uint32_t tsc[NSK];
#pragma unroll
            for (int gi = 0; gi < GSM; ++gi) {
                if (gi >= gs) continue;
                // the stage's DMAs (and at gi = 0 the chunk's token DMAs, issued after them) are this wave's
                // oldest; every later stage holds at least WINS
                if (s + SW - 2 < NIT) wait_vm<(SW - 2) * C::WINS>();
                else wait_vm<0>();
                ring_barrier();
                if (s + SW - 1 < NIT) issue(s + SW - 1);
                if (gi == 0) {
#pragma unroll
                    for (int h = 0; h < NSK / 4; ++h) {
                        uint32_t alo[4], ahi[4], as[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int ks = kp * NSK + 4 * h + i, ct = 4 * ks + g;
                            alo[i] = lds_addr(tslot + lr * C::TRB + ((ct ^ lr) << 4));
                            ahi[i] = lds_addr(tslot + lr * C::TRB + (((ct + 2) ^ lr) << 4));
                            as[i] = lds_addr(tslot + C::TB + lr * 16 + 2 * ks + g);
                        }
                        u32x4_t lo[4], hi[4];
                        uint32_t sc[4];
                        mxk_read4x2(lo, hi, sc, alo, ahi, as);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            tlo[4 * h + i] = lo[i];
                            thi[4 * h + i] = hi[i];
                            tsc[4 * h + i] = sc[i];
                        }
                    }
                }
                const uint8_t* slot = lds + (s % SW) * WSLOT;
#pragma unroll
                for (int h = 0; h < NSK / 4; ++h) {
                    uint32_t as[4], wsc[4];
                    i32x8_t aa[4];
                    if constexpr (W4) {
                        uint32_t aw[4];
                        u32x4_t w[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int ks = kp * NSK + 4 * h + i, cw = 2 * ks + g;
                            aw[i] = lds_addr(slot + row * C::WRB + ((cw ^ (row & (C::WCH - 1))) << 4));
                            as[i] = lds_addr(slot + C::WB + row * 16 + 2 * ks + g);
                        }
                        mxk_read4x1(w, wsc, aw, as);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            aa[i] = i32x8_t{(int)w[i].x, (int)w[i].y, (int)w[i].z, (int)w[i].w, 0, 0, 0, 0};
                    } else {
                        uint32_t alo[4], ahi[4];
                        u32x4_t wl[4], wh[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int ks = kp * NSK + 4 * h + i, ct = 4 * ks + g;
                            alo[i] = lds_addr(slot + row * C::WRB + ((ct ^ (row & (C::WCH - 1))) << 4));
                            ahi[i] = lds_addr(slot + row * C::WRB + (((ct + 2) ^ (row & (C::WCH - 1))) << 4));
                            as[i] = lds_addr(slot + C::WB + row * 16 + 2 * ks + g);
                        }
                        mxk_read4x2(wl, wh, wsc, alo, ahi, as);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            aa[i] = i32x8_t{(int)wl[i].x, (int)wl[i].y, (int)wl[i].z, (int)wl[i].w,
                                            (int)wh[i].x, (int)wh[i].y, (int)wh[i].z, (int)wh[i].w};
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 4 * h + i;
                        const i32x8_t bt{(int)tlo[t].x, (int)tlo[t].y, (int)tlo[t].z, (int)tlo[t].w,
                                         (int)thi[t].x, (int)thi[t].y, (int)thi[t].z, (int)thi[t].w};
                        acc[gi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aa[i], bt, acc[gi], W4 ? 4 : 0, 0, 0,
                                                                                 (int)wsc[i], 0, (int)tsc[t]);
                    }
                }
                ++s;
            }
        }
        // epilogue of the super-group (acc[gi][v]: token lr, slot row 32 rb + 8 (v / 4) + 4 g + v % 4); the
        // slot of the stage just consumed is free until the next stage's barrier
        const uint32_t red = lds_addr(lds + ((s - 1) % SW) * WSLOT);
#pragma unroll
        for (int gi = 0; gi < GSM; ++gi) {
            if (gi >= gs) continue;
            const int gidx = grp0 + (gfirst + gi + rot) % G;
            f32x16_t v = acc[gi];
            if constexpr (KP == 2) {
                lds_barrier();
                if (kp == 1) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) lds_store_f32(red + ((rb * 16 + q) * 64 + lane) * 4, v[q]);
                }
                lds_barrier();
                if (kp == 0) {
#pragma unroll
                    for (int q0 = 0; q0 < 16; q0 += 4) {
                        uint32_t p[4];
                        float o[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) p[i] = red + ((rb * 16 + q0 + i) * 64 + lane) * 4;
                        lds_load4_f32(o, p);
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[q0 + i] += o[i];
                    }
                }
            }
            if (GEMM1) {
                float up[16], act[16];
                float amax = 0.0f;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    up[q] = __shfl_xor(v[q], 32);
                    act[q] = v[q] / (1.0f + __expf(-v[q])) * up[q];
                    amax = fmaxf(amax, fabsf(act[q]));
                }
                const int buf = gi & 1;
                if (kp == 0 && g == 0) xamax[buf][rb][lr] = amax;
                lds_barrier();
                if (kp == 0 && g == 0 && lr < mt.rows) {
                    const int sc = mx_scale_exp(fmaxf(amax, xamax[buf][rb ^ 1][lr]));
                    const float inv = pow2f(-sc);
                    const int64_t trw = mt.row0 + lr;
                    const int col0 = gidx * (R / 2) + 16 * rb;  // act column v of this lane: col0 + v
                    uint32_t code[4];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        code[q4] = e4m3_encode(act[4 * q4] * inv, act[4 * q4]) |
                                   (e4m3_encode(act[4 * q4 + 1] * inv, act[4 * q4 + 1]) << 8) |
                                   (e4m3_encode(act[4 * q4 + 2] * inv, act[4 * q4 + 2]) << 16) |
                                   (e4m3_encode(act[4 * q4 + 3] * inv, act[4 * q4 + 3]) << 24);
                    *reinterpret_cast<uint4*>(a.act + trw * a.H + col0) = uint4{code[0], code[1], code[2], code[3]};
                    if ((rb & 1) == 0) a.act_s[trw * (a.H / 32) + col0 / 32] = static_cast<uint8_t>(sc + 127);
                }
            } else if (kp == 0 && lr < mt.rows) {
                uint16_t* dst = a.ypair + static_cast<int64_t>(ep) * a.D + gidx * R + 32 * rb + 4 * g;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<uint2*>(dst + 8 * q4) =
                        uint2{pack_bf16x2(v[4 * q4] * wt, v[4 * q4 + 1] * wt),
                              pack_bf16x2(v[4 * q4 + 2] * wt, v[4 * q4 + 3] * wt)};
            }
        }
    }
}

}  // namespace

bool decode_kernels_fit(int64_t T, int k, int E) {
    if (T <= 0 || k <= 0 || E <= 0 || k > E) return false;
    const double p = static_cast<double>(k) / E;
    if (static_cast<double>(T) * p > 32.0) return false;
    if (T <= 32) return true;
    if (p >= 1.0) return false;
    // upper tail of Binomial(T, p) from 33, summed in log space until it stops mattering
    const double lp = std::log(p), lq = std::log1p(-p);
    double tail = 0.0;
    for (int64_t x = 33; x <= T; ++x) {
        const double lpmf = std::lgamma(static_cast<double>(T) + 1) - std::lgamma(static_cast<double>(x) + 1) -
                            std::lgamma(static_cast<double>(T - x) + 1) + x * lp + (T - x) * lq;
        const double t = std::exp(lpmf);
        tail += t;
        if (t < 1e-12 * (tail + 1e-300) && x > 33 + 4 * std::sqrt(static_cast<double>(T) * p)) break;
    }
    return E * tail < 0.5;
}

// Decode-shaped MX GEMMs: few rows per expert (decode_kernels_fit), K (D for
// GEMM1, H for GEMM2) a multiple of the 512-value stage, and whole row
// groups (e2m1 weights: 128 rows per block, e4m3: 64).
bool skinny_mx_supported(const MxArgs& a) {
    const int R = a.w4 ? 128 : 64;
    return decode_kernels_fit(a.T, a.k, a.E) && a.D % kMx4KC == 0 && a.H % kMx4KC == 0 && a.H % (R / 2) == 0 &&
           a.D % R == 0;
}

const char* mx_decode_kernel_name(const MxArgs&, bool) { return "mx_kmajor_kernel"; }

hipError_t launch_skinny_mx(const MxArgs& a, bool gemm1, hipStream_t s) {
    // one block per CU, or one per m-tile when there can be more (decode_work)
    const unsigned g = static_cast<unsigned>(std::max(device_cu_count(), mtiles_upper(a.P, a.E, kMx4BM)));
    if (a.w4) {
        if (gemm1) mx_kmajor_kernel<128, true, true><<<g, kThreads, 0, s>>>(a);
        else mx_kmajor_kernel<128, true, false><<<g, kThreads, 0, s>>>(a);
    } else {
        if (gemm1) mx_kmajor_kernel<64, false, true><<<g, kThreads, 0, s>>>(a);
        else mx_kmajor_kernel<64, false, false><<<g, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
