// Pieces shared by the streaming kernels that fill an LDS ring with
// global->LDS DMA: the decode-shaped GEMMs (gemm_skinny.hip) and the fused
// pass (gemm_fused.hip). Everything here sits in an anonymous namespace, so
// each translation unit holds its own copy.
#pragma once

#include <cmath>

#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32 x 32 x 16: lane l holds A row (and B column) l % 32, k = 8 (l / 32) .. + 7;
// result v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
// Cache policy bits of the weight DMA: 2 = nontemporal (each weight byte is
// streamed once).
constexpr int kWeightDmaAux = 2;

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


__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// Eight 16-byte LDS reads and a wait for them, in one asm statement (as
// lds_read6, so that no vmcnt wait for the DMAs in flight comes before them).
__device__ __forceinline__ void lds_read8(bf16x8_t (&v)[8], const uint32_t (&p)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}

// Four 16-byte LDS reads and a wait for them, as asm (see lds_read8).
__device__ __forceinline__ void lds_read4(bf16x8_t (&f)[4], const uint32_t (&p)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
        : "memory");
}

// Plain LDS loads of four floats, written as asm: the compiler, which cannot
// tell an LDS tile from the ring slots DMAs are filling, would put a
// vmcnt(0) wait (draining the ring, and any atomics in flight) before its
// own accesses.
__device__ __forceinline__ void lds_load4_f32(float (&v)[4], const uint32_t (&p)[4]) {
    asm volatile(
        "ds_read_b32 %0, %4\n\t"
        "ds_read_b32 %1, %5\n\t"
        "ds_read_b32 %2, %6\n\t"
        "ds_read_b32 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
        : "memory");
}

// An 8-byte LDS store, written as asm (see lds_load4_f32).
__device__ __forceinline__ void lds_write_b64(uint32_t addr, uint32_t lo, uint32_t hi) {
    asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(uint2{lo, hi}) : "memory");
}

// ---- MX decode geometry (mx_kmajor_kernel, the fused MX kernel) ----
constexpr int kMx4KC = 512;   // K values per stage
constexpr int kMx4BM = 32;    // token rows per m-tile

template <int R, bool W4>
struct Mx4 {
    static constexpr int WRB = W4 ? kMx4KC / 2 : kMx4KC;  // weight bytes per row per stage (256 or 512)
    static constexpr int WCH = WRB / 16;              // 16-byte chunks per weight row per stage
    static constexpr int WRPI = 64 / WCH;             // weight rows per DMA instruction
    static constexpr int TRB = kMx4KC;                // token bytes per row per stage (512)
    static constexpr int WB = R * WRB;                // 32 KB
    static constexpr int TB = kMx4BM * TRB;           // 16 KB
    static constexpr int WINS = WB / 1024 / 4;        // weight DMA instructions per wave per stage
    static constexpr int TINS = TB / 1024 / 4;        // token DMA instructions per wave per chunk
    static constexpr int SWAVES = R / 64;             // waves that move weight scale rows
};

// Four k-steps' operands from LDS and a wait for them: two 16-byte chunks
// and one scale byte each (e4m3 weights, or the token fragments); asm for
// the same reason as lds_read8.
__device__ __forceinline__ void mxk_read4x2(u32x4_t (&lo)[4], u32x4_t (&hi)[4], uint32_t (&sc)[4],
                                            const uint32_t (&alo)[4], const uint32_t (&ahi)[4],
                                            const uint32_t (&as)[4]) {
    asm volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %13\n\t"
        "ds_read_b128 %2, %14\n\t"
        "ds_read_b128 %3, %15\n\t"
        "ds_read_b128 %4, %16\n\t"
        "ds_read_b128 %5, %17\n\t"
        "ds_read_b128 %6, %18\n\t"
        "ds_read_b128 %7, %19\n\t"
        "ds_read_u8 %8, %20\n\t"
        "ds_read_u8 %9, %21\n\t"
        "ds_read_u8 %10, %22\n\t"
        "ds_read_u8 %11, %23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
          "=&v"(hi[3]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3])
        : "v"(alo[0]), "v"(alo[1]), "v"(alo[2]), "v"(alo[3]), "v"(ahi[0]), "v"(ahi[1]), "v"(ahi[2]), "v"(ahi[3]),
          "v"(as[0]), "v"(as[1]), "v"(as[2]), "v"(as[3])
        : "memory");
}
// A plain LDS store of a float in a ring slot, written as asm (as
// lds_load4_f32: the compiler would drain the ring before its own access).
__device__ __forceinline__ void lds_store_f32(uint32_t addr, float v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// A 32-row m-tile found by one wave, its lanes reading the route step's tile
// prefix sums in parallel. A decode block starts with a chain of dependent
// loads, and a binary search over the experts' tile counts adds log2(E) of
// them; here the lookup is one round of loads (two from 64 experts on), then
// the expert's row count and offset. Lane l holds the sample tp[min(l S, E)],
// S = 1 below 64 experts, else ceil((E + 1) / 64), so the second round's 64
// lanes cover one sample's segment while E < 4096 (kWaveLookupMaxExperts);
// every lane ends with the same result.
constexpr int kWaveLookupMaxExperts = 4095;

struct TileSamples {
    int v, S, M;  // this lane's sample, the sample stride, the m-tile count tp[E]
};

__device__ __forceinline__ TileSamples tile_samples(const RouteView& rv, int E, int lane) {
    const int32_t* tp = rv.tile_prefix + tile_height_index(32) * (E + 1);
    TileSamples s;
    s.S = E < 64 ? 1 : (E + 64) / 64;
    s.v = tp[lane * s.S < E ? lane * s.S : E];
    s.M = tp[E];
    return s;
}

// m-tile g (0 <= g < s.M) of the samples' route.
__device__ __forceinline__ void find_mtile_wave(const RouteView& rv, int E, const TileSamples& s, int g, int lane,
                                                MTile& t) {
    const int32_t* tp = rv.tile_prefix + tile_height_index(32) * (E + 1);
    // tp is non-decreasing with tp[0] = 0 <= g < tp[E]: the expert is the last
    // e < E with tp[e] <= g
    int e = 63 - __clzll(__ballot(lane * s.S < E && s.v <= g));
    int tpe = __shfl(s.v, e);
    if (s.S > 1) {
        const int e0 = e * s.S, j = e0 + lane;
        const int v2 = lane < s.S && j < E ? tp[j] : 0x7fffffff;
        const int l2 = 63 - __clzll(__ballot(v2 <= g));
        e = e0 + l2;
        tpe = __shfl(v2, l2);
    }
    t.expert = e;
    t.m0 = (g - tpe) * 32;
    const int c = rv.counts[e];
    t.rows = c - t.m0 < 32 ? c - t.m0 : 32;
    t.row0 = rv.offsets[e] + t.m0;
}

// 32-row m-tiles expected for T tokens with k routes each over E experts,
// routes spread uniformly: the experts hit, each with ceil(rows / 32) tiles.
inline double expected_mtiles32(int64_t T, int k, int E) {
    const double hit = E * (1.0 - std::pow(1.0 - static_cast<double>(k) / E, static_cast<double>(T)));
    const double per = std::ceil(static_cast<double>(T) * k / E / 32.0);
    return hit * (per > 1.0 ? per : 1.0);
}

}  // namespace

}  // namespace moe
