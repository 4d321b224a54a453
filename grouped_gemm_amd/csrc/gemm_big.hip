// Prefill-shaped grouped GEMMs, bf16 and MX-fp8: many routed rows per expert.
//
// With hundreds to thousands of rows per expert the pass is bound by the
// matrix cores. A tile is BM token rows x 256 weight rows (GEMM1: 128 gate +
// 128 up rows, the gate/up pairing of "Prime Flash MoE", section 2, Trick 1;
// GEMM2: 256 output features). The weights are the MFMA's A operand, so each
// lane's results are 4 consecutive features of one token. Eight waves (two
// per SIMD) split a tile into two feature halves x four token groups: 128
// features x BM/4 tokens per wave.
//
// Formats. bf16: v_mfma_f32_32x32x16_bf16. MX-fp8 ("Prime Flash MoE",
// section 7: e4m3 codes with one e8m0 scale per 32 elements along K):
// v_mfma_scale_f32_32x32x64_f8f6f4; lane group g = lane >> 5 supplies codes
// k = 16g..16g+15 and 32+16g..32+16g+15 of a 64-code step (16-byte chunks g
// and 2+g) and the scale of 32-block g (layout measured on gfx950 with an
// in-bounds probe).
//
// Persistent schedule. One workgroup per CU walks a list of tiles. Workgroup
// b runs on XCD b % 8 (8 XCDs, each with its own L2); the logical tiles,
// n-tile fastest, are split into 8 contiguous ranges, and the workgroups of
// an XCD take every (workgroups per XCD)-th tile of that XCD's range, so the
// n-tiles sharing a token tile run side by side and reuse it from one L2.
//
// K stages. A stage holds 128 bytes of K per tile row (64 bf16 or 128 MX
// codes), so each row's piece of a stage is one whole 128-byte line; stages
// of 64 bytes, half a line per row, took twice the memory requests for the
// same bytes and ran 8-12% slower. Stages arrive by global->LDS DMA
// (global_load_lds_dwordx4: lane i's 16 bytes land at base + 16*i, 8 rows x
// 128 bytes per instruction; MX adds one dword DMA per wave with 64 rows'
// four scale bytes) into two stage buffers (2 x 64 KB for 256-row tiles):
// while stage kt is consumed, stage kt + 1 is in flight, and one barrier per
// stage guards both buffers (see ring_step). The ring runs on across tiles:
// the next tile's row map (and, for GEMM2, its routing weights) arrive by
// DMA during the current tile's first steps, and its first stage is issued
// during the current tile's last, so neither the tile lookup nor the first
// load's latency sits between two tiles. Results leave through a small
// per-wave LDS area as 64-byte row segments (see the epilogues).
//
// Swizzle: 16-byte chunk c of staged row r sits at chunk position
// c ^ ((r >> 1) & 7) of its 128-byte LDS row. gfx950's LDS serves 16 lanes
// of a 16-byte read per cycle from 64 banks; a fragment read has 16 lanes
// read the same chunk of 16 consecutive rows, the rows of one parity then
// take 8 distinct chunk positions and the two parities sit in different
// halves of the 256-byte bank row, so the 16 reads hit 16 distinct 16-byte
// bank groups. The waits are explicit per-wave vmcnt waits and the barrier
// carries no memory fence (a fence would wait for every DMA in flight).
//
// Token rows of GEMM1 are gathered on load (row r reads token
// sorted_to_pair[row0 + r] / k); rows past an expert's count read a valid
// row and are not stored.
#include <cstdlib>

#include "common.h"
#include "mxq.h"

namespace moe {

namespace {

constexpr int W = 8;               // waves per workgroup
constexpr int kThreads = 64 * W;
constexpr int RB = 128;            // bytes per tile row per stage
constexpr int BN = 256;            // weight rows per tile
// Result stores of rows past an expert's count go to a sink in the workspace
// instead of being skipped (see the epilogues): one area per wave of a
// workgroup slot, one 1 KB line per store of an epilogue.
constexpr int kSinkSlots = 8;
constexpr int kSinkWaveBytes = 16 * 1024;
constexpr int64_t kSinkBytes = int64_t(kSinkSlots) * W * kSinkWaveBytes;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// What both formats' kernels read and write. bf16: x, w1, w2 are bf16 and
// act is bf16 [P, H]; MX: they are e4m3 codes with e8m0 scales xs, w1s, w2s
// (one per 32 along K) and act is codes [P, H] with scales act_s [P, H/32].
struct BigArgs {
    int32_t T, D, H, E, k;
    int64_t P;
    const uint8_t* x;
    const uint8_t* xs;
    const uint8_t* w1;
    const uint8_t* w1s;
    const uint8_t* w2;
    const uint8_t* w2s;
    const float* wts;
    RouteView rv;
    uint8_t* act;
    uint8_t* act_s;
    uint16_t* ypair;
    uint8_t* sink;  // kSinkBytes
    ActVariant av;  // bf16 only; zero: the plain SwiGLU
    bool w4;        // MX: the weights are MXFP4 (packed e2m1, half the bytes per row)
};

template <bool MX>
struct Fmt {
    static constexpr int EB = MX ? 1 : 2;           // bytes per element
    static constexpr int kInfoCap = MX ? 128 : 512; // tile descriptors held in LDS at a time
};

template <int BM, bool MX>
struct Big {
    static constexpr int TB = BM / (W / 2);   // tokens per wave
    static constexpr int NT = TB / 32;        // token blocks per wave
    static constexpr int A_INS = BM / 8 / W;  // token-row DMA instructions per wave per stage (8 rows each)
    static constexpr int B_INS = BN / 8 / W;  // weight-row DMA instructions per wave per stage
    static constexpr int B_INS4 = BN / 16 / W; // the same for MXFP4 weights (64-byte rows: 16 rows each)
    static constexpr int PW = BM / 64;        // waves that move one BM-entry int/float vector (64 per wave)
    static_assert(NT >= 1 && A_INS >= 1 && A_INS * 8 * W == BM && B_INS * 8 * W == BN, "tile split");
    static_assert(B_INS % 2 == 0, "weight-row offsets alternate with the instruction's parity");
    static_assert(PW >= 1 && PW <= W, "row-vector DMA waves");
    // 16-byte result stores each wave issues per tile (epilogue_bf16, or the
    // code stores of epilogue_mx_gemm1)
    template <bool GEMM1>
    static constexpr int stores() { return NT * (GEMM1 ? (MX ? 2 : 4) : 8); }
    static_assert(stores<false>() * 1024 <= kSinkWaveBytes, "sink lines per wave");
    static_assert(!MX || BM / 64 + BN / 64 == W, "one scale-row DMA per wave");
};

// Both stage buffers in one object, token rows first: buffer 1's rows sit a
// fixed distance past buffer 0's, within a ds_read's immediate offset, so one
// address register serves a fragment row in both buffers. Buffers start on
// 1 KB boundaries, so a DMA instruction's 1 KB lands on whole 256-byte bank
// rows.
template <int BM>
struct StageBufs {
    uint8_t tok[2][BM * RB];
    uint8_t wt[2][BN * RB];
};

// MX: the scale dwords of one stage (one per token row and per weight row:
// the stage's four 32-blocks); one slot per stage buffer.
template <int BM>
struct ScaleSlot {
    uint32_t tok[BM];
    uint32_t wt[BN];
};

// Per-tile DMA sources: wave-uniform bases (scalar registers) plus 32-bit
// per-lane byte offsets. Token rows need one offset per instruction (they may
// be gathered); weight rows are consecutive and share an offset per
// instruction parity (Ring::boff0), which does not change from tile to tile.
template <int BM, bool MX>
struct DmaSrc {
    const char* abase;
    const char* bbase;
    uint32_t aoff[Big<BM, MX>::A_INS];
    const char* sbase;  // MX: scale rows of this wave (64 token or weight rows)
    uint32_t soff;
};

// A tile of this workgroup's list.
struct TileDesc {
    int expert, row0, rows, ntile;
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A wave-uniform pointer moved to scalar registers. readfirstlane returns a
// signed int: each half goes through uint32_t so the low half is not
// sign-extended into the high one.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v))));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v >> 32))));
    return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Global->LDS DMA instructions. They are written in assembly so that the
// compiler's wait-count insertion does not see an LDS write in flight: it
// cannot tell which stage buffer a DMA fills once the loop's back edge merges
// its state, and would then make the next fragment read wait for every DMA in
// flight, draining the ring. The explicit per-wave vmcnt waits below order
// the ring. M0 holds the LDS address; nothing else in these kernels uses M0.
// dma16: lane i's 16 bytes at sbase + voff land at lds + 16 * i.
// dma4:  lane i's 4 bytes at sbase + voff land at lds + 4 * i.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const char* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

// wait until at most n vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// the same, and also until this wave's LDS reads have returned
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// s_barrier without a memory fence; the asm statements stop the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Fragments in registers. bf16: one K quarter (16 elements) of all 4 weight
// and NT token fragments. MX: two weight fragments with their scale bytes;
// the token fragments of a K half are held once (TokFrag).
template <int BM, bool MX>
struct Frag;
template <int BM>
struct Frag<BM, false> {
    bf16x8_t w[4];
    bf16x8_t t[Big<BM, false>::NT];
};
template <int BM>
struct Frag<BM, true> {  // MX: two weight fragments with their scale bytes
    i32x8_t w[2];
    int sw[2];
};
// MX: the token fragments of a K half with their scale bytes.
template <int BM>
struct TokFrag {
    i32x8_t t[Big<BM, true>::NT];
    int st[Big<BM, true>::NT];
};

__device__ __forceinline__ i32x8_t frag32(const uint8_t* row, int lo, int hi) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(row + lo);
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(row + hi);
    return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
}

// Per-lane LDS offsets of the fragment rows and of chunk g = lane >> 5 of a
// row. bf16 quarter q (K elements 16q .. 16q + 15) reads chunk 2q + g; MX
// half h (codes 64h .. 64h + 63) reads chunks 4h + g and 4h + 2 + g, the
// lane layout of the scaled MFMA. Fragment rows start at multiples of 32, so
// the swizzle term s = ((lane & 31) >> 1) & 7 is the same for all of them,
// and chunk c + g (c even) sits at position c ^ g ^ s: the offset of chunk g
// with c << 4 XORed in. MX scale dwords of the rows sit at w / 32, t / 32.
struct LaneOff {
    int w, t;  // (first fragment row + (lane & 31)) * 128 of the weight and token rows
    int c0;    // position of chunk g, times 16
};

template <bool GEMM1>
__device__ __forceinline__ constexpr int frow_const(int f) {
    // GEMM1: gate rows 0..127 and up rows 128..255, a wave's 64 of each; GEMM2: 128 consecutive rows
    return GEMM1 ? (f < 2 ? 32 * f : 128 + 32 * (f - 2)) : 32 * f;
}

// bf16 fragment reads of quarter Q
template <int BM, bool GEMM1, int Q>
__device__ __forceinline__ void read_q(const uint8_t* tok, const uint8_t* wt, const LaneOff& o, Frag<BM, false>& f) {
    const int co = o.c0 ^ (Q << 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.w[i] = *reinterpret_cast<const bf16x8_t*>(wt + o.w + frow_const<GEMM1>(i) * RB + co);
#pragma unroll
    for (int i = 0; i < Big<BM, false>::NT; ++i) f.t[i] = *reinterpret_cast<const bf16x8_t*>(tok + o.t + 32 * i * RB + co);
}

// MX reads of K half H: weight fragments 2P, 2P + 1 with their scale bytes
// (32-block 2H + g of the stage: byte 2H + g of the row's scale dword), or
// the token fragments with theirs.
// W4: the weights are MXFP4, staged as 64-byte rows (128 e2m1 codes) with
// their four 16-byte chunks swizzled by ((row >> 2) & 3); the e2m1 operand
// takes 16 contiguous bytes per lane, K values 32g..32g+31 of the 64-wide
// step (chunk 2H + g), and the upper half of the operand is unused.
template <int BM, bool GEMM1, int H, int P, bool W4>
__device__ __forceinline__ void read_w_mx(const uint8_t* wt, const ScaleSlot<BM>& sc, const LaneOff& o,
                                          Frag<BM, true>& f) {
    const int g = (threadIdx.x & 63) >> 5;
    const int lo = o.c0 ^ (H << 6), hi = lo ^ 32;
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(sc.wt) + (o.w >> 5) + g;  // byte g of the row's dword
    // W4: row (o.w / 128) at (o.w / 2), chunk (2H + g) ^ ((row >> 2) & 3)
    const int c4 = ((2 * H + g) ^ (((threadIdx.x & 31) >> 2) & 3)) << 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int fr = frow_const<GEMM1>(2 * P + i);
        if constexpr (W4) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wt + (o.w >> 1) + fr * 64 + c4);
            f.w[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        } else {
            f.w[i] = frag32(wt + o.w + fr * RB, lo, hi);
        }
        f.sw[i] = sb[fr * 4 + 2 * H];
    }
}

template <int BM, int H>
__device__ __forceinline__ void read_t_mx(const uint8_t* tok, const ScaleSlot<BM>& sc, const LaneOff& o,
                                          TokFrag<BM>& f) {
    const int g = (threadIdx.x & 63) >> 5;
    const int lo = o.c0 ^ (H << 6), hi = lo ^ 32;
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(sc.tok) + (o.t >> 5) + g;
#pragma unroll
    for (int i = 0; i < Big<BM, true>::NT; ++i) {
        f.t[i] = frag32(tok + o.t + 32 * i * RB, lo, hi);
        f.st[i] = sb[32 * i * 4 + 2 * H];
    }
}

// Keeps the MX MFMAs where they are written: the empty asm makes the
// accumulators' new values needed at this point. Without it the compiler
// sinks the MFMAs of several steps past the barriers (their results are only
// read after the loop), and every fragment read in between stays live in
// registers: hundreds of spills. (The bf16 loop needs no such pin.)
template <int NT>
__device__ __forceinline__ void pin_acc(f32x16_t (&acc)[4][NT], int f0, int f1) {
#pragma unroll
    for (int f = f0; f < f1; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(acc[f][t]));
}

template <int BM>
__device__ __forceinline__ void mfma_half(const Frag<BM, false>& f, f32x16_t (&acc)[4][Big<BM, false>::NT]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < Big<BM, false>::NT; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[i], f.t[t], acc[i][t], 0, 0, 0);
}

// MFMAs of weight fragments 2P, 2P + 1 against the token fragments
template <int BM, int P, bool W4>
__device__ __forceinline__ void mfma_mx(const Frag<BM, true>& f, const TokFrag<BM>& tf,
                                        f32x16_t (&acc)[4][Big<BM, true>::NT]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < Big<BM, true>::NT; ++t)
            acc[2 * P + i][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                f.w[i], tf.t[t], acc[2 * P + i][t], W4 ? 4 : 0, 0, 0, f.sw[i], 0, tf.st[t]);
    pin_acc(acc, 2 * P, 2 * P + 2);
}

// Registers carried from one stage to the next. bf16: two quarters' fragment
// sets. MX: two weight-fragment pairs and the token fragments of one K half.
template <int BM, bool MX>
struct Regs;
template <int BM>
struct Regs<BM, false> {
    Frag<BM, false> x, y;
};
template <int BM>
struct Regs<BM, true> {
    Frag<BM, true> wa, wb;
    TokFrag<BM> t;
};

template <int BM, bool MX>
struct Ring {
    DmaSrc<BM, MX> src;  // this tile's DMA sources; from its last step on, the next tile's
    uint32_t bstride;  // bytes of 8 weight rows
    uint32_t wave;
    int KT;
    bool has_next, cont;
    TileDesc next;
    int nb;
};

// The lane index, recomputed where it is called: the empty volatile asm keeps
// the compiler from hoisting what the epilogues derive from it (addresses,
// the sink pointer, DMA offsets) out of the tile loop, where those values would hold
// registers through every K step and push the MX kernels into spills.
__device__ __forceinline__ int fresh_lane() {
    int lane = static_cast<int>(threadIdx.x & 63);
    asm volatile("" : "+v"(lane));
    return lane;
}

// DMA of a tile's row map: sorted_to_pair[row0 .. row0 + BM) -> pairs[0 .. BM).
// The map in the workspace is padded by 256 entries, so the window never
// leaves it; entries past the expert's rows are clamped before use.
template <int BM>
__device__ __forceinline__ void dma_row_map(const BigArgs& a, int row0, int32_t* pairs, uint32_t wave) {
    if (wave < static_cast<uint32_t>(BM / 64)) {
        const uint32_t lane = threadIdx.x & 63;
        dma4(uniform_ptr(a.rv.sorted_to_pair + row0), (wave * 64 + lane) * 4u, lds_addr(pairs) + wave * 256);
    }
}

// DMA of a tile's routing weights: wts[pair of row r] -> w[r] (GEMM2).
template <int BM>
__device__ __forceinline__ void dma_row_weights(const BigArgs& a, const int32_t* pairs, float* w, uint32_t wave) {
    if (wave < static_cast<uint32_t>(BM / 64)) {
        const int lane = threadIdx.x & 63;
        const int p = clamp_pair(pairs[wave * 64 + lane], a.P);
        dma4(uniform_ptr(a.wts), static_cast<uint32_t>(p) * 4u, lds_addr(w) + wave * 256);
    }
}

// Instruction j of a wave covers tile rows (wave * INS + j) * 8 + lane / 8;
// lane i's 16 bytes land at chunk position i & 7 of that row, so it fetches
// the global chunk that the swizzle puts there.
template <int BM, bool GEMM1, bool MX, bool W4>
__device__ __forceinline__ void make_src(const BigArgs& a, const TileDesc& t, const int32_t* pairs, uint32_t wave,
                                         DmaSrc<BM, MX>& s) {
    using C = Big<BM, MX>;
    constexpr int EB = Fmt<MX>::EB;
    const int64_t wrow = W4 ? (GEMM1 ? a.D : a.H) / 2 : (GEMM1 ? a.D : a.H) * EB;  // weight row bytes
    const int lane = fresh_lane();
    const int K = GEMM1 ? a.D : a.H;
    const int h0 = t.ntile * 128, n0 = t.ntile * 256;
    s.abase = uniform_ptr(GEMM1 ? a.x : a.act + static_cast<int64_t>(t.row0) * a.H * EB);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) {
        const int row = (static_cast<int>(wave) * C::A_INS + j) * 8 + lane / 8;
        const uint32_t r = GEMM1 ? static_cast<uint32_t>(clamp_pair(pairs[row], a.P) / a.k) * a.D
                                 : static_cast<uint32_t>(row < t.rows ? row : 0) * a.H;
        s.aoff[j] = r * EB + swz(row, lane & 7) * 16;
    }
    const int row0 = static_cast<int>(wave) * C::B_INS * 8;  // 32 weight rows per wave, never across gate/up
    const int64_t e2h = static_cast<int64_t>(t.expert) * 2 * a.H;
    if (GEMM1) {
        const int grow0 = row0 < 128 ? h0 + row0 : a.H + h0 + row0 - 128;
        s.bbase = uniform_ptr(a.w1 + (e2h + grow0) * wrow);
    } else {
        s.bbase = uniform_ptr(a.w2 + (static_cast<int64_t>(t.expert) * a.D + n0 + row0) * wrow);
    }
    if constexpr (MX) {
        // scale rows: waves 0 .. BM/64 - 1 take the token rows, the rest the weight rows
        const int KB = K / 32;
        if (wave < static_cast<uint32_t>(BM / 64)) {
            const int r = static_cast<int>(wave) * 64 + lane;
            if (GEMM1) {
                s.sbase = uniform_ptr(a.xs);
                s.soff = static_cast<uint32_t>(clamp_pair(pairs[r], a.P) / a.k) * KB;
            } else {
                s.sbase = uniform_ptr(a.act_s);
                s.soff = static_cast<uint32_t>(t.row0 + (r < t.rows ? r : 0)) * KB;
            }
        } else {
            const int r = (static_cast<int>(wave) - BM / 64) * 64 + lane;
            if (GEMM1) {
                const int grow = r < 128 ? h0 + r : a.H + h0 + r - 128;
                s.sbase = uniform_ptr(a.w1s);
                s.soff = static_cast<uint32_t>(e2h + grow) * KB;
            } else {
                s.sbase = uniform_ptr(a.w2s);
                s.soff = static_cast<uint32_t>(static_cast<int64_t>(t.expert) * a.D + n0 + r) * KB;
            }
        }
    }
}

template <int BM, bool MX, bool W4>
__device__ __forceinline__ void issue_stage(uint8_t* tok, uint8_t* wt, ScaleSlot<BM>* sc, const DmaSrc<BM, MX>& src,
                                            const Ring<BM, MX>& r, int kt) {
    using C = Big<BM, MX>;
    const char* ab = src.abase + kt * RB;
    const char* bb = src.bbase + kt * (W4 ? 64 : RB);
    const uint32_t tl = lds_addr(tok) + r.wave * (C::A_INS * 1024);
    const uint32_t wl = lds_addr(wt) + r.wave * ((W4 ? C::B_INS4 : C::B_INS) * 1024);
    const uint32_t lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) dma16(ab, src.aoff[j], tl + j * 1024);
    if constexpr (W4) {
        // weight row of instruction j: wave * 32 + 16j + lane / 4, 64 bytes; its
        // swizzle term ((row >> 2) & 3) is (lane >> 4) & 3 for every j.
        const uint32_t boff = (lane / 4) * (r.bstride / 16) + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
#pragma unroll
        for (int j = 0; j < C::B_INS4; ++j) dma16(bb, boff + j * r.bstride, wl + j * 1024);
    } else {
        // weight row of instruction j: wave * 8 * B_INS + 8j + lane / 8; with
        // B_INS even its swizzle term is 4 (j & 1) + lane / 16 (odd j: chunk ^ 4).
        // The offset is recomputed here rather than kept: registers are scarce.
        const uint32_t boff = (lane / 8) * (r.bstride / 8) + (((lane & 7) ^ (lane >> 4)) << 4);
#pragma unroll
        for (int j = 0; j < C::B_INS; ++j) dma16(bb, ((j & 1) ? boff ^ 64u : boff) + j * r.bstride, wl + j * 1024);
    }
    if constexpr (MX) {
        const uint32_t sl = r.wave < static_cast<uint32_t>(BM / 64) ? lds_addr(sc->tok) + r.wave * 256
                                                                     : lds_addr(sc->wt) + (r.wave - BM / 64) * 256;
        dma4(src.sbase, src.soff + kt * 4, sl);
    }
}

// One stage of the double-buffered ring:
//   wait for this wave's DMAs of stage kt and its LDS reads;  barrier
//   (FIRST) fetch the next tile's row map;  (SECOND) fetch its routing
//   weights;  issue stage kt + 1 into the other buffer (every wave is done
//   reading it: it held stage kt - 1)
//   bf16: read quarter 0;  MFMAs of quarter 3 of stage kt - 1;
//         read q1, MFMAs q0;  read q2, MFMAs q1;  read q3, MFMAs q2.
//   MX (units (K half, weight-fragment pair)): MFMAs of (1, 1) of stage
//         kt - 1;  read the tokens of half 0 and weights (0, 0), (0, 1);
//         MFMAs (0, 0);  read weights (1, 0);  MFMAs (0, 1);  read the
//         tokens of half 1 and weights (1, 1);  MFMAs (1, 0).
// The last unit's MFMAs move past the next barrier, so no wave comes out of
// it with nothing to compute; the reads and MFMAs are otherwise left to the
// compiler's schedule (forcing each read group ahead of the previous unit's
// MFMAs measured slower). Waits: a wave's vector-memory operations complete
// in issue order. In a tile's step 0 the previous tile's result stores (or
// the first tile's sink stores), issued after stage 0, may stay in flight;
// every later step waits for everything. Hand-over: step 0 fetches the next
// tile's row map (landed by step 1's barrier), step 1 its routing weights,
// and step KT - 1 builds its DMA sources and issues its stage 0.
// A wave whose token rows all lie past the tile's rows (`live` false: the
// short last m-tile of an expert) moves its share of the DMAs and keeps the
// barriers, but reads no fragments and issues no MFMAs; its accumulators stay
// zero and its epilogue stores go to the sink.
template <int BM, bool GEMM1, bool MX, bool VAR, bool W4, int B, bool FIRST, bool SECOND>
__device__ __forceinline__ void ring_step(const BigArgs& a, Ring<BM, MX>& r, StageBufs<BM>& L, ScaleSlot<BM>* sc,
                                          int kt, int32_t (*pairs)[BM], float (*wrow)[BM], const LaneOff& o,
                                          Regs<BM, MX>& g, f32x16_t (&acc)[4][Big<BM, MX>::NT], bool live) {
    // stage kt is in buffer B (B = kt & 1); stage kt + 1 goes into the other
    const uint8_t* ct = L.tok[B];
    const uint8_t* cw = L.wt[B];
    const ScaleSlot<BM>& csc = sc[MX ? B : 0];
    ScaleSlot<BM>* osc = &sc[MX ? B ^ 1 : 0];
    constexpr int S = Big<BM, MX>::template stores<GEMM1>();
    if (FIRST) wait_vm_lds<S>();
    else wait_vm_lds<0>();
    bare_barrier();
    if (FIRST && r.cont) dma_row_map<BM>(a, r.next.row0, pairs[r.nb], r.wave);
    if (SECOND && r.cont && (!GEMM1 || (VAR && a.av.wba))) dma_row_weights<BM>(a, pairs[r.nb], wrow[r.nb], r.wave);
    if (kt + 1 < r.KT) {
        issue_stage<BM, MX, W4>(L.tok[B ^ 1], L.wt[B ^ 1], osc, r.src, r, kt + 1);
    } else if (r.cont) {
        // the next tile's sources are built here, where they are used, so
        // they hold no registers through the tile's steps
        make_src<BM, GEMM1, MX, W4>(a, r.next, pairs[r.nb], r.wave, r.src);
        issue_stage<BM, MX, W4>(L.tok[B ^ 1], L.wt[B ^ 1], osc, r.src, r, 0);
    }
    if (!live) return;
    if constexpr (!MX) {
        read_q<BM, GEMM1, 0>(ct, cw, o, g.x);
        if (!FIRST) mfma_half<BM>(g.y, acc);
        read_q<BM, GEMM1, 1>(ct, cw, o, g.y);
        mfma_half<BM>(g.x, acc);
        read_q<BM, GEMM1, 2>(ct, cw, o, g.x);
        mfma_half<BM>(g.y, acc);
        read_q<BM, GEMM1, 3>(ct, cw, o, g.y);
        mfma_half<BM>(g.x, acc);
    } else {
        if (!FIRST) mfma_mx<BM, 1, W4>(g.wb, g.t, acc);
        read_t_mx<BM, 0>(ct, csc, o, g.t);
        read_w_mx<BM, GEMM1, 0, 0, W4>(cw, csc, o, g.wa);
        read_w_mx<BM, GEMM1, 0, 1, W4>(cw, csc, o, g.wb);
        mfma_mx<BM, 0, W4>(g.wa, g.t, acc);
        read_w_mx<BM, GEMM1, 1, 0, W4>(cw, csc, o, g.wa);
        mfma_mx<BM, 1, W4>(g.wb, g.t, acc);
        read_t_mx<BM, 1>(ct, csc, o, g.t);
        read_w_mx<BM, GEMM1, 1, 1, W4>(cw, csc, o, g.wb);
        mfma_mx<BM, 0, W4>(g.wa, g.t, acc);
    }
}

// Results of a tile. acc[f][t][4i + j] holds feature frow[f] + 8i +
// 4*(lane>>5) + j of token row tok_row0 + 32t + (lane & 31): a lane holds 8
// bytes of a bf16 row per register group. Each 32-row block goes through
// the wave's own 2 KB of LDS (row r at r * 64, its 16-byte chunk c at
// (c ^ ((r >> 2) & 3)) * 16: the writes and the 16-byte reads hit distinct
// banks) and leaves as 64-byte row segments, 4 lanes x 16 bytes each: a
// quarter of the write requests of storing the 8-byte pieces. The area is
// the wave's own, so no barrier is needed; LDS accesses of one wave complete
// in order.
//
// Every wave issues exactly Big::stores() 16-byte stores per tile with all
// lanes on: a lane whose row is past the tile's count writes into the wave's
// sink area instead (its row pointer moves there). The next tile's first
// waits count on that number.
__device__ __forceinline__ int stage_chunk_off(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

__device__ __forceinline__ uint8_t* wave_sink(const BigArgs& a, int lane) {
    return a.sink + ((blockIdx.x & (kSinkSlots - 1)) * W + (threadIdx.x >> 6)) * kSinkWaveBytes + lane * 16;
}

__device__ __forceinline__ void store16(void* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// The stores a wave's first tile finds in flight in place of a previous
// tile's: Big::stores() zero lines to its sink area.
template <int BM, bool GEMM1, bool MX>
__device__ __forceinline__ void sink_stores(const BigArgs& a) {
    uint8_t* sink = wave_sink(a, threadIdx.x & 63);
#pragma unroll
    for (int j = 0; j < Big<BM, MX>::template stores<GEMM1>(); ++j) store16(sink + 1024 * j, u32x4_t{0, 0, 0, 0});
}

// bf16 results: GEMM1 writes act = silu(gate) * up at act[row0 + row][h0 + col];
// GEMM2 (both formats) writes w * y at ypair[pair][n0 + feature].
template <int BM, bool GEMM1, bool MX, bool VAR>
__device__ __forceinline__ void epilogue_bf16(const BigArgs& a, const TileDesc& t, const int32_t* pairs,
                                              const float* w, int tok_row0, int wf, uint8_t* stg,
                                              const f32x16_t (&acc)[4][Big<BM, MX>::NT]) {
    using C = Big<BM, MX>;
    const int lane = fresh_lane();
    const int r = lane & 31, g = lane >> 5;
    const int rr = lane >> 2, c = lane & 3;  // staging reads: rows rr and rr + 16, chunk c
    const int rd0 = stage_chunk_off(rr, c), rd1 = stage_chunk_off(rr + 16, c);
    uint16_t* sink = reinterpret_cast<uint16_t*>(wave_sink(a, lane));
    // the activation variant (bf16 only; the VAR = false kernels keep the plain path)
    const bool variant = VAR && GEMM1 && !MX && a.av.on();
    const float alpha_e = variant && a.av.alpha ? a.av.alpha[t.expert] : 1.0f;
#pragma unroll
    for (int tb = 0; tb < C::NT; ++tb) {
        const int base = tok_row0 + 32 * tb;
        const bool ok0 = base + rr < t.rows, ok1 = base + rr + 16 < t.rows;
        uint16_t* d0;
        uint16_t* d1;
        if (GEMM1) {
            uint16_t* act = reinterpret_cast<uint16_t*>(a.act);
            d0 = act + static_cast<int64_t>(t.row0 + base + rr) * a.H + t.ntile * 128 + 64 * wf + 8 * c;
            d1 = d0 + static_cast<int64_t>(16) * a.H;
        } else {
            const int64_t col = t.ntile * 256 + 128 * wf + 8 * c;
            d0 = a.ypair + static_cast<int64_t>(clamp_pair(pairs[base + rr], a.P)) * a.D + col;
            d1 = a.ypair + static_cast<int64_t>(clamp_pair(pairs[base + rr + 16], a.P)) * a.D + col;
        }
        d0 = ok0 ? d0 : sink;
        d1 = ok1 ? d1 : sink;
        // GEMM2: the routing weight (1 when it went before the activation);
        // GEMM1 with the activation variant: its gate/up scale
        const float wt = GEMM1 ? (variant ? (a.av.wba ? alpha_e * w[base + r] : alpha_e) : 1.0f)
                               : ((VAR && a.av.wba) ? 1.0f : w[base + r]);
#pragma unroll
        for (int f = 0; f < (GEMM1 ? 2 : 4); ++f) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = acc[f][tb][4 * i + j];
                    if (GEMM1 && variant)
                        v[j] = act_variant(x, acc[f + 2][tb][4 * i + j], wt, a.av.kind, a.av.limit);
                    else
                        v[j] = GEMM1 ? x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)) * acc[f + 2][tb][4 * i + j]
                                     : x * wt;
                }
                *reinterpret_cast<uint2*>(stg + stage_chunk_off(r, i) + 8 * g) =
                    uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
            const u32x4_t q0 = *reinterpret_cast<const u32x4_t*>(stg + rd0);
            const u32x4_t q1 = *reinterpret_cast<const u32x4_t*>(stg + rd1);
            store16(d0 + 32 * f, q0);
            store16(d1 + 32 * f, q1);
        }
    }
}

// MX GEMM1 results: act = silu(gate) * up in fp32, requantized per 32 act
// columns by the MXQ rule ("Prime Flash MoE", section 7: the GEMM1
// epilogue quantizes act for GEMM2). A 32-column block of one token sits in
// lanes r and r + 32 (16 values each), so its amax takes one cross-lane
// swap. Codes of the wave's 64 act columns for 32 tokens (64 bytes per
// token) are staged and leave as 64-byte row segments; each token's two
// scale bytes leave as one 2-byte store.
template <int BM>
__device__ __forceinline__ void epilogue_mx_gemm1(const BigArgs& a, const TileDesc& t, int tok_row0, int wf,
                                                  uint8_t* stg, const f32x16_t (&acc)[4][Big<BM, true>::NT]) {
    using C = Big<BM, true>;
    const int lane = fresh_lane();
    const int r = lane & 31, g = lane >> 5;
    const int rr = lane >> 2, c = lane & 3;
    const int rd0 = stage_chunk_off(rr, c), rd1 = stage_chunk_off(rr + 16, c);
    const int HB = a.H / 32;
    const int col0 = t.ntile * 128 + 64 * wf;  // first act column of this wave
    uint8_t* sink = wave_sink(a, lane);
#pragma unroll
    for (int tb = 0; tb < C::NT; ++tb) {
        const int base = tok_row0 + 32 * tb;
        uint32_t sbytes = 0;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            float v[16];
            float amax = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float x = acc[f][tb][q];
                v[q] = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)) * acc[f + 2][tb][q];
                amax = fmaxf(amax, fabsf(v[q]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int s = mx_scale_exp(amax);
            const float inv = pow2f(-s);
            sbytes |= static_cast<uint32_t>(s + 127) << (8 * f);
            // act column 32f + 8i + 4g + j of the wave: 16-byte chunk 2f + (i >> 1), byte 8(i & 1) + 4g + j
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t code = e4m3_encode(v[4 * i] * inv, v[4 * i]) |
                                      (e4m3_encode(v[4 * i + 1] * inv, v[4 * i + 1]) << 8) |
                                      (e4m3_encode(v[4 * i + 2] * inv, v[4 * i + 2]) << 16) |
                                      (e4m3_encode(v[4 * i + 3] * inv, v[4 * i + 3]) << 24);
                *reinterpret_cast<uint32_t*>(stg + stage_chunk_off(r, 2 * f + (i >> 1)) + 8 * (i & 1) + 4 * g) = code;
            }
        }
        if (g == 0 && base + r < t.rows)
            *reinterpret_cast<uint16_t*>(a.act_s + static_cast<int64_t>(t.row0 + base + r) * HB + col0 / 32) =
                static_cast<uint16_t>(sbytes);
        const u32x4_t q0 = *reinterpret_cast<const u32x4_t*>(stg + rd0);
        const u32x4_t q1 = *reinterpret_cast<const u32x4_t*>(stg + rd1);
        uint8_t* d0 = a.act + static_cast<int64_t>(t.row0 + base + rr) * a.H + col0 + 16 * c;
        uint8_t* d1 = d0 + static_cast<int64_t>(16) * a.H;
        store16(base + rr < t.rows ? d0 : sink, q0);
        store16(base + rr + 16 < t.rows ? d1 : sink, q1);
    }
}

// Descriptors of this workgroup's tiles c0 .. c0 + CAP - 1 into LDS.
template <int CAP>
__device__ __forceinline__ void load_descs(const int4* mtiles, int first, int stride, int ny, int count, int c0,
                                           TileDesc* desc) {
    for (int i = threadIdx.x; i < CAP && c0 + i < count; i += kThreads) {
        const int logical = first + (c0 + i) * stride;
        const int m = logical / ny;
        const int4 d = mtiles[m];
        desc[i] = TileDesc{d.x, d.y, d.z, logical - m * ny};
    }
}

__device__ __forceinline__ TileDesc uniform_desc(const TileDesc& d) {
    return TileDesc{uniform_int(d.expert), uniform_int(d.row0), uniform_int(d.rows), uniform_int(d.ntile)};
}

template <int BM, bool GEMM1, bool MX, bool VAR, bool W4>
__global__ __launch_bounds__(kThreads, 1) void big_gemm_kernel(BigArgs a, const int4* __restrict__ mtiles) {
    using C = Big<BM, MX>;
    constexpr int CAP = Fmt<MX>::kInfoCap;
    __shared__ __attribute__((aligned(1024))) StageBufs<BM> L;
    __shared__ __attribute__((aligned(16))) int32_t sPair[2][BM];
    __shared__ __attribute__((aligned(16))) float sW[2][BM];
    __shared__ TileDesc sDesc[CAP];
    __shared__ __attribute__((aligned(16))) uint8_t sOut[W][2048];  // per-wave result staging
    __shared__ __attribute__((aligned(16))) ScaleSlot<BM> sSc[MX ? 2 : 1];  // MX: the scale slots of buffers 0, 1

    const int ny = GEMM1 ? a.H / 128 : a.D / 256;
    const int total = a.rv.tile_prefix[tile_height_index(BM) * (a.E + 1) + a.E] * ny;
    const int per = (total + 7) / 8;
    const int xcd = blockIdx.x & 7, stride = gridDim.x >> 3;
    const int first = xcd * per + (blockIdx.x >> 3);
    const int end = min(total, (xcd + 1) * per);
    const int count = first < end ? (end - first + stride - 1) / stride : 0;
    if (count == 0) return;

    const int tid = threadIdx.x, wave_v = tid >> 6;
    const int wtok = wave_v >> 1, wf = wave_v & 1;
    const int tok_row0 = wtok * C::TB;
    LaneOff o;
    {
        const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
        const int wrow0 = (GEMM1 ? 64 : 128) * wf;
        o.w = (wrow0 + lr) * RB;
        o.t = (tok_row0 + lr) * RB;
        o.c0 = swz(lr, g) << 4;
    }

    Ring<BM, MX> r;
    r.wave = static_cast<uint32_t>(uniform_int(wave_v));
    const int K = GEMM1 ? a.D : a.H;
    r.KT = K * Fmt<MX>::EB / RB;
    // bytes between the first rows of consecutive weight DMA instructions
    r.bstride = W4 ? 16u * (K / 2) : 8u * K * Fmt<MX>::EB;

    load_descs<CAP>(mtiles, first, stride, ny, count, 0, sDesc);
    __syncthreads();
    TileDesc t = uniform_desc(sDesc[0]);
    int cb = 0;
    dma_row_map<BM>(a, t.row0, sPair[0], r.wave);
    wait_vm<0>();
    bare_barrier();
    make_src<BM, GEMM1, MX, W4>(a, t, sPair[0], r.wave, r.src);
    if (!GEMM1 || (VAR && a.av.wba)) {
        dma_row_weights<BM>(a, sPair[0], sW[0], r.wave);
        wait_vm<0>();
        bare_barrier();
    }
    issue_stage<BM, MX, W4>(L.tok[0], L.wt[0], &sSc[0], r.src, r, 0);
    sink_stores<BM, GEMM1, MX>(a);

    Regs<BM, MX> g;
    f32x16_t acc[4][C::NT];
    for (int i = 0; i < count; ++i) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int tb = 0; tb < C::NT; ++tb) acc[f][tb] = f32x16_t{};
        r.has_next = i + 1 < count;
        r.nb = cb ^ 1;
        if (r.has_next) {
            if ((i + 1) % CAP == 0) {  // next descriptor chunk; t stays in registers
                __syncthreads();
                load_descs<CAP>(mtiles, first, stride, ny, count, i + 1, sDesc);
                __syncthreads();
            }
            r.next = uniform_desc(sDesc[(i + 1) % CAP]);
        }
        r.cont = r.has_next;
        const bool live = uniform_int(tok_row0 < t.rows ? 1 : 0) != 0;

        // KT is even: every tile starts in buffer 0
        ring_step<BM, GEMM1, MX, VAR, W4, 0, true, false>(a, r, L, sSc, 0, sPair, sW, o, g, acc, live);
        ring_step<BM, GEMM1, MX, VAR, W4, 1, false, true>(a, r, L, sSc, 1, sPair, sW, o, g, acc, live);
        for (int kt = 2; kt < r.KT; kt += 2) {
            ring_step<BM, GEMM1, MX, VAR, W4, 0, false, false>(a, r, L, sSc, kt, sPair, sW, o, g, acc, live);
            ring_step<BM, GEMM1, MX, VAR, W4, 1, false, false>(a, r, L, sSc, kt + 1, sPair, sW, o, g, acc, live);
        }
        // the last unit of the last stage
        if (live) {
            if constexpr (MX) mfma_mx<BM, 1, W4>(g.wb, g.t, acc);
            else mfma_half<BM>(g.y, acc);
        }

        if constexpr (GEMM1 && MX) epilogue_mx_gemm1<BM>(a, t, tok_row0, wf, sOut[wave_v], acc);
        else epilogue_bf16<BM, GEMM1, MX, VAR>(a, t, sPair[cb], sW[cb], tok_row0, wf, sOut[wave_v], acc);
        if (!r.has_next) break;
        t = r.next;
        cb ^= 1;
    }
}

// One m-tile descriptor per tile of height BM: {expert, first sorted row,
// rows, 0}, in tile order. One workgroup per expert.
template <int BM>
__global__ void mtile_table_kernel(RouteView rv, int E, int4* __restrict__ out) {
    const int e = blockIdx.x;
    const int32_t* tp = rv.tile_prefix + tile_height_index(BM) * (E + 1);
    const int t0 = tp[e], n = tp[e + 1] - t0;
    const int off = rv.offsets[e], cnt = rv.counts[e];
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int m0 = i * BM;
        out[t0 + i] = int4{e, off + m0, cnt - m0 < BM ? cnt - m0 : BM, 0};
    }
}

// One workgroup per CU (a multiple of 8: the same number on every XCD),
// never many more than there can be tiles. MOE_FFN_GRID_LIMIT=n caps it at n
// (rounded up to a multiple of 8), e.g. to leave CUs to other work or to give
// each workgroup many tiles.
int big_grid(int64_t P, int E, int bm, int ny) {
    const int64_t tiles_upper = ((P + bm - 1) / bm + E) * ny;
    int64_t grid = device_cu_count();
    if (const char* lim = std::getenv("MOE_FFN_GRID_LIMIT")) {
        const long v = std::strtol(lim, nullptr, 10);
        if (v > 0 && v < grid) grid = v;
    }
    if (grid > tiles_upper) grid = tiles_upper;
    return static_cast<int>((grid + 7) / 8 * 8);
}

template <int BM, bool MX>
hipError_t launch_big(const BigArgs& a, int4* tiles, bool gemm1, hipStream_t s) {
    if (gemm1) mtile_table_kernel<BM><<<a.E, 64, 0, s>>>(a.rv, a.E, tiles);  // the same m-tiles for both GEMMs
    const int g = big_grid(a.P, a.E, BM, gemm1 ? a.H / 128 : a.D / 256);
    if constexpr (MX) {
        if (a.w4) {
            if (gemm1) big_gemm_kernel<BM, true, true, false, true><<<g, kThreads, 0, s>>>(a, tiles);
            else big_gemm_kernel<BM, false, true, false, true><<<g, kThreads, 0, s>>>(a, tiles);
        } else {
            if (gemm1) big_gemm_kernel<BM, true, true, false, false><<<g, kThreads, 0, s>>>(a, tiles);
            else big_gemm_kernel<BM, false, true, false, false><<<g, kThreads, 0, s>>>(a, tiles);
        }
    } else {
        const bool var = a.av.on();  // the activation variant has kernels of its own
        if (gemm1) {
            if (var) big_gemm_kernel<BM, true, false, true, false><<<g, kThreads, 0, s>>>(a, tiles);
            else big_gemm_kernel<BM, true, false, false, false><<<g, kThreads, 0, s>>>(a, tiles);
        } else {
            if (var) big_gemm_kernel<BM, false, false, true, false><<<g, kThreads, 0, s>>>(a, tiles);
            else big_gemm_kernel<BM, false, false, false, false><<<g, kThreads, 0, s>>>(a, tiles);
        }
    }
    return hipGetLastError();
}

}  // namespace

int device_cu_count() {
    static const int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        return v;
    }();
    return n;
}

// Average rows per expert at or above which the 256-row tile is used: bf16
// from 128 (an expert of 128-256 rows then takes one 256-row tile instead of
// two 128-row tiles that each stream all its weights: 7% faster at 256 rows
// per expert, 6% at 128; at 64 rows per expert the 128-row tile is 20%
// faster). MX has only
// the 256-row tile here and takes it from 128 rows per expert (the generic
// MX kernels below that): measured 28-38% faster than the generic kernels at
// 192-384 rows per expert, within 3% at 48-96.
constexpr int64_t kBigTile256MinRowsBf16 = 128;
constexpr int64_t kBigMxMinRows = 128;

int64_t big_gemm_mtile_capacity(int64_t P, int E) { return (P + 127) / 128 + E; }

namespace {
int64_t table_bytes(int64_t P, int E) { return (16 * big_gemm_mtile_capacity(P, E) + 255) / 256 * 256; }
uint8_t* sink_of(int32_t* mtiles, int64_t P, int E) { return reinterpret_cast<uint8_t*>(mtiles) + table_bytes(P, E); }
}  // namespace

int64_t big_gemm_workspace_bytes(int64_t P, int E) { return table_bytes(P, E) + kSinkBytes; }

bool big_gemm_supported(const Bf16Args& a) {
    const int64_t lim = int64_t(1) << 32;  // the DMA offsets are 32-bit
    return a.mtiles != nullptr && a.D % 256 == 0 && a.H % 128 == 0 && int64_t(a.T) * a.D * 2 < lim &&
           a.P * a.H * 2 < lim && a.P * 4 < lim && int64_t(2) * a.H * a.D * 2 < lim;
}

int big_gemm_tile_rows(const Bf16Args& a) { return a.P >= kBigTile256MinRowsBf16 * a.E ? 256 : 128; }

hipError_t launch_big_gemm(const Bf16Args& b, bool gemm1, hipStream_t s) {
    BigArgs a{b.T, b.D, b.H, b.E, b.k, b.P,
              reinterpret_cast<const uint8_t*>(b.x), nullptr,
              reinterpret_cast<const uint8_t*>(b.w1), nullptr,
              reinterpret_cast<const uint8_t*>(b.w2), nullptr,
              b.wts, b.rv, reinterpret_cast<uint8_t*>(b.act), nullptr, b.ypair, sink_of(b.mtiles, b.P, b.E), b.av};
    int4* tiles = reinterpret_cast<int4*>(b.mtiles);
    if (big_gemm_tile_rows(b) == 256) return launch_big<256, false>(a, tiles, gemm1, s);
    return launch_big<128, false>(a, tiles, gemm1, s);
}

// MX: 256-row tiles only (eight waves move the 512 scale rows of a stage);
// a tile takes an even number of K stages of 128 codes (D and H multiples of 256).
bool big_mx_supported(const MxArgs& a) {
    const int64_t lim = int64_t(1) << 32;
    return a.mtiles != nullptr && a.P >= kBigMxMinRows * a.E && a.D % 256 == 0 && a.H % 256 == 0 &&
           int64_t(a.T) * a.D < lim && a.P * a.H < lim && a.P * 4 < lim && int64_t(a.E) * 2 * a.H * a.D < lim;
}

hipError_t launch_big_mx(const MxArgs& b, bool gemm1, hipStream_t s) {
    BigArgs a{b.T,   b.D,   b.H,     b.E,  b.k,  b.P,      b.x,     b.xs,    b.w1,
              b.w1s, b.w2,  b.w2s,   b.wts, b.rv, b.act,   b.act_s, b.ypair, sink_of(b.mtiles, b.P, b.E)};
    a.w4 = b.w4;
    return launch_big<256, true>(a, reinterpret_cast<int4*>(b.mtiles), gemm1, s);
}

}  // namespace moe
