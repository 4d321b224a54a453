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
// Formats. bf16: v_mfma_f32_32x32x16_bf16, 32 elements of K per stage.
// MX-fp8 ("Prime Flash MoE", section 7: e4m3 codes with one e8m0 scale per
// 32 elements along K): v_mfma_scale_f32_32x32x64_f8f6f4, 64 codes of K per
// stage, so a staged row holds 64 bytes in both formats. For the scaled
// MFMA, lane group g = lane >> 5 supplies codes k = 16g..16g+15 and
// 32+16g..32+16g+15 of the 64 (the row's 16-byte chunks g and 2+g) and the
// scale of 32-block g (layout measured on gfx950 with an in-bounds probe).
//
// Persistent schedule. One workgroup per CU walks a list of tiles. Workgroup
// b runs on XCD b % 8 (8 XCDs, each with its own L2); the logical tiles,
// n-tile fastest, are split into 8 contiguous ranges, and the workgroups of
// an XCD take every (workgroups per XCD)-th tile of that XCD's range, so the
// n-tiles sharing a token tile run side by side and reuse it from one L2.
//
// K stages go through a ring of 4 LDS buffers filled by global->LDS DMA
// (global_load_lds_dwordx4: lane i's 16 bytes land at base + 16*i; 16 rows x
// 64 bytes per instruction; MX adds one dword DMA per wave with 64 rows'
// scale bytes): three stages are in flight while one is consumed, and the
// one barrier per stage sits between the MFMAs of the stage's two halves
// (see ring_step). The ring runs on across tiles: the next tile's row map
// (and, for GEMM2, its routing weights) arrive by DMA during the current
// tile's first steps, and its first four stages are issued during the
// current tile's last four, so neither the tile lookup nor the first loads'
// latency sits between two tiles. Results leave through a small per-wave LDS
// area as 64-byte row segments (see the epilogues).
//
// The 16-byte chunks of a staged row are XOR-swizzled by ((row >> 2) & 3):
// gfx950's LDS serves 16 lanes of a 16-byte read per cycle from 64 banks, and
// the 16 consecutive rows a fragment read touches then fall in 16 distinct
// 16-byte bank groups. The four stages are distinct LDS objects and the loop
// is unrolled by four. The waits are explicit per-wave vmcnt budgets and the
// barrier carries no memory fence (a fence would wait for every DMA in
// flight).
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
constexpr int RB = 64;             // bytes per tile row per stage
constexpr int BN = 256;            // weight rows per tile
constexpr int kMinPipelinedKT = 8; // K stages a tile needs for the in-loop hand-over
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
};

template <bool MX>
struct Fmt {
    static constexpr int EB = MX ? 1 : 2;           // bytes per element
    static constexpr int KS = RB / EB;              // K elements per stage
    static constexpr int kInfoCap = MX ? 128 : 512; // tile descriptors held in LDS at a time
};

template <int BM, bool MX>
struct Big {
    static constexpr int TB = BM / (W / 2);    // tokens per wave
    static constexpr int NT = TB / 32;         // token blocks per wave
    static constexpr int NF = 4;               // feature blocks per wave (128 features)
    static constexpr int A_INS = BM / 16 / W;  // token-row DMA instructions per wave per stage
    static constexpr int B_INS = BN / 16 / W;  // weight-row DMA instructions per wave per stage
    static constexpr int L = A_INS + B_INS;    // code DMA instructions per wave per stage
    // MX adds one scale DMA per wave on even stages (its dword covers the
    // stage pair). Outstanding operations younger than a stage kt when the
    // next one, two or three stages are in flight: any two consecutive
    // stages hold one even stage.
    static constexpr int Y1 = L;
    static constexpr int Y2 = 2 * L + (MX ? 1 : 0);
    static constexpr int Y3 = 3 * L + (MX ? 1 : 0);
    static constexpr int PW = BM / 64;         // waves that move one BM-entry int/float vector (64 per wave)
    static_assert(NT >= 1 && A_INS >= 1 && A_INS * 16 * W == BM && B_INS * 16 * W == BN, "tile split");
    static_assert(PW >= 1 && PW <= W, "row-vector DMA waves");
    // 16-byte result stores each wave issues per tile (epilogue_bf16, or the
    // code stores of epilogue_mx_gemm1)
    template <bool GEMM1>
    static constexpr int stores() { return NT * (GEMM1 ? (MX ? 2 : 4) : 8); }
    static_assert(stores<false>() * 1024 <= kSinkWaveBytes, "sink lines per wave");
    static_assert(!MX || BM / 64 + BN / 64 == W, "one scale-row DMA per wave");
};

// One stage of the ring. Stage buffers start on 1 KB boundaries so that a
// DMA instruction's 1 KB lands on whole 256-byte bank rows.
template <int BM, bool MX>
struct StageBuf {
    uint8_t tok[BM * RB];
    uint8_t wt[BN * RB];
};
constexpr int kScaleSlots = 4;
// MX scale ring: slot (pair & 3) holds, per token row and per weight row,
// the scale dword of stage pair `pair` (32-blocks 4*pair .. 4*pair+3: the
// stage pair's two stages use two blocks each). The pair counter runs on
// across tiles, so a new tile's pairs never land in a slot still being read.
// A pair's dword is fetched once, with its even stage.
template <int BM>
struct ScaleSlot {
    uint32_t tok[BM];
    uint32_t wt[BN];
};

// Per-tile DMA sources: wave-uniform bases (scalar registers) plus 32-bit
// per-lane byte offsets. Token rows need one offset per instruction (they may
// be gathered); weight rows are consecutive and share `boff` + j * bstride,
// which does not change from tile to tile. MX: each wave also moves the
// scale dword of 64 rows (waves 0..3 token rows, 4..7 weight rows).
template <int BM, bool MX>
struct DmaSrc {
    const char* abase;
    const char* bbase;
    uint32_t aoff[Big<BM, MX>::A_INS];
};
template <int BM>
struct DmaSrc<BM, true> {
    const char* abase;
    const char* bbase;
    const char* sbase;
    uint32_t aoff[Big<BM, true>::A_INS];
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

__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

// Stage kt of a tile: L code DMA instructions per wave, plus (MX, even kt)
// the scale dword of the stage pair into `scale` (nullptr for bf16).
template <int BM, bool MX>
__device__ __forceinline__ void issue_stage(StageBuf<BM, MX>& b, const DmaSrc<BM, MX>& src, uint32_t boff,
                                            uint32_t bstride, int kt, uint32_t wave, ScaleSlot<BM>* scale) {
    using C = Big<BM, MX>;
    const char* ab = src.abase + kt * RB;
    const char* bb = src.bbase + kt * RB;
    const uint32_t tl = lds_addr(b.tok) + wave * (C::A_INS * 1024);
    const uint32_t wl = lds_addr(b.wt) + wave * (C::B_INS * 1024);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) dma16(ab, src.aoff[j], tl + j * 1024);
#pragma unroll
    for (int j = 0; j < C::B_INS; ++j) dma16(bb, boff + j * bstride, wl + j * 1024);
    if constexpr (MX) {
        if ((kt & 1) == 0) {
            const uint32_t sl = wave < static_cast<uint32_t>(BM / 64) ? lds_addr(scale->tok) + wave * 256
                                                                       : lds_addr(scale->wt) + (wave - BM / 64) * 256;
            dma4(src.sbase, src.soff + (kt >> 1) * 4, sl);
        }
    }
}

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

// until this wave's LDS reads have returned (vector memory not waited for)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8)); }

// s_barrier without a memory fence; the asm statements stop the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Half a stage in registers. bf16: the stage's k-half h (16 of its 32 K
// elements) for all 4 weight and NT token fragments. MX: the whole 64-wide K
// step for weight fragments 2h, 2h+1 with each row's scale byte; the token
// fragments of a stage are held once (TokFrag).
template <int BM, bool MX>
struct Frag;
template <int BM>
struct Frag<BM, false> {
    bf16x8_t w[4];
    bf16x8_t t[Big<BM, false>::NT];
};
template <int BM>
struct Frag<BM, true> {  // MX: two weight fragments (2h, 2h+1) with their scale bytes
    i32x8_t w[2];
    int sw[2];
};
// MX: the token fragments of a stage with their scale bytes.
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

// Per-lane LDS byte offsets of a wave's fragment rows, fixed for the whole
// kernel. A weight fragment f starts at tile row wrow0 + FROW[f] (FROW a
// compile-time table), a token fragment t at tok_row0 + 32t; a lane reads
// row (start) + (lane & 31). Every fragment's rows start at a multiple of
// 16, so the swizzle term is ((lane & 31) >> 2) & 3 for all of them.
// A lane reads 16-byte chunks g and 2 + g of a row (g = lane >> 5): the
// bf16 k-halves 0 and 1, or the two halves of an MX operand. Their swizzled
// offsets are kept as two values, not an array indexed by g, which the
// compiler would put in scratch memory; a scratch load in the loop makes it
// wait for every memory operation in flight, DMAs included.
struct LaneOff {
    int w, t;        // row offsets: (wrow0 + (lane & 31)) * RB, (tok_row0 + (lane & 31)) * RB
    int clo, chi;    // swizzled offsets of chunks g and 2 + g
    int sw, st;      // MX: scale dword offsets (wrow0 + (lane & 31)) * 4, (tok_row0 + (lane & 31)) * 4
};

template <bool GEMM1>
__device__ __forceinline__ constexpr int frow_const(int f) {
    // GEMM1: gate rows 0..127 and up rows 128..255, a wave's 64 of each; GEMM2: 128 consecutive rows
    return GEMM1 ? (f < 2 ? 32 * f : 128 + 32 * (f - 2)) : 32 * f;
}

// Fragment reads. PAR is the stage's parity (which MX scale bytes).
template <int BM, bool GEMM1, bool MX, int PAR>
__device__ __forceinline__ void read_half(const StageBuf<BM, MX>& b, const ScaleSlot<BM>* sc, int h, const LaneOff& o,
                                          Frag<BM, MX>& f) {
    using C = Big<BM, MX>;
    const int g = (threadIdx.x & 63) >> 5;
    if constexpr (!MX) {
        const int co = h == 0 ? o.clo : o.chi;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f.w[i] = *reinterpret_cast<const bf16x8_t*>(b.wt + o.w + frow_const<GEMM1>(i) * RB + co);
#pragma unroll
        for (int i = 0; i < C::NT; ++i) f.t[i] = *reinterpret_cast<const bf16x8_t*>(b.tok + o.t + 32 * i * RB + co);
    } else {
        const int lo = o.clo, hi = o.chi;
        const int sh = 8 * (2 * PAR + g);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int fr = frow_const<GEMM1>(2 * h + i);
            f.w[i] = frag32(b.wt + o.w + fr * RB, lo, hi);
            f.sw[i] = static_cast<int>((*reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(sc->wt) +
                                                                           o.sw + fr * 4) >> sh) & 0xffu);
        }
    }
}

template <int BM, int PAR>
__device__ __forceinline__ void read_tok(const StageBuf<BM, true>& b, const ScaleSlot<BM>* sc, const LaneOff& o,
                                         TokFrag<BM>& f) {
    const int g = (threadIdx.x & 63) >> 5;
    const int lo = o.clo, hi = o.chi;
    const int sh = 8 * (2 * PAR + g);
#pragma unroll
    for (int i = 0; i < Big<BM, true>::NT; ++i) {
        f.t[i] = frag32(b.tok + o.t + 32 * i * RB, lo, hi);
        f.st[i] = static_cast<int>((*reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(sc->tok) +
                                                                       o.st + 32 * i * 4) >> sh) & 0xffu);
    }
}

// Keeps the MFMAs of an MX half-stage where they are written: the empty asm
// makes the accumulators' new values needed at this point. Without it the
// compiler sinks the MFMAs of several steps past the barriers (their results
// are only read after the loop), and every fragment read in between stays
// live in registers: hundreds of spills. (The bf16 loop is left to the
// compiler's schedule, which is faster there.)
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

template <int BM>
__device__ __forceinline__ void mfma_mx(const Frag<BM, true>& f, const TokFrag<BM>& tf, int h,
                                        f32x16_t (&acc)[4][Big<BM, true>::NT]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < Big<BM, true>::NT; ++t)
            acc[2 * h + i][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[i], tf.t[t], acc[2 * h + i][t], 0,
                                                                                 0, 0, f.sw[i], 0, tf.st[t]);
    pin_acc(acc, 2 * h, 2 * h + 2);
}

// Registers a wave carries from one ring step to the next: bf16 the two
// k-halves of a stage; MX the two weight-fragment pairs and the stage's
// token fragments.
template <int BM, bool MX>
struct Regs;
template <int BM>
struct Regs<BM, false> {
    Frag<BM, false> f0, f1;
};
template <int BM>
struct Regs<BM, true> {
    Frag<BM, true> f0, f1;
    TokFrag<BM> tf;
};

// Everything a workgroup keeps across the steps of a tile.
template <int BM, bool MX>
struct Ring {
    DmaSrc<BM, MX> src, nsrc;  // this tile's and the next tile's DMA sources
    uint32_t boff, bstride;    // weight-row offsets (the same for every tile)
    uint32_t wave;             // wave index (uniform)
    int KT;                    // K stages per tile
    bool pipelined;            // KT is long enough for the in-loop hand-over
    bool has_next;
    bool cont;                 // the next tile's stages follow this tile's in the ring
    TileDesc next;             // the next tile (valid when has_next)
    int nb;                    // row-vector buffer of the next tile (0 or 1)
    ScaleSlot<BM>* scales;     // MX: the kScaleSlots scale slots
    int pair0;                 // MX: running stage-pair index of this tile's stage 0
    // MX: the scale slot of stage s of this tile (next = false) or of the next tile
    __device__ __forceinline__ ScaleSlot<BM>* slot(int s, bool next = false) const {
        if constexpr (!MX) return nullptr;
        else return scales + ((pair0 + (next ? KT / 2 : 0) + (s >> 1)) & (kScaleSlots - 1));
    }
};

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

// DMA sources of a tile. GEMM1: token rows gathered through the row map;
// weight rows 0..127 are gate rows h0.., 128..255 up rows H + h0.. (a wave's
// rows never straddle the two). GEMM2: act rows in sorted order. Offsets are
// 32-bit: the host only picks this kernel when each operand array (and, for
// the weights, one expert's) spans < 4 GiB. Instruction j of a wave covers
// tile rows (wave * INS + j) * 16 + lane / 4, chunk lane & 3.
template <int BM, bool GEMM1, bool MX>
__device__ __forceinline__ void make_src(const BigArgs& a, const TileDesc& t, const int32_t* pairs, uint32_t wave,
                                         DmaSrc<BM, MX>& s) {
    using C = Big<BM, MX>;
    constexpr int EB = Fmt<MX>::EB;
    const int lane = threadIdx.x & 63;
    const int K = GEMM1 ? a.D : a.H;
    const int h0 = t.ntile * 128, n0 = t.ntile * 256;
    s.abase = uniform_ptr(GEMM1 ? a.x : a.act + static_cast<int64_t>(t.row0) * a.H * EB);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) {
        const int row = (static_cast<int>(wave) * C::A_INS + j) * 16 + lane / 4;
        const uint32_t r = GEMM1 ? static_cast<uint32_t>(clamp_pair(pairs[row], a.P) / a.k) * a.D
                                 : static_cast<uint32_t>(row < t.rows ? row : 0) * a.H;
        s.aoff[j] = r * EB + swz_chunk(row, lane & 3) * 16;
    }
    const int row0 = static_cast<int>(wave) * C::B_INS * 16;  // first weight-tile row of this wave
    const int64_t e2h = static_cast<int64_t>(t.expert) * 2 * a.H;
    if (GEMM1) {
        const int grow0 = row0 < 128 ? h0 + row0 : a.H + h0 + row0 - 128;
        s.bbase = uniform_ptr(a.w1 + (e2h + grow0) * K * EB);
    } else {
        s.bbase = uniform_ptr(a.w2 + (static_cast<int64_t>(t.expert) * a.D + n0 + row0) * K * EB);
    }
    if constexpr (MX) {
        const int KB = K / 32;  // scale bytes per row
        if (wave < static_cast<uint32_t>(BM / 64)) {
            const int r = static_cast<int>(wave) * 64 + lane;  // token row
            if (GEMM1) {
                s.sbase = uniform_ptr(a.xs);
                s.soff = static_cast<uint32_t>(clamp_pair(pairs[r], a.P) / a.k) * KB;
            } else {
                s.sbase = uniform_ptr(a.act_s);
                s.soff = static_cast<uint32_t>(t.row0 + (r < t.rows ? r : 0)) * KB;
            }
        } else {
            const int r = (static_cast<int>(wave) - BM / 64) * 64 + lane;  // weight row
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

// One ring step. The barrier sits in the middle of stage kt's MFMAs, so a
// wave never comes out of it with nothing to compute:
//   read half 1 of stage kt (buffer cur);  MFMAs of half 0 (read last step)
//   wait for this wave's DMAs of stage kt+1 and its own LDS reads;  barrier
//   issue stage kt+4 into cur (every wave is done reading it);
//   read half 0 of stage kt+1 (buffer nxt);  MFMAs of half 1
// Stage kt+4 belongs to this tile, or to the next one once this tile has
// none left, so the ring runs on across tiles. PAR = kt & 1.
//
// Waits: before the barrier each wave waits until its own DMAs of stage kt+1
// are done; the stages it issued after it (kt+2, kt+3, while they exist) may
// stay in flight. Vector-memory operations of a wave (loads, LDS DMA and
// stores) leave the count in issue order, so a budget of n outstanding
// guarantees every operation older than the last n. Extra younger operations
// (the few row-vector DMAs) only make a wait stricter. The previous tile's
// result stores are younger than stages 1..3 of this one: in steps 0..2 the
// budget grows by their exact number, so those steps wait for their stage
// and not for the stores; step 3's stage was issued after the stores.
//
// Hand-over (pipelined tiles): step 0 fetches the next tile's row map,
// complete by step 3's barrier; step 3 builds the next tile's DMA sources
// from it and fetches its routing weights (GEMM2), complete by step 6's
// barrier; steps KT-4 .. KT-1 issue its stages 0..3.
template <int N, int EX>
__device__ __forceinline__ void wait_budget(bool extra) {
    if (extra) wait_vm_lds<N + EX>();
    else wait_vm_lds<N>();
}

template <int BM, bool GEMM1, bool MX, int PAR, bool VAR>
__device__ __forceinline__ void ring_step(const BigArgs& a, Ring<BM, MX>& r, StageBuf<BM, MX>& cur,
                                          const StageBuf<BM, MX>& nxt, int kt, int32_t (*pairs)[BM],
                                          float (*wrow)[BM], const LaneOff& o, Regs<BM, MX>& g,
                                          f32x16_t (&acc)[4][Big<BM, MX>::NT]) {
    using C = Big<BM, MX>;
    read_half<BM, GEMM1, MX, PAR>(cur, r.slot(kt), 1, o, g.f1);
    if constexpr (MX) mfma_mx<BM>(g.f0, g.tf, 0, acc);
    else mfma_half<BM>(g.f0, acc);
    const bool more1 = kt + 1 < r.KT || r.cont;  // stage kt+1 exists
    constexpr int S = C::template stores<GEMM1>();
    const bool after_stores = kt < 3;  // the previous tile's stores are in flight
    if (kt + 3 < r.KT || r.cont) wait_budget<C::Y2, S>(after_stores);
    else if (kt + 2 < r.KT) wait_budget<C::Y1, S>(after_stores);
    else wait_budget<0, S>(after_stores);
    // The budgets above already wait for the LDS reads; repeating that outside
    // the branches lets the compiler see it on every path, so it does not hold
    // the MFMAs of half 1 for the reads issued after the barrier.
    wait_lds();
    bare_barrier();
    if (r.cont) {
        if (kt == 0) dma_row_map<BM>(a, r.next.row0, pairs[r.nb], r.wave);
        if (kt == 3) {
            make_src<BM, GEMM1, MX>(a, r.next, pairs[r.nb], r.wave, r.nsrc);
            if (!GEMM1 || (VAR && a.av.wba)) dma_row_weights<BM>(a, pairs[r.nb], wrow[r.nb], r.wave);
        }
    }
    if (kt + 4 < r.KT) issue_stage<BM, MX>(cur, r.src, r.boff, r.bstride, kt + 4, r.wave, r.slot(kt + 4));
    else if (r.cont)
        issue_stage<BM, MX>(cur, r.nsrc, r.boff, r.bstride, kt + 4 - r.KT, r.wave, r.slot(kt + 4 - r.KT, true));
    ScaleSlot<BM>* nsc = kt + 1 < r.KT ? r.slot(kt + 1) : r.slot(0, true);  // scales of stage kt+1
    if (more1) read_half<BM, GEMM1, MX, PAR ^ 1>(nxt, nsc, 0, o, g.f0);
    if constexpr (MX) {
        // the token fragments of stage kt+1 go where this stage's were, once
        // its last MFMAs have been issued
        mfma_mx<BM>(g.f1, g.tf, 1, acc);
        if (more1) read_tok<BM, PAR ^ 1>(nxt, nsc, o, g.tf);
    } else {
        mfma_half<BM>(g.f1, acc);
    }
}

// The stage buffers come in as restrict pointers: with them, the compiler
// knows the fragment reads of one stage never alias the others.
template <int BM, bool GEMM1, bool MX, bool VAR>
__device__ __forceinline__ void main_loop(const BigArgs& a, Ring<BM, MX>& r, StageBuf<BM, MX>* __restrict__ b0,
                                          StageBuf<BM, MX>* __restrict__ b1, StageBuf<BM, MX>* __restrict__ b2,
                                          StageBuf<BM, MX>* __restrict__ b3, int32_t (*pairs)[BM],
                                          float (*wrow)[BM], const LaneOff& o, Regs<BM, MX>& g,
                                          f32x16_t (&acc)[4][Big<BM, MX>::NT]) {
    // KT is a multiple of 4: the unrolled body needs no exit in the middle,
    // which would make the compiler shuttle the accumulators between
    // registers at the loop head. Every tile starts at buffer 0, with the
    // previous tile's result stores (or the first tile's sink stores) in
    // flight. The body is unrolled by hand; for MX, more copies only raise
    // register pressure.
    if constexpr (MX) {
#pragma clang loop unroll(disable)
        for (int kt = 0; kt < r.KT; kt += 4) {
            ring_step<BM, GEMM1, MX, 0, VAR>(a, r, *b0, *b1, kt, pairs, wrow, o, g, acc);
            ring_step<BM, GEMM1, MX, 1, VAR>(a, r, *b1, *b2, kt + 1, pairs, wrow, o, g, acc);
            ring_step<BM, GEMM1, MX, 0, VAR>(a, r, *b2, *b3, kt + 2, pairs, wrow, o, g, acc);
            ring_step<BM, GEMM1, MX, 1, VAR>(a, r, *b3, *b0, kt + 3, pairs, wrow, o, g, acc);
        }
    } else {
        for (int kt = 0; kt < r.KT; kt += 4) {
            ring_step<BM, GEMM1, MX, 0, VAR>(a, r, *b0, *b1, kt, pairs, wrow, o, g, acc);
            ring_step<BM, GEMM1, MX, 1, VAR>(a, r, *b1, *b2, kt + 1, pairs, wrow, o, g, acc);
            ring_step<BM, GEMM1, MX, 0, VAR>(a, r, *b2, *b3, kt + 2, pairs, wrow, o, g, acc);
            ring_step<BM, GEMM1, MX, 1, VAR>(a, r, *b3, *b0, kt + 3, pairs, wrow, o, g, acc);
        }
    }
}

// Issue stages 0..3 of a tile (this one, or the next one: `next`), wait for
// stage 0 and read its first half.
template <int BM, bool GEMM1, bool MX>
__device__ __forceinline__ void ring_start(Ring<BM, MX>& r, const DmaSrc<BM, MX>& src, bool next,
                                           StageBuf<BM, MX>& b0, StageBuf<BM, MX>& b1, StageBuf<BM, MX>& b2,
                                           StageBuf<BM, MX>& b3, const LaneOff& o, Regs<BM, MX>& g) {
    issue_stage<BM, MX>(b0, src, r.boff, r.bstride, 0, r.wave, r.slot(0, next));
    issue_stage<BM, MX>(b1, src, r.boff, r.bstride, 1, r.wave, r.slot(1, next));
    issue_stage<BM, MX>(b2, src, r.boff, r.bstride, 2, r.wave, r.slot(2, next));
    issue_stage<BM, MX>(b3, src, r.boff, r.bstride, 3, r.wave, r.slot(3, next));
    wait_vm<Big<BM, MX>::Y3>();
    bare_barrier();
    read_half<BM, GEMM1, MX, 0>(b0, r.slot(0, next), 0, o, g.f0);
    if constexpr (MX) read_tok<BM, 0>(b0, r.slot(0, next), o, g.tf);
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

__device__ __forceinline__ uint8_t* wave_sink(const BigArgs& a) {
    return a.sink + ((blockIdx.x & (kSinkSlots - 1)) * W + (threadIdx.x >> 6)) * kSinkWaveBytes +
           (threadIdx.x & 63) * 16;
}

__device__ __forceinline__ void store16(void* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// The stores a wave's first tile finds in flight in place of a previous
// tile's: Big::stores() zero lines to its sink area.
template <int BM, bool GEMM1, bool MX>
__device__ __forceinline__ void sink_stores(const BigArgs& a) {
    uint8_t* sink = wave_sink(a);
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
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, g = lane >> 5;
    const int rr = lane >> 2, c = lane & 3;  // staging reads: rows rr and rr + 16, chunk c
    const int rd0 = stage_chunk_off(rr, c), rd1 = stage_chunk_off(rr + 16, c);
    uint16_t* sink = reinterpret_cast<uint16_t*>(wave_sink(a));
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
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, g = lane >> 5;
    const int rr = lane >> 2, c = lane & 3;
    const int rd0 = stage_chunk_off(rr, c), rd1 = stage_chunk_off(rr + 16, c);
    const int HB = a.H / 32;
    const int col0 = t.ntile * 128 + 64 * wf;  // first act column of this wave
    uint8_t* sink = wave_sink(a);
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

template <int BM, bool GEMM1, bool MX, bool VAR>
__global__ __launch_bounds__(kThreads, 1) void big_gemm_kernel(BigArgs a, const int4* __restrict__ mtiles) {
    using C = Big<BM, MX>;
    constexpr int CAP = Fmt<MX>::kInfoCap;
    __shared__ __attribute__((aligned(1024))) StageBuf<BM, MX> buf0;
    __shared__ __attribute__((aligned(1024))) StageBuf<BM, MX> buf1;
    __shared__ __attribute__((aligned(1024))) StageBuf<BM, MX> buf2;
    __shared__ __attribute__((aligned(1024))) StageBuf<BM, MX> buf3;
    __shared__ __attribute__((aligned(16))) int32_t sPair[2][BM];
    __shared__ __attribute__((aligned(16))) float sW[2][BM];
    __shared__ TileDesc sDesc[CAP];
    __shared__ __attribute__((aligned(16))) uint8_t sOut[W][2048];  // per-wave result staging
    __shared__ __attribute__((aligned(16))) ScaleSlot<BM> sScale[MX ? kScaleSlots : 1];

    // This workgroup's tiles: logical tiles first, first + stride, ... of its
    // XCD's range. The tile count comes from the route step.
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
        const int lane = tid & 63, lr = lane & 31;
        const int wrow0 = (GEMM1 ? 64 : 128) * wf;
        o.w = (wrow0 + lr) * RB;
        o.t = (tok_row0 + lr) * RB;
        o.clo = swz_chunk(lr, lane >> 5) << 4;
        o.chi = swz_chunk(lr, 2 + (lane >> 5)) << 4;
        o.sw = (wrow0 + lr) * 4;
        o.st = (tok_row0 + lr) * 4;
    }

    Ring<BM, MX> r;
    r.wave = static_cast<uint32_t>(uniform_int(wave_v));
    r.scales = sScale;
    r.pair0 = 0;
    const int K = GEMM1 ? a.D : a.H;
    r.KT = K / Fmt<MX>::KS;
    r.pipelined = r.KT >= kMinPipelinedKT;
    {
        const int lane = tid & 63;
        const int row = static_cast<int>(r.wave) * C::B_INS * 16 + lane / 4;  // +16 rows per instruction
        r.boff = static_cast<uint32_t>(lane / 4) * K * Fmt<MX>::EB + swz_chunk(row, lane & 3) * 16;
        r.bstride = 16u * K * Fmt<MX>::EB;
    }

    load_descs<CAP>(mtiles, first, stride, ny, count, 0, sDesc);
    __syncthreads();
    TileDesc t = uniform_desc(sDesc[0]);

    // first tile: row map (and weights) now, then its first four stages
    int cb = 0;
    dma_row_map<BM>(a, t.row0, sPair[0], r.wave);
    wait_vm<0>();
    bare_barrier();
    make_src<BM, GEMM1, MX>(a, t, sPair[0], r.wave, r.src);
    if (!GEMM1 || (VAR && a.av.wba)) {
        dma_row_weights<BM>(a, sPair[0], sW[0], r.wave);
        wait_vm<0>();
        bare_barrier();
    }
    Regs<BM, MX> g;
    ring_start<BM, GEMM1, MX>(r, r.src, false, buf0, buf1, buf2, buf3, o, g);
    sink_stores<BM, GEMM1, MX>(a);

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
        r.cont = r.has_next && r.pipelined;

        main_loop<BM, GEMM1, MX, VAR>(a, r, &buf0, &buf1, &buf2, &buf3, sPair, sW, o, g, acc);

        if (r.has_next && !r.pipelined) {
            // short K: hand over after the ring has drained
            dma_row_map<BM>(a, r.next.row0, sPair[r.nb], r.wave);
            wait_vm<0>();
            bare_barrier();
            make_src<BM, GEMM1, MX>(a, r.next, sPair[r.nb], r.wave, r.nsrc);
            if (!GEMM1 || (VAR && a.av.wba)) {
                dma_row_weights<BM>(a, sPair[r.nb], sW[r.nb], r.wave);
                wait_vm<0>();
                bare_barrier();
            }
            ring_start<BM, GEMM1, MX>(r, r.nsrc, true, buf0, buf1, buf2, buf3, o, g);
        }
        if constexpr (GEMM1 && MX) epilogue_mx_gemm1<BM>(a, t, tok_row0, wf, sOut[wave_v], acc);
        else epilogue_bf16<BM, GEMM1, MX, VAR>(a, t, sPair[cb], sW[cb], tok_row0, wf, sOut[wave_v], acc);
        if (!r.has_next) break;
        t = r.next;
        r.src = r.nsrc;
        r.pair0 += r.KT / 2;
        cb ^= 1;
    }
}

// ---------------------------------------------------------------------------
// bf16 with 128-byte stages. A stage holds 64 elements of K per tile row, so
// every row's piece of a stage is one whole 128-byte line: half the memory
// requests of the 64-byte stages above for the same bytes. Two stage buffers
// (2 x 64 KB for 256-row tiles) make a double-buffered ring: while stage kt
// is consumed, stage kt + 1 is in flight, and one barrier per stage (a K
// step of 64) guards both buffers. Tiles, waves and epilogues are those of
// the kernel above; the ring runs on across tiles the same way.
//
// Swizzle: 16-byte chunk c of row r sits at chunk position c ^ ((r >> 1) & 7)
// of its 128-byte LDS row. A fragment read has 16 lanes read the same chunk
// of 16 consecutive rows; the rows of one parity then take 8 distinct chunk
// positions, and the two parities sit in different 128-byte halves of the
// 256-byte bank row, so the 16 reads hit 16 distinct bank groups.
constexpr int RB2 = 128;  // bytes per tile row per stage

template <int BM>
struct StageBuf2 {
    uint8_t tok[BM * RB2];
    uint8_t wt[BN * RB2];
};

template <int BM>
struct Deep {
    static constexpr int NT = Big<BM, false>::NT;
    static constexpr int A_INS = BM / 8 / W;  // token-row DMA instructions per wave per stage (8 rows each)
    static constexpr int B_INS = BN / 8 / W;  // weight-row DMA instructions per wave per stage
    static_assert(A_INS >= 1 && A_INS * 8 * W == BM && B_INS * 8 * W == BN, "tile split");
    static_assert(B_INS % 2 == 0, "weight-row offsets alternate with the instruction's parity");
};

__device__ __forceinline__ int swz8(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int BM>
struct DmaSrc2 {
    const char* abase;
    const char* bbase;
    uint32_t aoff[Deep<BM>::A_INS];
};

// Per-lane LDS offsets of the fragment rows and of the four quarters' chunks
// (quarter q: K elements 16q .. 16q + 15, chunks 2q and 2q + 1; lane group
// g = lane >> 5 reads chunk 2q + g).
struct LaneOff2 {
    int w, t;
    int c0, c1, c2, c3;
};

template <int BM>
struct Ring2 {
    DmaSrc2<BM> src, nsrc;
    uint32_t boff0, boff1, bstride;  // weight-row offsets of even and odd instructions (the same for every tile)
    uint32_t wave;
    int KT;
    bool has_next, cont;
    TileDesc next;
    int nb;
};

// Instruction j of a wave covers tile rows (wave * INS + j) * 8 + lane / 8;
// lane i's 16 bytes land at chunk position i & 7 of that row, so it fetches
// the global chunk that the swizzle puts there.
template <int BM, bool GEMM1>
__device__ __forceinline__ void make_src2(const BigArgs& a, const TileDesc& t, const int32_t* pairs, uint32_t wave,
                                          DmaSrc2<BM>& s) {
    using C = Deep<BM>;
    const int lane = threadIdx.x & 63;
    const int K = GEMM1 ? a.D : a.H;
    const int h0 = t.ntile * 128, n0 = t.ntile * 256;
    s.abase = uniform_ptr(GEMM1 ? a.x : a.act + static_cast<int64_t>(t.row0) * a.H * 2);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) {
        const int row = (static_cast<int>(wave) * C::A_INS + j) * 8 + lane / 8;
        const uint32_t r = GEMM1 ? static_cast<uint32_t>(clamp_pair(pairs[row], a.P) / a.k) * a.D
                                 : static_cast<uint32_t>(row < t.rows ? row : 0) * a.H;
        s.aoff[j] = r * 2 + swz8(row, lane & 7) * 16;
    }
    const int row0 = static_cast<int>(wave) * C::B_INS * 8;  // 32 weight rows per wave, never across gate/up
    if (GEMM1) {
        const int grow0 = row0 < 128 ? h0 + row0 : a.H + h0 + row0 - 128;
        s.bbase = uniform_ptr(a.w1 + (static_cast<int64_t>(t.expert) * 2 * a.H + grow0) * K * 2);
    } else {
        s.bbase = uniform_ptr(a.w2 + (static_cast<int64_t>(t.expert) * a.D + n0 + row0) * K * 2);
    }
}

template <int BM>
__device__ __forceinline__ void issue2(StageBuf2<BM>& b, const DmaSrc2<BM>& src, const Ring2<BM>& r, int kt) {
    using C = Deep<BM>;
    const char* ab = src.abase + kt * RB2;
    const char* bb = src.bbase + kt * RB2;
    const uint32_t tl = lds_addr(b.tok) + r.wave * (C::A_INS * 1024);
    const uint32_t wl = lds_addr(b.wt) + r.wave * (C::B_INS * 1024);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) dma16(ab, src.aoff[j], tl + j * 1024);
#pragma unroll
    for (int j = 0; j < C::B_INS; ++j) dma16(bb, ((j & 1) ? r.boff1 : r.boff0) + j * r.bstride, wl + j * 1024);
}

template <int BM, bool GEMM1, int Q>
__device__ __forceinline__ void read_q(const StageBuf2<BM>& b, const LaneOff2& o, Frag<BM, false>& f) {
    const int co = Q == 0 ? o.c0 : Q == 1 ? o.c1 : Q == 2 ? o.c2 : o.c3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.w[i] = *reinterpret_cast<const bf16x8_t*>(b.wt + o.w + frow_const<GEMM1>(i) * RB2 + co);
#pragma unroll
    for (int i = 0; i < Deep<BM>::NT; ++i) f.t[i] = *reinterpret_cast<const bf16x8_t*>(b.tok + o.t + 32 * i * RB2 + co);
}

// One stage (K step of 64) of the double-buffered ring:
//   wait for this wave's DMAs of stage kt and its LDS reads;  barrier
//   (FIRST) hand-over work for the next tile;  issue stage kt + 1 into the
//   other buffer (every wave is done reading it: stage kt - 1);
//   read quarter 0 of stage kt;  MFMAs of quarter 3 of stage kt - 1;
//   read q1, MFMAs q0;  read q2, MFMAs q1;  read q3, MFMAs q2.
// Quarter 3's MFMAs move past the next barrier, so no wave comes out of it
// with nothing to compute. Waits: a wave's vector-memory operations complete
// in issue order. In a tile's step 0 the previous tile's result stores (or
// the first tile's sink stores), issued after stage 0, may stay in flight;
// every later step waits for everything: the only operations younger than
// stage kt then are none. Hand-over: step 0 fetches the next tile's row map
// (landed by step 1's barrier), step 1 builds its DMA sources and fetches its
// routing weights, and step KT - 1 issues its stage 0.
template <int BM, bool GEMM1, bool VAR, bool FIRST, bool SECOND>
__device__ __forceinline__ void deep_step(const BigArgs& a, Ring2<BM>& r, const StageBuf2<BM>& cur,
                                          StageBuf2<BM>& oth, int kt, int32_t (*pairs)[BM], float (*wrow)[BM],
                                          const LaneOff2& o, Frag<BM, false>& x, Frag<BM, false>& y,
                                          f32x16_t (&acc)[4][Deep<BM>::NT]) {
    constexpr int S = Big<BM, false>::template stores<GEMM1>();
    if (FIRST) wait_vm_lds<S>();
    else wait_vm_lds<0>();
    bare_barrier();
    if (FIRST && r.cont) dma_row_map<BM>(a, r.next.row0, pairs[r.nb], r.wave);
    if (SECOND && r.cont) {
        make_src2<BM, GEMM1>(a, r.next, pairs[r.nb], r.wave, r.nsrc);
        if (!GEMM1 || (VAR && a.av.wba)) dma_row_weights<BM>(a, pairs[r.nb], wrow[r.nb], r.wave);
    }
    if (kt + 1 < r.KT) issue2<BM>(oth, r.src, r, kt + 1);
    else if (r.cont) issue2<BM>(oth, r.nsrc, r, 0);
    read_q<BM, GEMM1, 0>(cur, o, x);
    if (!FIRST) mfma_half<BM>(y, acc);
    read_q<BM, GEMM1, 1>(cur, o, y);
    mfma_half<BM>(x, acc);
    read_q<BM, GEMM1, 2>(cur, o, x);
    mfma_half<BM>(y, acc);
    read_q<BM, GEMM1, 3>(cur, o, y);
    mfma_half<BM>(x, acc);
    // Keep that order: each quarter's fragment reads go out as a group ahead
    // of the previous quarter's MFMAs, which hide their latency. Left alone,
    // the scheduler moves each read next to its first use.
    constexpr int R = 4 + Deep<BM>::NT, M = 4 * Deep<BM>::NT;
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    if (!FIRST) __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    }
}

template <int BM, bool GEMM1, bool VAR>
__global__ __launch_bounds__(kThreads, 1) void big_deep_kernel(BigArgs a, const int4* __restrict__ mtiles) {
    using C = Deep<BM>;
    constexpr int CAP = Fmt<false>::kInfoCap;
    __shared__ __attribute__((aligned(1024))) StageBuf2<BM> buf0;
    __shared__ __attribute__((aligned(1024))) StageBuf2<BM> buf1;
    __shared__ __attribute__((aligned(16))) int32_t sPair[2][BM];
    __shared__ __attribute__((aligned(16))) float sW[2][BM];
    __shared__ TileDesc sDesc[CAP];
    __shared__ __attribute__((aligned(16))) uint8_t sOut[W][2048];  // per-wave result staging

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
    const int tok_row0 = wtok * Big<BM, false>::TB;
    LaneOff2 o;
    {
        const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
        const int wrow0 = (GEMM1 ? 64 : 128) * wf;
        o.w = (wrow0 + lr) * RB2;
        o.t = (tok_row0 + lr) * RB2;
        // fragment rows start at multiples of 32: the swizzle term is ((lane & 31) >> 1) & 7
        o.c0 = swz8(lr, g) << 4;
        o.c1 = swz8(lr, 2 + g) << 4;
        o.c2 = swz8(lr, 4 + g) << 4;
        o.c3 = swz8(lr, 6 + g) << 4;
    }

    Ring2<BM> r;
    r.wave = static_cast<uint32_t>(uniform_int(wave_v));
    const int K = GEMM1 ? a.D : a.H;
    r.KT = K / 64;
    {
        // weight row of instruction j: wave * 8 * B_INS + 8j + lane / 8; with
        // B_INS even its swizzle term is 4 (j & 1) + lane / 16
        const int lane = tid & 63;
        const uint32_t rowoff = static_cast<uint32_t>(lane / 8) * K * 2;
        r.boff0 = rowoff + (((lane & 7) ^ (lane >> 4)) << 4);
        r.boff1 = rowoff + (((lane & 7) ^ (4 + (lane >> 4))) << 4);
        r.bstride = 8u * K * 2;
    }

    load_descs<CAP>(mtiles, first, stride, ny, count, 0, sDesc);
    __syncthreads();
    TileDesc t = uniform_desc(sDesc[0]);
    int cb = 0;
    dma_row_map<BM>(a, t.row0, sPair[0], r.wave);
    wait_vm<0>();
    bare_barrier();
    make_src2<BM, GEMM1>(a, t, sPair[0], r.wave, r.src);
    if (!GEMM1 || (VAR && a.av.wba)) {
        dma_row_weights<BM>(a, sPair[0], sW[0], r.wave);
        wait_vm<0>();
        bare_barrier();
    }
    issue2<BM>(buf0, r.src, r, 0);
    sink_stores<BM, GEMM1, false>(a);

    Frag<BM, false> x, y;
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

        // KT is even: every tile starts in buffer 0
        deep_step<BM, GEMM1, VAR, true, false>(a, r, buf0, buf1, 0, sPair, sW, o, x, y, acc);
        deep_step<BM, GEMM1, VAR, false, true>(a, r, buf1, buf0, 1, sPair, sW, o, x, y, acc);
        for (int kt = 2; kt < r.KT; kt += 2) {
            deep_step<BM, GEMM1, VAR, false, false>(a, r, buf0, buf1, kt, sPair, sW, o, x, y, acc);
            deep_step<BM, GEMM1, VAR, false, false>(a, r, buf1, buf0, kt + 1, sPair, sW, o, x, y, acc);
        }
        mfma_half<BM>(y, acc);  // quarter 3 of the last stage

        epilogue_bf16<BM, GEMM1, false, VAR>(a, t, sPair[cb], sW[cb], tok_row0, wf, sOut[wave_v], acc);
        if (!r.has_next) break;
        t = r.next;
        r.src = r.nsrc;
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
        if (gemm1) big_gemm_kernel<BM, true, true, false><<<g, kThreads, 0, s>>>(a, tiles);
        else big_gemm_kernel<BM, false, true, false><<<g, kThreads, 0, s>>>(a, tiles);
    } else {
        const bool var = a.av.on();  // the activation variant has kernels of its own
        if (gemm1) {
            if (var) big_deep_kernel<BM, true, true><<<g, kThreads, 0, s>>>(a, tiles);
            else big_deep_kernel<BM, true, false><<<g, kThreads, 0, s>>>(a, tiles);
        } else {
            if (var) big_deep_kernel<BM, false, true><<<g, kThreads, 0, s>>>(a, tiles);
            else big_deep_kernel<BM, false, false><<<g, kThreads, 0, s>>>(a, tiles);
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

// Average rows per expert at or above which the 256-row tile is used.
constexpr int64_t kBigTile256MinRows = 512;

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

hipError_t launch_big_gemm(const Bf16Args& b, bool gemm1, hipStream_t s) {
    BigArgs a{b.T, b.D, b.H, b.E, b.k, b.P,
              reinterpret_cast<const uint8_t*>(b.x), nullptr,
              reinterpret_cast<const uint8_t*>(b.w1), nullptr,
              reinterpret_cast<const uint8_t*>(b.w2), nullptr,
              b.wts, b.rv, reinterpret_cast<uint8_t*>(b.act), nullptr, b.ypair, sink_of(b.mtiles, b.P, b.E), b.av};
    int4* tiles = reinterpret_cast<int4*>(b.mtiles);
    if (b.P >= kBigTile256MinRows * b.E) return launch_big<256, false>(a, tiles, gemm1, s);
    return launch_big<128, false>(a, tiles, gemm1, s);
}

// MX: 256-row tiles only (eight waves move the 512 scale rows of a stage);
// K stages of 64 codes must come in multiples of 4 (D and H multiples of 256).
bool big_mx_supported(const MxArgs& a) {
    const int64_t lim = int64_t(1) << 32;
    return a.mtiles != nullptr && a.P >= kBigTile256MinRows * a.E && a.D % 256 == 0 && a.H % 256 == 0 &&
           int64_t(a.T) * a.D < lim && a.P * a.H < lim && a.P * 4 < lim && int64_t(a.E) * 2 * a.H * a.D < lim;
}

hipError_t launch_big_mx(const MxArgs& b, bool gemm1, hipStream_t s) {
    BigArgs a{b.T,   b.D,   b.H,     b.E,  b.k,  b.P,      b.x,     b.xs,    b.w1,
              b.w1s, b.w2,  b.w2s,   b.wts, b.rv, b.act,   b.act_s, b.ypair, sink_of(b.mtiles, b.P, b.E)};
    return launch_big<256, true>(a, reinterpret_cast<int4*>(b.mtiles), gemm1, s);
}

}  // namespace moe
