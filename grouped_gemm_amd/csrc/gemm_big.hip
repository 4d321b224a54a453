// Prefill-shaped bf16 grouped GEMMs: many routed rows per expert.
//
// With hundreds to thousands of rows per expert the pass is bound by the
// matrix cores. A tile is BM token rows x 256 weight rows (GEMM1: 128 gate +
// 128 up rows, the gate/up pairing of "Prime Flash MoE", section 2, Trick 1;
// GEMM2: 256 output features). The weights are the MFMA's A operand
// (v_mfma_f32_32x32x16_bf16), so each lane's results are 4 consecutive
// features of one token. Eight waves (two per SIMD) split a tile into two
// feature halves x four token groups: 128 features x BM/4 tokens per wave.
//
// Persistent schedule. One workgroup per CU walks a list of tiles. Workgroup
// b runs on XCD b % 8 (8 XCDs, each with its own L2); the logical tiles,
// n-tile fastest, are split into 8 contiguous ranges, and the workgroups of
// an XCD take every (workgroups per XCD)-th tile of that XCD's range, so the
// n-tiles sharing a token tile run side by side and reuse it from one L2.
//
// K steps of 32 (64 bytes per row) go through a ring of 4 LDS stages filled
// by global->LDS DMA (global_load_lds_dwordx4: lane i's 16 bytes land at
// base + 16*i; 16 rows x 64 bytes per instruction): three stages are in
// flight while one is consumed, and the one barrier per stage sits between
// the MFMAs of the stage's two k-halves (see ring_step). The ring runs on
// across tiles: the next tile's row map (and, for GEMM2, its routing
// weights) arrive by DMA during the current tile's first steps, and its
// first four stages are issued during the current tile's last four, so
// neither the tile lookup nor the first loads' latency sits between two
// tiles. Results leave through a small per-wave LDS area as 64-byte row
// segments (see epilogue).
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
#include "common.h"

namespace moe {

namespace {

#ifndef MOE_BIG_WAVES
#define MOE_BIG_WAVES 8
#endif
constexpr int W = MOE_BIG_WAVES;   // waves per workgroup (2 feature halves x W/2 token groups)
constexpr int kThreads = 64 * W;
constexpr int BK = 32;             // K per stage
constexpr int RB = 64;             // bytes per tile row per stage
constexpr int BN = 256;            // weight rows per tile
constexpr int kInfoCap = 512;      // tile descriptors held in LDS at a time
constexpr int kMinPipelinedKT = 8; // K steps a tile needs for the in-loop hand-over

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

template <int BM>
struct Big {
    static constexpr int TB = BM / (W / 2);    // tokens per wave
    static constexpr int NT = TB / 32;         // token blocks per wave
    static constexpr int NF = 4;               // feature blocks per wave (128 features)
    static constexpr int A_INS = BM / 16 / W;  // token-row DMA instructions per wave per stage
    static constexpr int B_INS = BN / 16 / W;  // weight-row DMA instructions per wave per stage
    static constexpr int L = A_INS + B_INS;    // DMA instructions per wave per stage
    static constexpr int PW = BM / 64;         // waves that move one BM-entry int/float vector (64 per wave)
    static constexpr int TOK_BYTES = BM * RB, W_BYTES = BN * RB;
    static_assert(NT >= 1 && A_INS >= 1 && A_INS * 16 * W == BM && B_INS * 16 * W == BN, "tile split");
    static_assert(PW >= 1 && PW <= W, "row-vector DMA waves");
};

template <int BM>
struct StageBuf {
    uint8_t tok[Big<BM>::TOK_BYTES];
    uint8_t wt[Big<BM>::W_BYTES];
};

// Per-tile DMA sources: wave-uniform bases (scalar registers) plus 32-bit
// per-lane byte offsets. Token rows need one offset per instruction (they may
// be gathered); weight rows are consecutive and share `boff` + j * bstride,
// which does not change from tile to tile.
template <int BM>
struct DmaSrc {
    const char* abase;
    const char* bbase;
    uint32_t aoff[Big<BM>::A_INS];
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

template <int BM>
__device__ __forceinline__ void issue_stage(StageBuf<BM>& b, const DmaSrc<BM>& src, uint32_t boff, uint32_t bstride,
                                            int kt, uint32_t wave) {
    using C = Big<BM>;
    const char* ab = src.abase + kt * RB;
    const char* bb = src.bbase + kt * RB;
    const uint32_t tl = lds_addr(b.tok) + wave * (C::A_INS * 1024);
    const uint32_t wl = lds_addr(b.wt) + wave * (C::B_INS * 1024);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) dma16(ab, src.aoff[j], tl + j * 1024);
#pragma unroll
    for (int j = 0; j < C::B_INS; ++j) dma16(bb, boff + j * bstride, wl + j * 1024);
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

// s_barrier without a memory fence; the asm statements stop the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 16-wide k-half of a stage in registers: 4 weight fragments (32 rows
// each) and NT token fragments.
template <int BM>
struct Frag {
    bf16x8_t w[Big<BM>::NF];
    bf16x8_t t[Big<BM>::NT];
};

// Fragment reads of k-half kk of a stage: every fragment's 32 rows start at a
// multiple of 16, so a lane's row is (row base) + (lane & 31) and its swizzle
// term is ((lane & 31) >> 2) & 3.
template <int BM>
__device__ __forceinline__ void read_frag(const StageBuf<BM>& b, int kk, const int (&frow)[4], int tok_row0,
                                          Frag<BM>& f) {
    using C = Big<BM>;
    const int lane = threadIdx.x & 63;
    const int lrow = (lane & 31) * RB;
    const int coff = swz_chunk(lane & 31, 2 * kk + (lane >> 5)) << 4;
#pragma unroll
    for (int i = 0; i < C::NF; ++i) f.w[i] = *reinterpret_cast<const bf16x8_t*>(b.wt + frow[i] * RB + lrow + coff);
#pragma unroll
    for (int i = 0; i < C::NT; ++i)
        f.t[i] = *reinterpret_cast<const bf16x8_t*>(b.tok + (tok_row0 + 32 * i) * RB + lrow + coff);
}

template <int BM>
__device__ __forceinline__ void mfma_frag(const Frag<BM>& f, f32x16_t (&acc)[4][Big<BM>::NT]) {
    using C = Big<BM>;
#pragma unroll
    for (int i = 0; i < C::NF; ++i)
#pragma unroll
        for (int t = 0; t < C::NT; ++t) acc[i][t] = mfma32(f.w[i], f.t[t], acc[i][t]);
}

// Everything a workgroup keeps across the steps of a tile.
template <int BM>
struct Ring {
    DmaSrc<BM> src, nsrc;     // this tile's and the next tile's DMA sources
    uint32_t boff, bstride;   // weight-row offsets (the same for every tile)
    uint32_t wave;            // wave index (uniform)
    int KT;                   // K steps per tile
    bool pipelined;           // KT is long enough for the in-loop hand-over
    bool has_next;
    bool cont;                // the next tile's stages follow this tile's in the ring
    TileDesc next;            // the next tile (valid when has_next)
    int nb;                   // row-vector buffer of the next tile (0 or 1)
};

// DMA of a tile's row map: sorted_to_pair[row0 .. row0 + BM) -> pairs[0 .. BM).
// The map in the workspace is padded by 256 entries, so the window never
// leaves it; entries past the expert's rows are clamped before use.
template <int BM>
__device__ __forceinline__ void dma_row_map(const Bf16Args& a, int row0, int32_t* pairs, uint32_t wave) {
    if (wave < static_cast<uint32_t>(Big<BM>::PW)) {
        const uint32_t lane = threadIdx.x & 63;
        dma4(uniform_ptr(a.rv.sorted_to_pair + row0), (wave * 64 + lane) * 4u, lds_addr(pairs) + wave * 256);
    }
}

// DMA of a tile's routing weights: wts[pair of row r] -> w[r] (GEMM2).
template <int BM>
__device__ __forceinline__ void dma_row_weights(const Bf16Args& a, const int32_t* pairs, float* w, uint32_t wave) {
    if (wave < static_cast<uint32_t>(Big<BM>::PW)) {
        const int lane = threadIdx.x & 63;
        const int p = clamp_pair(pairs[wave * 64 + lane], a.P);
        dma4(uniform_ptr(a.wts), static_cast<uint32_t>(p) * 4u, lds_addr(w) + wave * 256);
    }
}

// DMA sources of a tile. GEMM1: token rows gathered through the row map;
// weight rows 0..127 are gate rows h0.., 128..255 up rows H + h0.. (a wave's
// rows never straddle the two). GEMM2: act rows in sorted order. Offsets are
// 32-bit: the host only picks this kernel when x, act and one expert's
// weights each span < 4 GiB. Instruction j of a wave covers tile rows
// (wave * INS + j) * 16 + lane / 4, chunk lane & 3.
template <int BM, bool GEMM1>
__device__ __forceinline__ void make_src(const Bf16Args& a, const TileDesc& t, const int32_t* pairs, uint32_t wave,
                                         DmaSrc<BM>& s) {
    using C = Big<BM>;
    const int lane = threadIdx.x & 63;
    const int K = GEMM1 ? a.D : a.H;
    s.abase = uniform_ptr(GEMM1 ? a.x : a.act + static_cast<int64_t>(t.row0) * a.H);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) {
        const int row = (static_cast<int>(wave) * C::A_INS + j) * 16 + lane / 4;
        const uint32_t r = GEMM1 ? static_cast<uint32_t>(clamp_pair(pairs[row], a.P) / a.k) * a.D
                                 : static_cast<uint32_t>(row < t.rows ? row : 0) * a.H;
        s.aoff[j] = r * 2 + swz_chunk(row, lane & 3) * 16;
    }
    const int row0 = static_cast<int>(wave) * C::B_INS * 16;  // first weight-tile row of this wave
    if (GEMM1) {
        const int h0 = t.ntile * 128;
        const int grow0 = row0 < 128 ? h0 + row0 : a.H + h0 + row0 - 128;
        s.bbase = uniform_ptr(a.w1 + (static_cast<int64_t>(t.expert) * 2 * a.H + grow0) * K);
    } else {
        s.bbase = uniform_ptr(a.w2 + (static_cast<int64_t>(t.expert) * a.D + t.ntile * 256 + row0) * K);
    }
}

// One ring step. The barrier sits in the middle of stage kt's MFMAs, so a
// wave never comes out of it with nothing to compute:
//   read k-half 1 of stage kt (buffer cur);  MFMAs of k-half 0 (read last step)
//   wait for this wave's DMAs of stage kt+1 and its own LDS reads;  barrier
//   issue stage kt+4 into cur (every wave is done reading it);
//   read k-half 0 of stage kt+1 (buffer nxt);  MFMAs of k-half 1
// Stage kt+4 belongs to this tile, or to the next one once this tile has
// none left, so the ring runs on across tiles.
//
// Waits: before the barrier each wave waits until its own DMAs of stage kt+1
// are done; the stages it issued after it (kt+2, kt+3, while they exist) may
// stay in flight. Loads, LDS DMA included, complete in order, so this holds
// with the previous tile's result stores or the few row-vector DMAs also in
// flight: at most 2L operations outstanding leaves at least as many of this
// wave's loads done as there were older ones.
//
// Hand-over (pipelined tiles): step 0 fetches the next tile's row map,
// complete by step 3's barrier; step 3 builds the next tile's DMA sources
// from it and fetches its routing weights (GEMM2), complete by step 6's
// barrier; steps KT-4 .. KT-1 issue its stages 0..3.
template <int BM, bool GEMM1>
__device__ __forceinline__ void ring_step(const Bf16Args& a, Ring<BM>& r, StageBuf<BM>& cur,
                                          const StageBuf<BM>& nxt, int kt, int32_t (*pairs)[BM], float (*wrow)[BM],
                                          const int (&frow)[4], int tok_row0, Frag<BM>& f0, Frag<BM>& f1,
                                          f32x16_t (&acc)[4][Big<BM>::NT]) {
    constexpr int L = Big<BM>::L;
    read_frag<BM>(cur, 1, frow, tok_row0, f1);
    mfma_frag<BM>(f0, acc);
    const bool more1 = kt + 1 < r.KT || r.cont;  // stage kt+1 exists
    if (kt + 3 < r.KT || r.cont) wait_vm_lds<2 * L>();
    else if (kt + 2 < r.KT) wait_vm_lds<L>();
    else wait_vm_lds<0>();
    bare_barrier();
    if (r.cont) {
        if (kt == 0) dma_row_map<BM>(a, r.next.row0, pairs[r.nb], r.wave);
        if (kt == 3) {
            make_src<BM, GEMM1>(a, r.next, pairs[r.nb], r.wave, r.nsrc);
            if (!GEMM1) dma_row_weights<BM>(a, pairs[r.nb], wrow[r.nb], r.wave);
        }
    }
    if (kt + 4 < r.KT) issue_stage<BM>(cur, r.src, r.boff, r.bstride, kt + 4, r.wave);
    else if (r.cont) issue_stage<BM>(cur, r.nsrc, r.boff, r.bstride, kt + 4 - r.KT, r.wave);
    if (more1) read_frag<BM>(nxt, 0, frow, tok_row0, f0);
    mfma_frag<BM>(f1, acc);
}

// The stage buffers come in as restrict pointers: with them, the compiler
// knows the fragment reads of one stage never alias the others.
template <int BM, bool GEMM1>
__device__ __forceinline__ void main_loop(const Bf16Args& a, Ring<BM>& r, StageBuf<BM>* __restrict__ b0,
                                          StageBuf<BM>* __restrict__ b1, StageBuf<BM>* __restrict__ b2,
                                          StageBuf<BM>* __restrict__ b3, int32_t (*pairs)[BM], float (*wrow)[BM],
                                          const int (&frow)[4], int tok_row0, Frag<BM>& f0, Frag<BM>& f1,
                                          f32x16_t (&acc)[4][Big<BM>::NT]) {
    // KT is a multiple of 4 (K is a multiple of 128): the unrolled body needs
    // no exit in the middle, which would make the compiler shuttle the
    // accumulators between registers at the loop head. Every tile starts at
    // buffer 0.
    for (int kt = 0; kt < r.KT; kt += 4) {
        ring_step<BM, GEMM1>(a, r, *b0, *b1, kt, pairs, wrow, frow, tok_row0, f0, f1, acc);
        ring_step<BM, GEMM1>(a, r, *b1, *b2, kt + 1, pairs, wrow, frow, tok_row0, f0, f1, acc);
        ring_step<BM, GEMM1>(a, r, *b2, *b3, kt + 2, pairs, wrow, frow, tok_row0, f0, f1, acc);
        ring_step<BM, GEMM1>(a, r, *b3, *b0, kt + 3, pairs, wrow, frow, tok_row0, f0, f1, acc);
    }
}

// Issue stages 0..3 of a tile, wait for stage 0 and read its first k-half.
template <int BM>
__device__ __forceinline__ void ring_start(Ring<BM>& r, const DmaSrc<BM>& src, StageBuf<BM>& b0, StageBuf<BM>& b1,
                                           StageBuf<BM>& b2, StageBuf<BM>& b3, const int (&frow)[4], int tok_row0,
                                           Frag<BM>& f0) {
    constexpr int L = Big<BM>::L;
    issue_stage<BM>(b0, src, r.boff, r.bstride, 0, r.wave);
    issue_stage<BM>(b1, src, r.boff, r.bstride, 1, r.wave);
    issue_stage<BM>(b2, src, r.boff, r.bstride, 2, r.wave);
    issue_stage<BM>(b3, src, r.boff, r.bstride, 3, r.wave);
    wait_vm<3 * L>();
    bare_barrier();
    read_frag<BM>(b0, 0, frow, tok_row0, f0);
}

// Results of a tile. acc[f][t][4i + j] holds feature frow[f] + 8i +
// 4*(lane>>5) + j of token row tok_row0 + 32t + (lane & 31): a lane holds 8
// bytes of a row per register group. Each 32-row x 32-feature block goes
// through the wave's own 2 KB of LDS (row r at r * 64, its 16-byte chunk c
// at (c ^ ((r >> 2) & 3)) * 16: both the 8-byte writes and the 16-byte
// reads hit distinct banks) and leaves as 64-byte row segments, 4 lanes x 16
// bytes each: a quarter of the write requests of storing the 8-byte pieces.
// The area is the wave's own, so no barrier is needed; LDS accesses of one
// wave complete in order.
// GEMM1 writes act = silu(gate) * up (bf16) at act[row0 + row][h0 + col];
// GEMM2 writes w * y (bf16) at ypair[pair][n0 + feature].
template <int BM, bool GEMM1>
__device__ __forceinline__ void epilogue(const Bf16Args& a, const TileDesc& t, const int32_t* pairs, const float* w,
                                         int tok_row0, int wf, uint8_t* stg, const f32x16_t (&acc)[4][Big<BM>::NT]) {
    using C = Big<BM>;
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, g = lane >> 5;
    const int wr = r * 64 + 8 * g, wsw = (r >> 2) & 3;  // staging writes: row r, half g of chunk i
    const int rr = lane >> 2, c = lane & 3;              // staging reads: rows rr and rr + 16, chunk c
    const int rd0 = rr * 64 + ((c ^ ((rr >> 2) & 3)) << 4);
    const int rd1 = (rr + 16) * 64 + ((c ^ (((rr + 16) >> 2) & 3)) << 4);
#pragma unroll
    for (int tb = 0; tb < C::NT; ++tb) {
        const int base = tok_row0 + 32 * tb;
        const bool ok0 = base + rr < t.rows, ok1 = base + rr + 16 < t.rows;
        uint16_t* d0;
        uint16_t* d1;
        if (GEMM1) {
            const int64_t col = t.ntile * 128 + 64 * wf + 8 * c;
            d0 = a.act + static_cast<int64_t>(t.row0 + base + rr) * a.H + col;
            d1 = d0 + static_cast<int64_t>(16) * a.H;
        } else {
            const int64_t col = t.ntile * 256 + 128 * wf + 8 * c;
            d0 = a.ypair + static_cast<int64_t>(clamp_pair(pairs[base + rr], a.P)) * a.D + col;
            d1 = a.ypair + static_cast<int64_t>(clamp_pair(pairs[base + rr + 16], a.P)) * a.D + col;
        }
        const float wt = GEMM1 ? 1.0f : w[base + r];
#pragma unroll
        for (int f = 0; f < (GEMM1 ? 2 : 4); ++f) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = acc[f][tb][4 * i + j];
                    v[j] = GEMM1 ? x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)) * acc[f + 2][tb][4 * i + j] : x * wt;
                }
                *reinterpret_cast<uint2*>(stg + wr + ((i ^ wsw) << 4)) =
                    uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
            const u32x4_t q0 = *reinterpret_cast<const u32x4_t*>(stg + rd0);
            const u32x4_t q1 = *reinterpret_cast<const u32x4_t*>(stg + rd1);
            if (ok0) *reinterpret_cast<u32x4_t*>(d0 + 32 * f) = q0;
            if (ok1) *reinterpret_cast<u32x4_t*>(d1 + 32 * f) = q1;
        }
    }
}

// Descriptors of this workgroup's tiles c0 .. c0 + kInfoCap - 1 into LDS.
__device__ __forceinline__ void load_descs(const int4* mtiles, int first, int stride, int ny, int count, int c0,
                                           TileDesc* desc) {
    for (int i = threadIdx.x; i < kInfoCap && c0 + i < count; i += kThreads) {
        const int logical = first + (c0 + i) * stride;
        const int m = logical / ny;
        const int4 d = mtiles[m];
        desc[i] = TileDesc{d.x, d.y, d.z, logical - m * ny};
    }
}

__device__ __forceinline__ TileDesc uniform_desc(const TileDesc& d) {
    return TileDesc{uniform_int(d.expert), uniform_int(d.row0), uniform_int(d.rows), uniform_int(d.ntile)};
}

template <int BM, bool GEMM1>
__global__ __launch_bounds__(kThreads, 1) void big_gemm_kernel(Bf16Args a, const int4* __restrict__ mtiles) {
    using C = Big<BM>;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf0;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf1;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf2;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf3;
    __shared__ __attribute__((aligned(16))) int32_t sPair[2][BM];
    __shared__ __attribute__((aligned(16))) float sW[2][BM];
    __shared__ TileDesc sDesc[kInfoCap];
    __shared__ __attribute__((aligned(16))) uint8_t sOut[W][2048];  // per-wave result staging

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
    int frow[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
        frow[f] = GEMM1 ? (f < 2 ? 64 * wf + 32 * f : 128 + 64 * wf + 32 * (f - 2)) : 128 * wf + 32 * f;
    const int tok_row0 = wtok * C::TB;

    Ring<BM> r;
    r.wave = static_cast<uint32_t>(uniform_int(wave_v));
    const int K = GEMM1 ? a.D : a.H;
    r.KT = K / BK;
    r.pipelined = r.KT >= kMinPipelinedKT;
    {
        const int lane = tid & 63;
        const int row = static_cast<int>(r.wave) * C::B_INS * 16 + lane / 4;  // +16 rows per instruction
        r.boff = static_cast<uint32_t>(lane / 4) * K * 2 + swz_chunk(row, lane & 3) * 16;
        r.bstride = 16u * K * 2;
    }

    load_descs(mtiles, first, stride, ny, count, 0, sDesc);
    __syncthreads();
    TileDesc t = uniform_desc(sDesc[0]);

    // first tile: row map (and weights) now, then its first four stages
    int cb = 0;
    dma_row_map<BM>(a, t.row0, sPair[0], r.wave);
    wait_vm<0>();
    bare_barrier();
    make_src<BM, GEMM1>(a, t, sPair[0], r.wave, r.src);
    if (!GEMM1) {
        dma_row_weights<BM>(a, sPair[0], sW[0], r.wave);
        wait_vm<0>();
        bare_barrier();
    }
    Frag<BM> f0, f1;
    ring_start<BM>(r, r.src, buf0, buf1, buf2, buf3, frow, tok_row0, f0);

    f32x16_t acc[4][C::NT];
    for (int i = 0; i < count; ++i) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int tb = 0; tb < C::NT; ++tb) acc[f][tb] = f32x16_t{};
        r.has_next = i + 1 < count;
        r.nb = cb ^ 1;
        if (r.has_next) {
            if ((i + 1) % kInfoCap == 0) {  // next descriptor chunk; t stays in registers
                __syncthreads();
                load_descs(mtiles, first, stride, ny, count, i + 1, sDesc);
                __syncthreads();
            }
            r.next = uniform_desc(sDesc[(i + 1) % kInfoCap]);
        }
        r.cont = r.has_next && r.pipelined;

        main_loop<BM, GEMM1>(a, r, &buf0, &buf1, &buf2, &buf3, sPair, sW, frow, tok_row0, f0, f1, acc);

        if (r.has_next && !r.pipelined) {
            // short K: hand over after the ring has drained
            dma_row_map<BM>(a, r.next.row0, sPair[r.nb], r.wave);
            wait_vm<0>();
            bare_barrier();
            make_src<BM, GEMM1>(a, r.next, sPair[r.nb], r.wave, r.nsrc);
            if (!GEMM1) {
                dma_row_weights<BM>(a, sPair[r.nb], sW[r.nb], r.wave);
                wait_vm<0>();
                bare_barrier();
            }
            ring_start<BM>(r, r.nsrc, buf0, buf1, buf2, buf3, frow, tok_row0, f0);
        }
        epilogue<BM, GEMM1>(a, t, sPair[cb], sW[cb], tok_row0, wf, sOut[wave_v], acc);
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

int num_cus() {
    static const int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        return v;
    }();
    return n;
}

}  // namespace

// Average rows per expert at or above which the 256-row tile is used.
constexpr int64_t kBigTile256MinRows = 512;

int64_t big_gemm_mtile_capacity(int64_t P, int E) { return (P + 127) / 128 + E; }

bool big_gemm_supported(const Bf16Args& a) {
    const int64_t lim = int64_t(1) << 32;  // the DMA offsets are 32-bit
    return a.mtiles != nullptr && a.D % 256 == 0 && a.H % 128 == 0 && int64_t(a.T) * a.D * 2 < lim &&
           a.P * a.H * 2 < lim && a.P * 4 < lim && int64_t(2) * a.H * a.D * 2 < lim;
}

hipError_t launch_big_gemm(const Bf16Args& a, bool gemm1, hipStream_t s) {
    const bool t256 = a.P >= kBigTile256MinRows * a.E;
    const int bm = t256 ? 256 : 128;
    int4* tiles = reinterpret_cast<int4*>(a.mtiles);
    if (gemm1) {  // the m-tiles are the same for both GEMMs
        if (t256) mtile_table_kernel<256><<<a.E, 64, 0, s>>>(a.rv, a.E, tiles);
        else mtile_table_kernel<128><<<a.E, 64, 0, s>>>(a.rv, a.E, tiles);
    }
    // one workgroup per CU (a multiple of 8: the same number on every XCD),
    // never many more than there can be tiles
    const int ny = gemm1 ? a.H / 128 : a.D / 256;
    const int64_t tiles_upper = ((a.P + bm - 1) / bm + a.E) * ny;
    int64_t grid = num_cus();
    if (grid > tiles_upper) grid = tiles_upper;
    grid = (grid + 7) / 8 * 8;
    const int g = static_cast<int>(grid);
    if (t256) {
        if (gemm1) big_gemm_kernel<256, true><<<g, kThreads, 0, s>>>(a, tiles);
        else big_gemm_kernel<256, false><<<g, kThreads, 0, s>>>(a, tiles);
    } else {
        if (gemm1) big_gemm_kernel<128, true><<<g, kThreads, 0, s>>>(a, tiles);
        else big_gemm_kernel<128, false><<<g, kThreads, 0, s>>>(a, tiles);
    }
    return hipGetLastError();
}

}  // namespace moe
