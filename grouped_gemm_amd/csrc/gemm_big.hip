// Prefill-shaped bf16 grouped GEMMs: many routed rows per expert.
//
// With hundreds to thousands of rows per expert the pass is bound by the
// matrix cores. A workgroup (4 waves) computes a tile of BM token rows x 256
// weight rows (GEMM1: 128 gate + 128 up rows, the gate/up pairing of "Prime
// Flash MoE", section 2, Trick 1; GEMM2: 256 output features). The weights
// are the MFMA's A operand (v_mfma_f32_32x32x16_bf16), so each lane's
// results are 4 consecutive features of one token and the epilogues write
// them as packed 8-byte rows.
//
// Each wave owns 128 features x BM/2 tokens: per 16-wide k-step it reads 4
// weight and BM/64 token fragments from LDS for 4*BM/64 MFMAs.
//
// K steps of 32 (64 bytes per row) go through a ring of 4 LDS stages filled
// by global->LDS DMA (global_load_lds_dwordx4: lane i's 16 bytes land at
// base + 16*i; 16 rows x 64 bytes per instruction), so three stages are in
// flight while one is consumed: enough lead to cover L2 misses. The 16-byte
// chunks of a row are XOR-swizzled by ((row >> 2) & 3): gfx950's LDS serves
// 16 lanes of a 16-byte read per cycle from 64 banks (256 bytes), and the 16
// consecutive rows a fragment read touches then fall in 16 distinct 16-byte
// bank groups. The four stages are distinct LDS objects and the loop is
// unrolled by four, so the compiler sees that the fragment reads of one stage
// never alias the DMA filling another; the waits are explicit per-wave
// vmcnt budgets and the barrier carries no memory fence (a fence would wait
// for every DMA in flight).
//
// Token rows of GEMM1 are gathered on load (row r reads token
// sorted_to_pair[row0 + r] / k); rows past an expert's count read a valid
// row and are not stored. Tiles are mapped to workgroups XCD by XCD (see
// xcd_tile) so that the tiles sharing a token tile reuse it from one L2.
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int BK = 32;    // K per stage
constexpr int RB = 64;    // bytes per tile row per stage
constexpr int BN = 256;   // weight rows per tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

template <int BM>
struct Big {
    static constexpr int TB = BM / 2;          // tokens per wave
    static constexpr int NT = TB / 32;         // token blocks per wave
    static constexpr int NF = 4;               // feature blocks per wave (128 features)
    static constexpr int A_INS = BM / 16 / 4;  // token-row DMA instructions per wave per stage
    static constexpr int B_INS = BN / 16 / 4;  // weight-row DMA instructions per wave per stage
    static constexpr int L = A_INS + B_INS;    // DMA instructions per wave per stage
    static constexpr int TOK_BYTES = BM * RB, W_BYTES = BN * RB;
};

template <int BM>
struct StageBuf {
    uint8_t tok[Big<BM>::TOK_BYTES];
    uint8_t wt[Big<BM>::W_BYTES];
};

// DMA sources: wave-uniform bases plus 32-bit per-lane byte offsets (the saddr
// form of the DMA). Token rows need one offset per instruction (they may be
// gathered); weight rows are consecutive (instruction j reads 16 rows after
// instruction j-1: a fixed stride).
struct DmaSrc {
    const char* abase;
    const char* bbase;
    uint32_t bstride;
};

template <int BM>
__device__ __forceinline__ void issue_stage(StageBuf<BM>& b, const DmaSrc& src, const uint32_t* aoff, uint32_t boff,
                                            int kt) {
    using C = Big<BM>;
    const int wave = threadIdx.x >> 6;
    const char* ab = src.abase + kt * RB;
    const char* bb = src.bbase + kt * RB;
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j)
        __builtin_amdgcn_global_load_lds(ab + aoff[j], (lds_ptr_t)(b.tok + (wave * C::A_INS + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < C::B_INS; ++j)
        __builtin_amdgcn_global_load_lds(bb + (boff + j * src.bstride), (lds_ptr_t)(b.wt + (wave * C::B_INS + j) * 1024),
                                         16, 0, 0);
}

// wait until at most n vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_barrier without a memory fence; the asm statements stop the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Fragment reads of one stage: every fragment's 32 rows start at a multiple
// of 16, so a lane's row is (row base) + (lane & 31) and its swizzle term is
// ((lane & 31) >> 2) & 3.
template <int BM>
__device__ __forceinline__ void compute_stage(const StageBuf<BM>& b, const int (&frow)[4], int tok_row0,
                                              f32x16_t (&acc)[4][Big<BM>::NT]) {
    using C = Big<BM>;
    const int lane = threadIdx.x & 63;
    const int lrow = (lane & 31) * RB;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        const int coff = swz_chunk(lane & 31, 2 * kk + (lane >> 5)) << 4;
        bf16x8_t wf[C::NF], tf[C::NT];
#pragma unroll
        for (int f = 0; f < C::NF; ++f) wf[f] = *reinterpret_cast<const bf16x8_t*>(b.wt + frow[f] * RB + lrow + coff);
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
            tf[t] = *reinterpret_cast<const bf16x8_t*>(b.tok + (tok_row0 + 32 * t) * RB + lrow + coff);
#pragma unroll
        for (int f = 0; f < C::NF; ++f)
#pragma unroll
            for (int t = 0; t < C::NT; ++t) acc[f][t] = mfma32(wf[f], tf[t], acc[f][t]);
    }
}

// Consume stage kt from buffer `cur`, after issuing stage kt+3 into `nxt`
// (the buffer consumed one step earlier, free once every wave has passed
// this step's barrier). Before the barrier each wave waits until its own DMAs
// of stage kt are done: the newer stages it has issued (kt+1, kt+2 while they
// exist) may stay in flight.
template <int BM>
__device__ __forceinline__ void ring_step(const StageBuf<BM>& cur, StageBuf<BM>& nxt, const DmaSrc& src,
                                          const uint32_t* aoff, uint32_t boff, int kt, int KT, const int (&frow)[4],
                                          int tok_row0, f32x16_t (&acc)[4][Big<BM>::NT]) {
    constexpr int L = Big<BM>::L;
    if (kt + 2 < KT) wait_vm<2 * L>();
    else if (kt + 1 < KT) wait_vm<L>();
    else wait_vm<0>();
    bare_barrier();
    if (kt + 3 < KT) issue_stage<BM>(nxt, src, aoff, boff, kt + 3);
    compute_stage<BM>(cur, frow, tok_row0, acc);
}

// 1-D grid of at least (m-tiles upper bound) x NY blocks, a multiple of 8.
// Workgroup b runs on XCD b % 8 (8 XCDs, each with its own L2). The actual
// tile count T is read from the route step; the logical tiles, n-tile
// fastest, are split into 8 contiguous ranges of ceil(T*NY/8), and XCD x walks
// range x in order. The NY tiles sharing one token tile then run back to
// back on one XCD and reuse it from that XCD's L2.
template <int BM>
__device__ __forceinline__ bool xcd_tile(const RouteView& rv, int E, int ny, int& mtile, int& ntile) {
    const int tiles = rv.tile_prefix[tile_height_index(BM) * (E + 1) + E];
    const int total = tiles * ny;
    const int per = (total + 7) / 8;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((blockIdx.x >> 3) >= per || logical >= total) return false;
    mtile = logical / ny;
    ntile = logical - mtile * ny;
    return true;
}

// Staged output rows: [tokens][128 features] bf16, 256 bytes per row, 16-byte
// chunks XOR-swizzled by (token & 15).
__device__ __forceinline__ int stage_off(int tok, int col) {
    return tok * 256 + ((((col >> 3) ^ (tok & 15)) << 4) | ((col & 7) << 1));
}

template <int BM, bool GEMM1>
__global__ __launch_bounds__(kThreads, 1) void big_gemm_kernel(Bf16Args a) {
    using C = Big<BM>;
    constexpr int HALF = BM / 2;  // tokens staged in each of buffers 0 and 1
    static_assert(HALF * 256 <= static_cast<int>(sizeof(StageBuf<BM>)), "output staging fits two stage buffers");
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf0;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf1;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf2;
    __shared__ __attribute__((aligned(16))) StageBuf<BM> buf3;
    __shared__ int32_t sRow[BM];
    __shared__ float sW[BM];
    const int ny = GEMM1 ? a.H / 128 : a.D / 256;
    int mtile, ntile;
    if (!xcd_tile<BM>(a.rv, a.E, ny, mtile, ntile)) return;
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, mtile, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wtok = wave >> 1, wf = wave & 1;
    for (int r = tid; r < BM; r += kThreads) {
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P);
        sRow[r] = GEMM1 ? p / a.k : p;
        if (!GEMM1) sW[r] = a.wts[p];
    }
    __syncthreads();
    const int K = GEMM1 ? a.D : a.H;
    const int h0 = ntile * 128;  // GEMM1: act columns of this tile
    const int n0 = ntile * 256;  // GEMM2: output features of this tile

    // DMA sources. Offsets are 32-bit: the host only picks this kernel when x,
    // act and one expert's weights each span < 4 GiB. Instruction j of a wave
    // covers tile rows (wave * INS + j) * 16 + lane / 4, chunk lane & 3.
    DmaSrc src;
    uint32_t aoff[C::A_INS];
    src.abase = reinterpret_cast<const char*>(GEMM1 ? a.x : a.act + static_cast<int64_t>(mt.row0) * a.H);
#pragma unroll
    for (int j = 0; j < C::A_INS; ++j) {
        const int row = (wave * C::A_INS + j) * 16 + lane / 4;
        const uint32_t r = GEMM1 ? static_cast<uint32_t>(sRow[row]) * a.D
                                 : static_cast<uint32_t>(row < mt.rows ? row : 0) * a.H;
        aoff[j] = r * 2 + swz_chunk(row, lane & 3) * 16;
    }
    uint32_t boff;
    {
        const int row0 = wave * C::B_INS * 16;  // first weight-tile row of this wave's instructions
        const int row = row0 + lane / 4;        // later instructions: +16 rows, same swizzle term
        if (GEMM1) {
            // tile rows 0..127 are gate rows h0.., 128..255 up rows H+h0..; a wave's 64 rows never straddle
            const int64_t e0 = static_cast<int64_t>(mt.expert) * 2 * a.H;
            const int grow0 = row0 < 128 ? h0 + row0 : a.H + h0 + row0 - 128;
            src.bbase = reinterpret_cast<const char*>(a.w1 + (e0 + grow0) * K);
        } else {
            src.bbase = reinterpret_cast<const char*>(a.w2 + (static_cast<int64_t>(mt.expert) * a.D + n0 + row0) * K);
        }
        boff = static_cast<uint32_t>(lane / 4) * K * 2 + swz_chunk(row, lane & 3) * 16;
        src.bstride = 16u * K * 2;
    }
    int frow[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
        frow[f] = GEMM1 ? (f < 2 ? 64 * wf + 32 * f : 128 + 64 * wf + 32 * (f - 2)) : 128 * wf + 32 * f;
    const int tok_row0 = wtok * C::TB;
    f32x16_t acc[4][C::NT];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < C::NT; ++t) acc[f][t] = f32x16_t{};

    // K / 32 is a multiple of 4 (K is a multiple of 128): the unrolled body
    // needs no exit in the middle, which would make the compiler shuttle the
    // accumulators between AGPRs and VGPRs at the loop head.
    const int KT = K / BK;
    issue_stage<BM>(buf0, src, aoff, boff, 0);
    issue_stage<BM>(buf1, src, aoff, boff, 1);
    issue_stage<BM>(buf2, src, aoff, boff, 2);
    for (int kt = 0; kt < KT; kt += 4) {
        ring_step<BM>(buf0, buf3, src, aoff, boff, kt, KT, frow, tok_row0, acc);
        ring_step<BM>(buf1, buf0, src, aoff, boff, kt + 1, KT, frow, tok_row0, acc);
        ring_step<BM>(buf2, buf1, src, aoff, boff, kt + 2, KT, frow, tok_row0, acc);
        ring_step<BM>(buf3, buf2, src, aoff, boff, kt + 3, KT, frow, tok_row0, acc);
    }

    // Epilogue. acc[f][t][4i + j] holds feature frow[f] + 8i + 4*(lane>>5) + j
    // of token tok_row0 + 32t + (lane & 31). The output rows are staged in LDS
    // (tokens below HALF in buffer 0, the rest in buffer 1), then written as
    // 16-byte chunks, 16 lanes per 256-byte row. GEMM2's 256 features go in two
    // passes of 128.
    const int g4 = 4 * (lane >> 5);
    for (int pass = 0; pass < (GEMM1 ? 1 : 2); ++pass) {
        __syncthreads();
        if (GEMM1 || wf == pass) {
#pragma unroll
            for (int t = 0; t < C::NT; ++t) {
                const int tok = tok_row0 + 32 * t + (lane & 31);
                uint8_t* stg = reinterpret_cast<uint8_t*>(tok < HALF ? &buf0 : &buf1);
                const int tl = tok < HALF ? tok : tok - HALF;
                const float wt = GEMM1 ? 1.0f : sW[tok];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int f = 0; f < (GEMM1 ? 2 : 4); ++f) {
                        float v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float x = acc[f][t][4 * i + j];
                            v[j] = GEMM1 ? x / (1.0f + __expf(-x)) * acc[f + 2][t][4 * i + j] : x * wt;
                        }
                        // staged column: GEMM1 act column, GEMM2 feature within this pass's 128
                        const int col = (GEMM1 ? 64 * wf + 32 * f : 32 * f) + 8 * i + g4;
                        *reinterpret_cast<uint2*>(stg + stage_off(tl, col)) =
                            uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    }
                }
            }
        }
        __syncthreads();
        for (int idx = tid; idx < BM * 16; idx += kThreads) {
            const int r = idx >> 4, c = idx & 15;
            if (r >= mt.rows) continue;
            const uint8_t* stg = reinterpret_cast<const uint8_t*>(r < HALF ? &buf0 : &buf1);
            const int rl = r < HALF ? r : r - HALF;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rl * 256 + ((c ^ (rl & 15)) << 4));
            uint16_t* dst = GEMM1 ? a.act + static_cast<int64_t>(mt.row0 + r) * a.H + h0 + c * 8
                                  : a.ypair + static_cast<int64_t>(sRow[r]) * a.D + n0 + 128 * pass + c * 8;
            *reinterpret_cast<u32x4_t*>(dst) = v;
        }
    }
}

inline int mtiles_upper(int64_t P, int E, int bm) { return static_cast<int>((P + bm - 1) / bm + E); }

}  // namespace

// Average rows per expert at or above which the 256-row tile is used.
constexpr int64_t kBigTile256MinRows = 512;

bool big_gemm_supported(const Bf16Args& a) {
    const int64_t lim = int64_t(1) << 32;  // the DMA offsets are 32-bit
    return a.D % 256 == 0 && a.H % 128 == 0 && int64_t(a.T) * a.D * 2 < lim && a.P * a.H * 2 < lim &&
           int64_t(2) * a.H * a.D * 2 < lim;
}

hipError_t launch_big_gemm(const Bf16Args& a, bool gemm1, hipStream_t s) {
    const bool t256 = a.P >= kBigTile256MinRows * a.E;
    const int ny = gemm1 ? a.H / 128 : a.D / 256;
    const int64_t blocks = static_cast<int64_t>(mtiles_upper(a.P, a.E, t256 ? 256 : 128)) * ny;
    const int grid = static_cast<int>((blocks + 7) / 8 * 8);
    if (t256) {
        if (gemm1) big_gemm_kernel<256, true><<<grid, kThreads, 0, s>>>(a);
        else big_gemm_kernel<256, false><<<grid, kThreads, 0, s>>>(a);
    } else {
        if (gemm1) big_gemm_kernel<128, true><<<grid, kThreads, 0, s>>>(a);
        else big_gemm_kernel<128, false><<<grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
