// MX-fp8 pieces of the MoE SwiGLU FFN on gfx950.
//
// Data format ("Prime Flash MoE", section 7): e4m3 codes with one e8m0
// scale (value 2^(byte-127)) per 32 contiguous elements along K. Scale rule
// ("Porting Block-Scaled GEMM Kernels from Blackwell to Rubin", section
// 6.2, read as: the scale byte is amax/448 rounded up to a power of two):
// s = the smallest integer with amax <= 448 * 2^s, clamped to [-127, 127];
// codes = e4m3(v * 2^-s), round to nearest even, saturating at 448.
// s is read off amax's exponent and mantissa bits, so no division is made.
//
// GEMMs: v_mfma_scale_f32_32x32x64_f8f6f4 takes 32 e4m3 codes per lane for
// A (row lane&31) and B (column lane&31) and one e8m0 scale per lane. With
// g = lane>>5, a lane's first 16 codes are k = 16g..16g+15 of the MFMA's 64
// (scale block 0) and its last 16 are k = 32+16g..32+16g+15 (block 1);
// lanes of group g supply the scale of block g for their row or column
// (layout measured on gfx950 with an in-bounds probe). Tiles are staged
// like the bf16 kernels: 128 codes (128 bytes) of K per row per stage,
// 16-byte chunks XOR-swizzled by ((row >> 1) & 7) (16 rows read together hit
// 16 distinct 16-byte bank groups of gfx950's 64-bank LDS), double-buffered.
//
// GEMM1's epilogue computes SwiGLU in fp32, stages the act tile in LDS and
// requantizes it per 32 along H with the same rule (section 7, "The
// epilogue also quantizes"), writing codes [P, H] and scales [P, H/32].
#include "common.h"
#include "mxq.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int BKB = 128;  // K bytes (= codes) per stage

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ int acc_row(int lane, int v) { return ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3); }

// ---------------- standalone quantizer ----------------
// 8 lanes per 32-element block, 4 values per lane.
__global__ __launch_bounds__(256) void mx_quantize_kernel(const float* __restrict__ src, int64_t nblk,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    const int sub = threadIdx.x & 7;
    for (int64_t b = (blockIdx.x * 256ll + threadIdx.x) >> 3; b < nblk;
         b += (static_cast<int64_t>(gridDim.x) * 256) >> 3) {
        const float4 v = *reinterpret_cast<const float4*>(src + b * 32 + sub * 4);
        float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
        const int s = mx_scale_exp(amax);
        const float inv = pow2f(-s);
        const uint32_t c = e4m3_encode(v.x * inv, v.x) | (e4m3_encode(v.y * inv, v.y) << 8) |
                           (e4m3_encode(v.z * inv, v.z) << 16) | (e4m3_encode(v.w * inv, v.w) << 24);
        *reinterpret_cast<uint32_t*>(codes + b * 32 + sub * 4) = c;
        if (sub == 0) scales[b] = static_cast<uint8_t>(s + 127);
    }
}

// MXQ4 quantizer (packed e2m1 codes, even index in the low nibble): 8 lanes
// per 32-element block, 4 values (2 bytes) per lane.
__global__ __launch_bounds__(256) void mx4_quantize_kernel(const float* __restrict__ src, int64_t nblk,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
    const int sub = threadIdx.x & 7;
    for (int64_t b = (blockIdx.x * 256ll + threadIdx.x) >> 3; b < nblk;
         b += (static_cast<int64_t>(gridDim.x) * 256) >> 3) {
        const float4 v = *reinterpret_cast<const float4*>(src + b * 32 + sub * 4);
        float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
        const int s = mx4_scale_exp(amax);
        const float inv = pow2f(-s);
        const uint32_t c = e2m1_encode(v.x * inv, v.x) | (e2m1_encode(v.y * inv, v.y) << 4) |
                           (e2m1_encode(v.z * inv, v.z) << 8) | (e2m1_encode(v.w * inv, v.w) << 12);
        *reinterpret_cast<uint16_t*>(codes + b * 16 + sub * 2) = static_cast<uint16_t>(c);
        if (sub == 0) scales[b] = static_cast<uint8_t>(s + 127);
    }
}

// ---------------- block-scaled grouped GEMM main loop ----------------
// acc[mi][nj] += A . B^T with e8m0 scales. aptr/bptr: this thread's 16-byte
// chunk of stage 0 for each of its rows; asp/bsp: per (wave block, lane) the
// scale row of that lane's A row / B row (K/32 bytes per row).
//
// W4: B holds MXFP4 weights, packed e2m1 codes (64 bytes per row per stage
// of 128 K values; staged rows of 64 bytes with their four 16-byte chunks
// swizzled by ((row >> 2) & 3)). For an e2m1 operand the scaled MFMA takes
// 32 contiguous values per lane: lane group g holds k = 32g..32g+31 of the
// 64-wide step, 16 bytes (measured on gfx950 with an in-bounds probe).
template <int BM, int BN, bool W4 = false>
struct MxTile {
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int MB = WM / 32, NB = WN / 32;
    static constexpr int BRB = W4 ? BKB / 2 : BKB;  // B bytes per row per stage
    static constexpr int A_CH = BM * 8 / kThreads;
    static constexpr int B_CH = BN * (BRB / 16) / kThreads;
    static constexpr int STAGE = BM * BKB + BN * BRB;  // bytes
};

// 64-byte staged rows, 16-byte chunk c of row r at (c ^ ((r >> 2) & 3)): the 16
// rows a fragment read touches fall in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz64(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

template <int BM, int BN, bool W4>
__device__ __forceinline__ void mx_mainloop(uint8_t* lds, const uint8_t* const* aptr, const uint8_t* const* bptr,
                                            const uint8_t* const* asp, const uint8_t* const* bsp, int KT,
                                            const int* brow,
                                            f32x16_t (&acc)[MxTile<BM, BN, W4>::MB][MxTile<BM, BN, W4>::NB]) {
    using C = MxTile<BM, BN, W4>;
    const int tid = threadIdx.x, lane = tid & 63, wm = (tid >> 6) >> 1;
    const int c16 = tid & 7, r16 = tid >> 3;
    const int c4 = tid & 3, r4 = tid >> 2;  // W4: chunk and row of this thread's B loads
    u32x4_t ra[C::A_CH], rb[C::B_CH];
    uint32_t sa[C::MB], sb[C::NB];  // 4 scale bytes (blocks of this stage) per lane row
    uint32_t na[C::MB], nb[C::NB];
    auto gload = [&](int kt) {
#pragma unroll
        for (int q = 0; q < C::A_CH; ++q) ra[q] = *reinterpret_cast<const u32x4_t*>(aptr[q] + kt * BKB);
#pragma unroll
        for (int q = 0; q < C::B_CH; ++q) rb[q] = *reinterpret_cast<const u32x4_t*>(bptr[q] + kt * C::BRB);
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi) na[mi] = *reinterpret_cast<const uint32_t*>(asp[mi] + kt * 4);
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) nb[nj] = *reinterpret_cast<const uint32_t*>(bsp[nj] + kt * 4);
    };
    auto sstore = [&](int buf) {
        uint8_t* sA = lds + buf * C::STAGE;
        uint8_t* sB = sA + BM * BKB;
#pragma unroll
        for (int q = 0; q < C::A_CH; ++q) *reinterpret_cast<u32x4_t*>(sA + swz(r16 + 32 * q, c16)) = ra[q];
#pragma unroll
        for (int q = 0; q < C::B_CH; ++q) {
            if constexpr (W4) *reinterpret_cast<u32x4_t*>(sB + swz64(r4 + 64 * q, c4)) = rb[q];
            else *reinterpret_cast<u32x4_t*>(sB + swz(r16 + 32 * q, c16)) = rb[q];
        }
    };
    gload(0);
    sstore(0);
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi) sa[mi] = na[mi];
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj) sb[nj] = nb[nj];
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) gload(kt + 1);
        const uint8_t* sA = lds + (kt & 1) * C::STAGE;
        const uint8_t* sB = sA + BM * BKB;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // 16-byte chunks of block 0 and block 1 of this 64-wide step
            const int ch0 = 4 * kk + (lane >> 5), ch1 = ch0 + 2;
            const int sh = 8 * (2 * kk + (lane >> 5));
            i32x8_t af[C::MB], bfr[C::NB];
#pragma unroll
            for (int mi = 0; mi < C::MB; ++mi) {
                const int r = wm * C::WM + 32 * mi + (lane & 31);
                const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sA + swz(r, ch0));
                const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(sA + swz(r, ch1));
                af[mi] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int nj = 0; nj < C::NB; ++nj) {
                const int r = brow[nj] + (lane & 31);
                if constexpr (W4) {
                    // e2m1: 16 bytes, chunk 2kk + g of the 64-byte row (the upper half of the operand is unused)
                    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sB + swz64(r, 2 * kk + (lane >> 5)));
                    bfr[nj] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
                } else {
                    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sB + swz(r, ch0));
                    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(sB + swz(r, ch1));
                    bfr[nj] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
            }
#pragma unroll
            for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
                for (int nj = 0; nj < C::NB; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[mi], bfr[nj], acc[mi][nj], 0, W4 ? 4 : 0, 0, static_cast<int>((sa[mi] >> sh) & 0xffu), 0,
                        static_cast<int>((sb[nj] >> sh) & 0xffu));
        }
        if (kt + 1 < KT) sstore((kt + 1) & 1);
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi) sa[mi] = na[mi];
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) sb[nj] = nb[nj];
        __syncthreads();
    }
}

// ---------------- MX GEMM1 + SwiGLU + requant ----------------
// W4: w1 is packed e2m1 [E, 2H, D/2] (MXFP4 weights).
template <int BM, int BN, bool W4>
__global__ __launch_bounds__(kThreads) void mx_gemm1_kernel(MxArgs a) {
    using C = MxTile<BM, BN, W4>;
    static_assert(C::NB % 2 == 0, "gate and up need the same number of blocks");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
    __shared__ int32_t sTok[BM];
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int BH = BN / 2, h0 = blockIdx.y * BH;
    const int DB = a.D / 32;
    for (int r = tid; r < BM; r += kThreads)
        sTok[r] = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P) / a.k;
    __syncthreads();

    const int c16 = tid & 7, r16 = tid >> 3;
    const uint8_t* aptr[C::A_CH];
    const uint8_t* bptr[C::B_CH];
#pragma unroll
    for (int q = 0; q < C::A_CH; ++q) aptr[q] = a.x + static_cast<int64_t>(sTok[r16 + 32 * q]) * a.D + c16 * 16;
    const int64_t w1row0 = static_cast<int64_t>(mt.expert) * 2 * a.H;
    auto w1row = [&](int r) { return w1row0 + (r < BH ? h0 + r : a.H + h0 + (r - BH)); };
    const int c4 = tid & 3, r4 = tid >> 2;
#pragma unroll
    for (int q = 0; q < C::B_CH; ++q)
        bptr[q] = W4 ? a.w1 + w1row(r4 + 64 * q) * (a.D / 2) + c4 * 16 : a.w1 + w1row(r16 + 32 * q) * a.D + c16 * 16;
    int brow[C::NB];
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj)
        brow[nj] = nj < C::NB / 2 ? wn * (BH / 2) + 32 * nj : BH + wn * (BH / 2) + 32 * (nj - C::NB / 2);
    const uint8_t* asp[C::MB];
    const uint8_t* bsp[C::NB];
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
        asp[mi] = a.xs + static_cast<int64_t>(sTok[wm * C::WM + 32 * mi + (lane & 31)]) * DB;
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj) bsp[nj] = a.w1s + w1row(brow[nj] + (lane & 31)) * DB;

    f32x16_t acc[C::MB][C::NB];
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = f32x16_t{};
    mx_mainloop<BM, BN, W4>(lds, aptr, bptr, asp, bsp, a.D / BKB, brow, acc);

    // SwiGLU in fp32 -> LDS [BM][BH + 4] floats -> requant per 32 along H.
    constexpr int OS = BN / 2 + 4;
    float* sO = reinterpret_cast<float*>(lds);
    static_assert(BM * (BN / 2 + 4) * 4 <= 2 * C::STAGE, "act staging must fit the stage buffers");
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int j = 0; j < C::NB / 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = wm * C::WM + 32 * mi + acc_row(lane, v);
                const int col = wn * (BH / 2) + 32 * j + (lane & 31);
                const float g = acc[mi][j][v], u = acc[mi][j + C::NB / 2][v];
                sO[m * OS + col] = g / (1.0f + __expf(-g)) * u;
            }
    __syncthreads();
    const int HB = a.H / 32;
    constexpr int BPR = BN / 2 / 32;  // scale blocks per tile row
    const int sub = tid & 7;
    for (int item = tid >> 3; item < BM * BPR; item += kThreads / 8) {
        const int r = item / BPR, blk = item % BPR;
        const float4 v = *reinterpret_cast<const float4*>(sO + r * OS + blk * 32 + sub * 4);
        float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
        const int s = mx_scale_exp(amax);
        const float inv = pow2f(-s);
        const uint32_t c = e4m3_encode(v.x * inv, v.x) | (e4m3_encode(v.y * inv, v.y) << 8) |
                           (e4m3_encode(v.z * inv, v.z) << 16) | (e4m3_encode(v.w * inv, v.w) << 24);
        if (r < mt.rows) {
            const int64_t row = mt.row0 + r;
            *reinterpret_cast<uint32_t*>(a.act + row * a.H + h0 + blk * 32 + sub * 4) = c;
            if (sub == 0) a.act_s[row * HB + h0 / 32 + blk] = static_cast<uint8_t>(s + 127);
        }
    }
}

// ---------------- MX GEMM2 + routing weight ----------------
// W4: w2 is packed e2m1 [E, D, H/2] (MXFP4 weights).
template <int BM, int BN, bool W4>
__global__ __launch_bounds__(kThreads) void mx_gemm2_kernel(MxArgs a) {
    using C = MxTile<BM, BN, W4>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
    __shared__ int32_t sPair[BM];
    __shared__ float sW[BM];
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.y * BN;
    const int HB = a.H / 32;
    for (int r = tid; r < BM; r += kThreads) {
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P);
        sPair[r] = p;
        sW[r] = a.wts[p];
    }
    __syncthreads();
    const int c16 = tid & 7, r16 = tid >> 3;
    auto arow = [&](int r) { return static_cast<int64_t>(mt.row0 + (r < mt.rows ? r : 0)); };
    const uint8_t* aptr[C::A_CH];
    const uint8_t* bptr[C::B_CH];
#pragma unroll
    for (int q = 0; q < C::A_CH; ++q) aptr[q] = a.act + arow(r16 + 32 * q) * a.H + c16 * 16;
    const int64_t w2row0 = static_cast<int64_t>(mt.expert) * a.D + n0;
    const int c4 = tid & 3, r4 = tid >> 2;
#pragma unroll
    for (int q = 0; q < C::B_CH; ++q)
        bptr[q] = W4 ? a.w2 + (w2row0 + r4 + 64 * q) * (a.H / 2) + c4 * 16 : a.w2 + (w2row0 + r16 + 32 * q) * a.H + c16 * 16;
    int brow[C::NB];
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj) brow[nj] = wn * C::WN + 32 * nj;
    const uint8_t* asp[C::MB];
    const uint8_t* bsp[C::NB];
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi) asp[mi] = a.act_s + arow(wm * C::WM + 32 * mi + (lane & 31)) * HB;
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj) bsp[nj] = a.w2s + (w2row0 + brow[nj] + (lane & 31)) * HB;

    f32x16_t acc[C::MB][C::NB];
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = f32x16_t{};
    mx_mainloop<BM, BN, W4>(lds, aptr, bptr, asp, bsp, a.H / BKB, brow, acc);

    constexpr int OS = BN + 8;
    uint16_t* sO = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = wm * C::WM + 32 * mi + acc_row(lane, v);
                const int col = wn * C::WN + 32 * nj + (lane & 31);
                sO[m * OS + col] = f32_to_bf16(acc[mi][nj][v] * sW[m]);
            }
    __syncthreads();
    constexpr int CPR = BN / 8;
    for (int idx = tid; idx < BM * CPR; idx += kThreads) {
        const int r = idx / CPR, c = idx % CPR;
        if (r < mt.rows)
            *reinterpret_cast<u32x4_t*>(a.ypair + static_cast<int64_t>(sPair[r]) * a.D + n0 + c * 8) =
                *reinterpret_cast<const u32x4_t*>(sO + r * OS + c * 8);
    }
}

// ---------------- fused MX: GEMM1 -> SwiGLU -> requant in LDS -> split-K GEMM2 ----------------
// One workgroup per (m-tile of BM rows, 64-wide H slice): the GEMM1 tile
// (64 gate + 64 up rows), SwiGLU in fp32, the act requantized per 32 along H
// by MXQ into LDS (two scale blocks per row: exactly one K step of the
// scaled MFMA), then the down projection over that slice for 128 output
// features at a time, w * partial added into acc32 with fp32 atomics
// ("Prime Flash MoE", section 7: the fused MX path quantizes act in the
// epilogue and runs the down projection split over H).
constexpr int kFusedSlice = 64;        // act columns per workgroup (one scaled-MFMA K step)
constexpr int kFusedRowBytes = 64;     // act / W2 slice row in LDS: 64 codes, four 16-byte chunks (swz64)

// 32 codes of one row for the scaled MFMA: chunks g and g + 2 of the row
// (k = 16g..16g+15 and 32+16g..32+16g+15), g = lane >> 5.
__device__ __forceinline__ i32x8_t frag64(const uint8_t* base, int row, int g) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + swz64(row, g));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + swz64(row, g + 2));
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int BM>
__global__ __launch_bounds__(kThreads) void mx_fused_kernel(MxArgs a) {
    constexpr int BN = 2 * kFusedSlice;
    using C = MxTile<BM, BN>;
    constexpr int OS = kFusedSlice + 4;  // fp32 act staging row
    static_assert(BM * OS * 4 <= 2 * C::STAGE, "act staging must fit the stage buffers");
    static_assert(2 * 128 * kFusedRowBytes <= 2 * C::STAGE, "W2 slices must fit the stage buffers");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t sAct[BM * kFusedRowBytes];
    __shared__ uint8_t sActS[BM][2];
    __shared__ uint8_t sW2S[2][128][2];
    __shared__ int32_t sTok[BM];
    __shared__ float sW[BM];
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5;
    const int h0 = blockIdx.y * kFusedSlice;
    const int DB = a.D / 32, HB = a.H / 32;
    for (int r = tid; r < BM; r += kThreads) {
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P);
        sTok[r] = p / a.k;
        sW[r] = r < mt.rows ? a.wts[p] : 0.0f;
    }
    __syncthreads();

    // GEMM1 tile: gate rows h0.. and up rows H + h0.. of W1[e]
    const int c16 = tid & 7, r16 = tid >> 3;
    {
        constexpr int BH = kFusedSlice;
        const uint8_t* aptr[C::A_CH];
        const uint8_t* bptr[C::B_CH];
#pragma unroll
        for (int q = 0; q < C::A_CH; ++q) aptr[q] = a.x + static_cast<int64_t>(sTok[r16 + 32 * q]) * a.D + c16 * 16;
        const int64_t w1row0 = static_cast<int64_t>(mt.expert) * 2 * a.H;
        auto w1row = [&](int r) { return w1row0 + (r < BH ? h0 + r : a.H + h0 + (r - BH)); };
#pragma unroll
        for (int q = 0; q < C::B_CH; ++q) bptr[q] = a.w1 + w1row(r16 + 32 * q) * a.D + c16 * 16;
        int brow[C::NB];
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj)
            brow[nj] = nj < C::NB / 2 ? wn * (BH / 2) + 32 * nj : BH + wn * (BH / 2) + 32 * (nj - C::NB / 2);
        const uint8_t* asp[C::MB];
        const uint8_t* bsp[C::NB];
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi)
            asp[mi] = a.xs + static_cast<int64_t>(sTok[wm * C::WM + 32 * mi + (lane & 31)]) * DB;
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) bsp[nj] = a.w1s + w1row(brow[nj] + (lane & 31)) * DB;
        f32x16_t acc[C::MB][C::NB];
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
            for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = f32x16_t{};
        mx_mainloop<BM, BN, false>(lds, aptr, bptr, asp, bsp, a.D / BKB, brow, acc);

        // SwiGLU in fp32 into the (now idle) stage buffers
        float* sO = reinterpret_cast<float*>(lds);
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
            for (int j = 0; j < C::NB / 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = wm * C::WM + 32 * mi + acc_row(lane, v);
                    const int col = wn * (BH / 2) + 32 * j + (lane & 31);
                    const float gt = acc[mi][j][v], up = acc[mi][j + C::NB / 2][v];
                    sO[m * OS + col] = gt / (1.0f + __expf(-gt)) * up;
                }
    }
    __syncthreads();
    // MXQ per 32 act columns: 8 lanes per block, 4 values each -> codes and
    // scale bytes in LDS (the down projection's A operand)
    {
        const float* sO = reinterpret_cast<const float*>(lds);
        const int sub = tid & 7;
        for (int item = tid >> 3; item < BM * 2; item += kThreads / 8) {
            const int r = item >> 1, blk = item & 1;
            const float4 v = *reinterpret_cast<const float4*>(sO + r * OS + blk * 32 + sub * 4);
            float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
            amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
            const int sc = mx_scale_exp(amax);
            const float inv = pow2f(-sc);
            const uint32_t c = e4m3_encode(v.x * inv, v.x) | (e4m3_encode(v.y * inv, v.y) << 8) |
                               (e4m3_encode(v.z * inv, v.z) << 16) | (e4m3_encode(v.w * inv, v.w) << 24);
            // byte 32*blk + 4*sub of the row: chunk 2*blk + sub/4, offset 4*(sub&3)
            *reinterpret_cast<uint32_t*>(sAct + swz64(r, 2 * blk + (sub >> 2)) + 4 * (sub & 3)) = c;
            if (sub == 0) sActS[r][blk] = static_cast<uint8_t>(sc + 127);
        }
    }
    __syncthreads();

    // Down projection over this slice, 128 output features per step; W2
    // slices (128 rows x 64 codes + 2 scale bytes per row) double-buffered
    // in the stage buffers through registers.
    const uint8_t* w2e = a.w2 + static_cast<int64_t>(mt.expert) * a.D * a.H + h0;
    const uint8_t* w2se = a.w2s + static_cast<int64_t>(mt.expert) * a.D * HB + h0 / 32;
    const int NT = a.D / 128;
    const int wr = tid >> 2, wc = tid & 3;  // W2 load: rows wr, wr + 64; chunk wc
    u32x4_t rb[2];
    uint16_t rs = 0;
    auto gload = [&](int nt) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            rb[q] = *reinterpret_cast<const u32x4_t*>(w2e + static_cast<int64_t>(nt * 128 + wr + 64 * q) * a.H + wc * 16);
        if (tid < 128) rs = *reinterpret_cast<const uint16_t*>(w2se + static_cast<int64_t>(nt * 128 + tid) * HB);
    };
    auto sstore = [&](int buf) {
        uint8_t* sB = lds + buf * 128 * kFusedRowBytes;
#pragma unroll
        for (int q = 0; q < 2; ++q) *reinterpret_cast<u32x4_t*>(sB + swz64(wr + 64 * q, wc)) = rb[q];
        if (tid < 128) {
            sW2S[buf][tid][0] = static_cast<uint8_t>(rs & 0xffu);
            sW2S[buf][tid][1] = static_cast<uint8_t>(rs >> 8);
        }
    };
    // this wave's act fragments and scales, fixed for every step
    constexpr int MB2 = BM / 2 / 32;
    i32x8_t af[MB2];
    int as[MB2];
#pragma unroll
    for (int mi = 0; mi < MB2; ++mi) {
        const int r = wm * (BM / 2) + 32 * mi + (lane & 31);
        af[mi] = frag64(sAct, r, g);
        as[mi] = sActS[r][g];
    }
    gload(0);
    sstore(0);
    __syncthreads();
    for (int nt = 0; nt < NT; ++nt) {
        if (nt + 1 < NT) gload(nt + 1);
        const uint8_t* sB = lds + (nt & 1) * 128 * kFusedRowBytes;
        f32x16_t acc2[MB2][2];
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            const int col = wn * 64 + 32 * nj + (lane & 31);
            const i32x8_t bf = frag64(sB, col, g);
            const int bs = sW2S[nt & 1][col][g];
#pragma unroll
            for (int mi = 0; mi < MB2; ++mi)
                acc2[mi][nj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bf, f32x16_t{}, 0, 0, 0, as[mi],
                                                                              0, bs);
        }
#pragma unroll
        for (int mi = 0; mi < MB2; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = wm * (BM / 2) + 32 * mi + acc_row(lane, v);
                if (m < mt.rows) {
                    float* dst = a.acc32 + static_cast<int64_t>(sTok[m]) * a.D + nt * 128 + wn * 64 + (lane & 31);
#pragma unroll
                    for (int nj = 0; nj < 2; ++nj) unsafeAtomicAdd(dst + 32 * nj, sW[m] * acc2[mi][nj][v]);
                }
            }
        if (nt + 1 < NT) sstore((nt + 1) & 1);
        __syncthreads();
    }
}

inline int mtiles_upper(int64_t P, int E, int bm) { return static_cast<int>((P + bm - 1) / bm + E); }

}  // namespace

// The route step has cleared acc32 and the token counters. The ring kernel
// converts each token's row itself; the generic one leaves the conversion to
// a kernel of its own.
hipError_t launch_fused_mx(const MxArgs& a, hipStream_t s, hipEvent_t* ev) {
    constexpr int BM = 128;
    const int64_t n = static_cast<int64_t>(a.T) * a.D;
    record(ev, 0, s);
    if (mx_fused_dma_supported(a)) {
        const hipError_t e = launch_mx_fused_dma(a, s);
        record(ev, 1, s);
        record(ev, 2, s);
        return e;
    }
    dim3 g(mtiles_upper(a.P, a.E, BM), a.H / kFusedSlice);
    mx_fused_kernel<BM><<<g, kThreads, 0, s>>>(a);
    record(ev, 1, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_f32_to_bf16(a.acc32, a.out, n, s);
    record(ev, 2, s);
    return e;
}

hipError_t launch_mx_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
    const int64_t nblk = rows * (K / 32);
    if (nblk == 0) return hipSuccess;
    int64_t g = (nblk * 8 + 255) / 256;
    if (g > 8192) g = 8192;
    mx_quantize_kernel<<<static_cast<int>(g), 256, 0, s>>>(src, nblk, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx4_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t s) {
    const int64_t nblk = rows * (K / 32);
    if (nblk == 0) return hipSuccess;
    int64_t g = (nblk * 8 + 255) / 256;
    if (g > 8192) g = 8192;
    mx4_quantize_kernel<<<static_cast<int>(g), 256, 0, s>>>(src, nblk, codes, scales);
    return hipGetLastError();
}

hipError_t launch_split_mx(const MxArgs& a, hipStream_t s, hipEvent_t* ev) {
    constexpr int BM = 128, BN1 = 128, BN2 = 128;
    const bool big = big_mx_supported(a);
    const dim3 g1(mtiles_upper(a.P, a.E, BM), a.H / (BN1 / 2));
    const dim3 g2(mtiles_upper(a.P, a.E, BM), a.D / BN2);
    const bool skinny = !big && skinny_mx_supported(a);
    if (big) launch_big_mx(a, true, s);
    else if (skinny) launch_skinny_mx(a, true, s);
    else if (a.w4) mx_gemm1_kernel<BM, BN1, true><<<g1, kThreads, 0, s>>>(a);
    else mx_gemm1_kernel<BM, BN1, false><<<g1, kThreads, 0, s>>>(a);
    record(ev, 0, s);
    if (big) launch_big_mx(a, false, s);
    else if (skinny) launch_skinny_mx(a, false, s);
    else if (a.w4) mx_gemm2_kernel<BM, BN2, true><<<g2, kThreads, 0, s>>>(a);
    else mx_gemm2_kernel<BM, BN2, false><<<g2, kThreads, 0, s>>>(a);
    record(ev, 1, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_combine(a.ypair, a.rv.pair_to_sorted, a.T, a.k, a.D, a.out, s);
    record(ev, 2, s);
    return e;
}

}  // namespace moe
