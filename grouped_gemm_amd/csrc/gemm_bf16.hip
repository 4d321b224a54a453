// bf16 grouped GEMMs of the MoE SwiGLU FFN on gfx950 MFMA.
//
// GEMM1 ("Prime Flash MoE", section 1 and section 2 "Trick 1"): for the
// sorted rows of one expert, gate|up = x W1[e]^T. A workgroup's N-tile pairs
// gate rows [h0, h0+BH) with up rows [H+h0, H+h0+BH) of W1, so each wave
// holds a gate block and its up partner in identically laid out
// accumulators and the SwiGLU epilogue is elementwise in registers; W1 is
// read in its natural [E, 2H, D] layout, the pairing is only address math.
// The token rows are gathered on load (row r of the tile reads token
// sorted_to_pair[row0 + r] / k), so the sorted copy of x is never written.
//
// GEMM2 (section 1, and section 6 for the split pipeline): y = act W2[e]^T
// over the whole H, times the pair's routing weight in fp32, written as
// bf16 rows in pair order; the combine kernel then sums each token's k rows
// in fp32 and writes out once (a segmented combine: no atomics, no zeroing,
// deterministic).
//
// Fused (section 2 "Trick 2"): one workgroup per (m-tile, H slice) runs the
// GEMM1 tile, keeps the SwiGLU output in LDS as the A operand of a split-K
// down projection over its slice, and adds weight * partial into an fp32
// accumulator with float atomics; a last kernel converts it to bf16.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid, each wave a (BM/2)x(BN/2)
// block of 32x32x16 bf16 MFMAs. K steps of 64 bf16 (128 bytes per row) are
// double-buffered in LDS with 16-byte chunks XOR-swizzled by ((row >> 1) & 7):
// gfx950's LDS serves 16 lanes of a 16-byte read per cycle from 64 banks, so
// the 16 rows read together must land in 16 distinct 16-byte bank groups
// (two 128-byte rows span 256 bytes = one pass over the banks).
#include "common.h"

namespace moe {

namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Row of the 32x32 MFMA output held by item v of lane `lane`; the column is lane & 31.
__device__ __forceinline__ int acc_row(int lane, int v) { return ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3); }

template <int BM, int BN>
struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int MB = WM / 32, NB = WN / 32;
    static constexpr int A_CH = BM * 8 / kThreads;  // 16-byte chunks per thread per K step
    static constexpr int B_CH = BN * 8 / kThreads;
    static constexpr int STAGE = (BM + BN) * BK;    // bf16 elements per LDS stage
    static_assert(MB >= 1 && NB >= 1 && A_CH >= 1 && B_CH >= 1, "tile too small");
};

// Main loop shared by GEMM1 and GEMM2: acc[mi][nj] += A[rows] . B[rows]^T over K.
// aptr/bptr point at this thread's 16-byte chunk of K step 0 for each of its rows.
template <int BM, int BN>
__device__ __forceinline__ void mainloop(uint16_t* lds, const uint16_t* const* aptr,
                                         const uint16_t* const* bptr, int KT, const int* brow,
                                         f32x16_t (&acc)[Tile<BM, BN>::MB][Tile<BM, BN>::NB]) {
    using C = Tile<BM, BN>;
    const int tid = threadIdx.x, lane = tid & 63, wm = (tid >> 6) >> 1;
    const int c16 = tid & 7, r16 = tid >> 3;
    u32x4_t ra[C::A_CH], rb[C::B_CH];
    auto gload = [&](int kt) {
#pragma unroll
        for (int q = 0; q < C::A_CH; ++q) ra[q] = *reinterpret_cast<const u32x4_t*>(aptr[q] + kt * BK);
#pragma unroll
        for (int q = 0; q < C::B_CH; ++q) rb[q] = *reinterpret_cast<const u32x4_t*>(bptr[q] + kt * BK);
    };
    auto sstore = [&](int buf) {
        uint16_t* sA = lds + buf * C::STAGE;
        uint16_t* sB = sA + BM * BK;
#pragma unroll
        for (int q = 0; q < C::A_CH; ++q) *reinterpret_cast<u32x4_t*>(sA + swz(r16 + 32 * q, c16)) = ra[q];
#pragma unroll
        for (int q = 0; q < C::B_CH; ++q) *reinterpret_cast<u32x4_t*>(sB + swz(r16 + 32 * q, c16)) = rb[q];
    };
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) gload(kt + 1);
        const uint16_t* sA = lds + (kt & 1) * C::STAGE;
        const uint16_t* sB = sA + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = 2 * kk + (lane >> 5);
            bf16x8_t af[C::MB], bfr[C::NB];
#pragma unroll
            for (int mi = 0; mi < C::MB; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8_t*>(sA + swz(wm * C::WM + 32 * mi + (lane & 31), chunk));
#pragma unroll
            for (int nj = 0; nj < C::NB; ++nj)
                bfr[nj] = *reinterpret_cast<const bf16x8_t*>(sB + swz(brow[nj] + (lane & 31), chunk));
#pragma unroll
            for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
                for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = mfma32(af[mi], bfr[nj], acc[mi][nj]);
        }
        if (kt + 1 < KT) sstore((kt + 1) & 1);
        __syncthreads();
    }
}

// ---------------- GEMM1 + SwiGLU (split pipeline) ----------------
// grid: (m-tile upper bound, H / (BN/2)); writes act [P, H] bf16.
template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm1_swiglu_kernel(Bf16Args a) {
    using C = Tile<BM, BN>;
    static_assert(C::NB % 2 == 0, "gate and up need the same number of blocks");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];
    __shared__ int32_t sTok[BM];
    __shared__ float sScale[BM];  // activation variant: alpha[e] * (wba ? w : 1) per row
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int BH = BN / 2, h0 = blockIdx.y * BH;
    const bool variant = a.av.on();
    for (int r = tid; r < BM; r += kThreads) {
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P);
        sTok[r] = p / a.k;
        if (variant) {
            const float al = a.av.alpha ? a.av.alpha[mt.expert] : 1.0f;
            sScale[r] = a.av.wba ? al * a.wts[p] : al;
        }
    }
    __syncthreads();

    const int c16 = tid & 7, r16 = tid >> 3;
    const uint16_t* aptr[C::A_CH];
    const uint16_t* bptr[C::B_CH];
#pragma unroll
    for (int q = 0; q < C::A_CH; ++q)
        aptr[q] = a.x + static_cast<int64_t>(sTok[r16 + 32 * q]) * a.D + c16 * 8;
    const uint16_t* w1e = a.w1 + static_cast<int64_t>(mt.expert) * 2 * a.H * a.D;
#pragma unroll
    for (int q = 0; q < C::B_CH; ++q) {
        const int r = r16 + 32 * q;
        const int grow = r < BH ? h0 + r : a.H + h0 + (r - BH);
        bptr[q] = w1e + static_cast<int64_t>(grow) * a.D + c16 * 8;
    }
    int brow[C::NB];
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj)
        brow[nj] = nj < C::NB / 2 ? wn * (BH / 2) + 32 * nj : BH + wn * (BH / 2) + 32 * (nj - C::NB / 2);

    f32x16_t acc[C::MB][C::NB];
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = f32x16_t{};
    mainloop<BM, BN>(lds, aptr, bptr, a.D / BK, brow, acc);

    // SwiGLU in registers, staged through LDS as bf16, stored as 16-byte row chunks.
    constexpr int OS = BN / 2 + 8;
    uint16_t* sO = lds;
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int j = 0; j < C::NB / 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = wm * C::WM + 32 * mi + acc_row(lane, v);
                const int col = wn * (BH / 2) + 32 * j + (lane & 31);
                const float g = acc[mi][j][v], u = acc[mi][j + C::NB / 2][v];
                sO[m * OS + col] =
                    f32_to_bf16(variant ? act_variant(g, u, sScale[m], a.av.kind, a.av.limit) : silu_mul(g, u));
            }
    __syncthreads();
    constexpr int CPR = BH / 8;
    for (int idx = tid; idx < BM * CPR; idx += kThreads) {
        const int r = idx / CPR, c = idx % CPR;
        if (r < mt.rows)
            *reinterpret_cast<u32x4_t*>(a.act + static_cast<int64_t>(mt.row0 + r) * a.H + h0 + c * 8) =
                *reinterpret_cast<const u32x4_t*>(sO + r * OS + c * 8);
    }
}

// ---------------- GEMM2 + routing weight (split pipeline) ----------------
// grid: (m-tile upper bound, D / BN); writes ypair [P, D] bf16 at row = pair.
template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm2_weight_kernel(Bf16Args a) {
    using C = Tile<BM, BN>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];
    __shared__ int32_t sPair[BM];
    __shared__ float sW[BM];
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.y * BN;
    for (int r = tid; r < BM; r += kThreads) {
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P);
        sPair[r] = p;
        sW[r] = a.av.wba ? 1.0f : a.wts[p];  // with the weight applied before the activation, y is not scaled
    }
    __syncthreads();

    const int c16 = tid & 7, r16 = tid >> 3;
    const uint16_t* aptr[C::A_CH];
    const uint16_t* bptr[C::B_CH];
#pragma unroll
    for (int q = 0; q < C::A_CH; ++q) {
        const int r = r16 + 32 * q;
        aptr[q] = a.act + static_cast<int64_t>(mt.row0 + (r < mt.rows ? r : 0)) * a.H + c16 * 8;
    }
    const uint16_t* w2e = a.w2 + static_cast<int64_t>(mt.expert) * a.D * a.H;
#pragma unroll
    for (int q = 0; q < C::B_CH; ++q) bptr[q] = w2e + static_cast<int64_t>(n0 + r16 + 32 * q) * a.H + c16 * 8;
    int brow[C::NB];
#pragma unroll
    for (int nj = 0; nj < C::NB; ++nj) brow[nj] = wn * C::WN + 32 * nj;

    f32x16_t acc[C::MB][C::NB];
#pragma unroll
    for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = f32x16_t{};
    mainloop<BM, BN>(lds, aptr, bptr, a.H / BK, brow, acc);

    constexpr int OS = BN + 8;
    uint16_t* sO = lds;
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

// ---------------- fused GEMM1 -> SwiGLU -> split-K GEMM2 ----------------
// grid: (m-tile upper bound, H / BH). BM = 128, BH = 64 (GEMM1 N-tile 128),
// down-projection N-chunks of 128 over D with K = BH.
template <int BM, int BH, int BN2>
__global__ __launch_bounds__(kThreads) void fused_bf16_kernel(Bf16Args a) {
    constexpr int BN = 2 * BH;
    using C = Tile<BM, BN>;
    using C2 = Tile<BM, BN2>;
    static_assert(2 * BN2 * BK <= 2 * C::STAGE, "W2 chunks must fit the stage buffers");
    static_assert(BH == BK, "the act slice is exactly one K step of the down projection");
    // one LDS array: two GEMM stages, then the act tile (A operand of the
    // down projection)
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE + BM * BK];
    __shared__ int32_t sTok[BM];
    __shared__ float sW[BM];
    uint16_t* sAct = lds + 2 * C::STAGE;
    MTile mt;
    if (!find_mtile<BM>(a.rv, a.E, blockIdx.x, mt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int h0 = blockIdx.y * BH;
    for (int r = tid; r < BM; r += kThreads) {
        const int p = clamp_pair(a.rv.sorted_to_pair[mt.row0 + (r < mt.rows ? r : 0)], a.P);
        sTok[r] = p / a.k;
        sW[r] = r < mt.rows ? a.wts[p] : 0.0f;
    }
    __syncthreads();

    const int c16 = tid & 7, r16 = tid >> 3;
    {
        const uint16_t* aptr[C::A_CH];
        const uint16_t* bptr[C::B_CH];
#pragma unroll
        for (int q = 0; q < C::A_CH; ++q)
            aptr[q] = a.x + static_cast<int64_t>(sTok[r16 + 32 * q]) * a.D + c16 * 8;
        const uint16_t* w1e = a.w1 + static_cast<int64_t>(mt.expert) * 2 * a.H * a.D;
#pragma unroll
        for (int q = 0; q < C::B_CH; ++q) {
            const int r = r16 + 32 * q;
            const int grow = r < BH ? h0 + r : a.H + h0 + (r - BH);
            bptr[q] = w1e + static_cast<int64_t>(grow) * a.D + c16 * 8;
        }
        int brow[C::NB];
#pragma unroll
        for (int nj = 0; nj < C::NB; ++nj)
            brow[nj] = nj < C::NB / 2 ? wn * (BH / 2) + 32 * nj : BH + wn * (BH / 2) + 32 * (nj - C::NB / 2);
        f32x16_t acc[C::MB][C::NB];
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
            for (int nj = 0; nj < C::NB; ++nj) acc[mi][nj] = f32x16_t{};
        mainloop<BM, BN>(lds, aptr, bptr, a.D / BK, brow, acc);
        // act tile -> LDS in the swizzled operand layout (row m, k = act column)
#pragma unroll
        for (int mi = 0; mi < C::MB; ++mi)
#pragma unroll
            for (int j = 0; j < C::NB / 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = wm * C::WM + 32 * mi + acc_row(lane, v);
                    const int col = wn * (BH / 2) + 32 * j + (lane & 31);
                    sAct[swz(m, col >> 3) + (col & 7)] =
                        f32_to_bf16(silu_mul(acc[mi][j][v], acc[mi][j + C::NB / 2][v]));
                }
    }
    // Down projection over this H slice, BN2 output columns at a time.
    const uint16_t* w2e = a.w2 + static_cast<int64_t>(mt.expert) * a.D * a.H + h0 + c16 * 8;
    const int NT = a.D / BN2;
    u32x4_t rb[C2::B_CH];
    auto gload = [&](int nt) {
#pragma unroll
        for (int q = 0; q < C2::B_CH; ++q)
            rb[q] = *reinterpret_cast<const u32x4_t*>(w2e + static_cast<int64_t>(nt * BN2 + r16 + 32 * q) * a.H);
    };
    auto sstore = [&](int buf) {
        uint16_t* sB = lds + buf * BN2 * BK;
#pragma unroll
        for (int q = 0; q < C2::B_CH; ++q) *reinterpret_cast<u32x4_t*>(sB + swz(r16 + 32 * q, c16)) = rb[q];
    };
    gload(0);
    sstore(0);
    __syncthreads();
    for (int nt = 0; nt < NT; ++nt) {
        if (nt + 1 < NT) gload(nt + 1);
        const uint16_t* sB = lds + (nt & 1) * BN2 * BK;
        f32x16_t acc2[C2::MB][C2::NB];
#pragma unroll
        for (int mi = 0; mi < C2::MB; ++mi)
#pragma unroll
            for (int nj = 0; nj < C2::NB; ++nj) acc2[mi][nj] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = 2 * kk + (lane >> 5);
            bf16x8_t af[C2::MB], bfr[C2::NB];
#pragma unroll
            for (int mi = 0; mi < C2::MB; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8_t*>(sAct + swz(wm * C2::WM + 32 * mi + (lane & 31), chunk));
#pragma unroll
            for (int nj = 0; nj < C2::NB; ++nj)
                bfr[nj] = *reinterpret_cast<const bf16x8_t*>(sB + swz(wn * C2::WN + 32 * nj + (lane & 31), chunk));
#pragma unroll
            for (int mi = 0; mi < C2::MB; ++mi)
#pragma unroll
                for (int nj = 0; nj < C2::NB; ++nj) acc2[mi][nj] = mfma32(af[mi], bfr[nj], acc2[mi][nj]);
        }
#pragma unroll
        for (int mi = 0; mi < C2::MB; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = wm * C2::WM + 32 * mi + acc_row(lane, v);
                if (m < mt.rows) {
                    float* dst = a.acc32 + static_cast<int64_t>(sTok[m]) * a.D + nt * BN2 + wn * C2::WN + (lane & 31);
#pragma unroll
                    for (int nj = 0; nj < C2::NB; ++nj) unsafeAtomicAdd(dst + 32 * nj, sW[m] * acc2[mi][nj][v]);
                }
            }
        if (nt + 1 < NT) sstore((nt + 1) & 1);
        __syncthreads();
    }
}

// ---------------- combine / conversions ----------------

// out[t, :] = bf16( sum over valid slots j of ypair[t*k + j, :] [+ shared_y[t, :]] ),
// 8 columns per thread; the shared expert's row (if any) joins the fp32 sum
// last. Every ypair byte is read once and every out byte written once: both
// go through nontemporal accesses (streamed past the caches), launched with
// one item per thread for all but huge T.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ ypair,
                                                      const int32_t* __restrict__ p2s, int32_t T,
                                                      int32_t k, int32_t D, const uint16_t* __restrict__ shared_y,
                                                      uint16_t* __restrict__ out) {
    const int cpr = D / 8;
    const int64_t n = static_cast<int64_t>(T) * cpr;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t t = i / cpr;
        const int c = static_cast<int>(i - t * cpr);
        float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        // slots in groups of 8 with all loads of a group issued before use
        for (int j0 = 0; j0 < k; j0 += 8) {
            u32x4_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t p = t * k + j0 + j;
                const bool ok = j0 + j < k && p2s[p] >= 0;
                v[j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ypair + p * D + c * 8))
                          : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    s[2 * q] += bf16_to_f32(static_cast<uint16_t>(v[j][q] & 0xffffu));
                    s[2 * q + 1] += bf16_to_f32(static_cast<uint16_t>(v[j][q] >> 16));
                }
        }
        if (shared_y) {
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(shared_y + t * D + c * 8));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s[2 * q] += bf16_to_f32(static_cast<uint16_t>(v[q] & 0xffffu));
                s[2 * q + 1] += bf16_to_f32(static_cast<uint16_t>(v[q] >> 16));
            }
        }
        u32x4_t o;
        o.x = pack_bf16x2(s[0], s[1]);
        o.y = pack_bf16x2(s[2], s[3]);
        o.z = pack_bf16x2(s[4], s[5]);
        o.w = pack_bf16x2(s[6], s[7]);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + t * D + c * 8));
    }
}

// dst = bf16(src [+ extra]), 4 values per thread; extra (nullable) is bf16.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4* src, const uint2* extra, uint2* dst,
                                                          int64_t n4) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256) {
        float4 v = src[i];
        if (extra) {
            const uint2 e = extra[i];
            v.x += bf16_to_f32(static_cast<uint16_t>(e.x & 0xffffu));
            v.y += bf16_to_f32(static_cast<uint16_t>(e.x >> 16));
            v.z += bf16_to_f32(static_cast<uint16_t>(e.y & 0xffffu));
            v.w += bf16_to_f32(static_cast<uint16_t>(e.y >> 16));
        }
        dst[i] = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    }
}

// Route maps of the identity routing (T tokens, one slot each, expert 0).
__global__ __launch_bounds__(256) void identity_route_kernel(int64_t T, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tile_prefix,
                                                             int32_t* __restrict__ s2p, int32_t* __restrict__ p2s,
                                                             float* __restrict__ ones) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < T; i += static_cast<int64_t>(gridDim.x) * 256) {
        s2p[i] = static_cast<int32_t>(i);
        p2s[i] = static_cast<int32_t>(i);
        ones[i] = 1.0f;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        counts[0] = static_cast<int32_t>(T);
        offsets[0] = 0;
        offsets[1] = static_cast<int32_t>(T);
        for (int b = 0; b < kNumTileHeights; ++b) {  // [kNumTileHeights][E + 1] with E = 1
            const int64_t bm = 16 << b;
            tile_prefix[b * 2] = 0;
            tile_prefix[b * 2 + 1] = static_cast<int32_t>((T + bm - 1) / bm);
        }
    }
}

inline int grid_for(int64_t work, int per_block, int64_t cap = 256 * 32) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > cap) g = cap;
    return static_cast<int>(g < 1 ? 1 : g);
}
constexpr int64_t kCombineMaxBlocks = int64_t(1) << 20;

inline int mtiles_upper(int64_t P, int E, int bm) {
    return static_cast<int>((P + bm - 1) / bm + E);
}

}  // namespace

// The skinny kernels stream the weights once per 32-row m-tile. A single
// group (one expert: a shared expert, a dense FFN) with few rows would give
// the prefill ring fewer tiles than half the CUs, so it streams too.
bool bf16_uses_decode_kernels(const Bf16Args& a) {
    if (a.D % 128 || a.H % 128) return false;  // their K stages are 128 or 256 values
    const int64_t ring_tiles = (a.P / 128 + a.E) * (a.H / 128);
    return decode_kernels_fit(a.T, a.k, a.E) || (a.E == 1 && ring_tiles < device_cu_count() / 2);
}

hipError_t launch_gemms_bf16(const Bf16Args& a, hipStream_t s, hipEvent_t* ev) {
    constexpr int BM = 128, BN1 = 128, BN2 = 128;
    const bool skinny = bf16_uses_decode_kernels(a);
    const bool big = !skinny && big_gemm_supported(a);
    if (skinny) {
        launch_skinny_gemm1(a, s);
    } else if (big) {
        launch_big_gemm(a, true, s);
    } else {
        dim3 g1(mtiles_upper(a.P, a.E, BM), a.H / (BN1 / 2));
        gemm1_swiglu_kernel<BM, BN1><<<g1, kThreads, 0, s>>>(a);
    }
    record(ev, 0, s);
    if (skinny) {
        launch_skinny_gemm2(a, s);
    } else if (big) {
        launch_big_gemm(a, false, s);
    } else if (a.D % BN2 == 0) {
        dim3 g2(mtiles_upper(a.P, a.E, BM), a.D / BN2);
        gemm2_weight_kernel<BM, BN2><<<g2, kThreads, 0, s>>>(a);
    } else {  // D a multiple of 64 only
        dim3 g2(mtiles_upper(a.P, a.E, BM), a.D / 64);
        gemm2_weight_kernel<BM, 64><<<g2, kThreads, 0, s>>>(a);
    }
    record(ev, 1, s);
    return hipGetLastError();
}

hipError_t launch_split_bf16(const Bf16Args& a, hipStream_t s, hipEvent_t* ev) {
    const hipError_t e = launch_gemms_bf16(a, s, ev);
    if (e != hipSuccess) return e;
    combine_kernel<<<grid_for(static_cast<int64_t>(a.T) * a.D / 8, 256, kCombineMaxBlocks), 256, 0, s>>>(
        a.ypair, a.rv.pair_to_sorted, a.T, a.k, a.D, a.shared_y, a.out);
    record(ev, 2, s);
    return hipGetLastError();
}

hipError_t launch_identity_route(int64_t T, int32_t* counts, int32_t* offsets, int32_t* tile_prefix,
                                 int32_t* sorted_to_pair, int32_t* pair_to_sorted, float* ones, hipStream_t s) {
    identity_route_kernel<<<grid_for(T, 256), 256, 0, s>>>(T, counts, offsets, tile_prefix, sorted_to_pair,
                                                          pair_to_sorted, ones);
    return hipGetLastError();
}

// The route step has cleared acc32 and the token counters. The decode-ring
// kernel converts each token's row itself once it is complete; the generic
// kernel leaves the conversion to a kernel of its own.
hipError_t launch_fused_bf16(const Bf16Args& a, hipStream_t s, hipEvent_t* ev) {
    constexpr int BM = 128, BH = 64;
    const int64_t n = static_cast<int64_t>(a.T) * a.D;
    record(ev, 0, s);
    if (fused_decode_supported(a)) {
        launch_fused_decode(a, s);
        record(ev, 1, s);
        record(ev, 2, s);
        return hipGetLastError();
    }
    dim3 g(mtiles_upper(a.P, a.E, BM), a.H / BH);
    if (a.D % 128 == 0) fused_bf16_kernel<BM, BH, 128><<<g, kThreads, 0, s>>>(a);
    else fused_bf16_kernel<BM, BH, 64><<<g, kThreads, 0, s>>>(a);
    record(ev, 1, s);
    f32_to_bf16_kernel<<<grid_for(n / 4, 256), 256, 0, s>>>(reinterpret_cast<const float4*>(a.acc32),
                                                             reinterpret_cast<const uint2*>(a.shared_y),
                                                             reinterpret_cast<uint2*>(a.out), n / 4);
    record(ev, 2, s);
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* ypair, const int32_t* p2s, int32_t T, int32_t k, int32_t D,
                          uint16_t* out, hipStream_t s) {
    combine_kernel<<<grid_for(static_cast<int64_t>(T) * D / 8, 256, kCombineMaxBlocks), 256, 0, s>>>(
        ypair, p2s, T, k, D, nullptr, out);
    return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
    f32_to_bf16_kernel<<<grid_for(n / 4, 256), 256, 0, s>>>(reinterpret_cast<const float4*>(src), nullptr,
                                                            reinterpret_cast<uint2*>(dst), n / 4);
    return hipGetLastError();
}

}  // namespace moe
