/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) routed MoE SwiGLU FFN forward pass.
 *
 * The operation ("Prime Flash MoE - Faster MoE Kernels optimized for
 * Blackwell", section 1 "The computation"): the pass is handed each
 * token's k experts and their normalized weights by an upstream router.
 * For every routed (token t, expert e) pair,
 *     gate|up = W1[e] x_t         (W1 [E, 2H, D], output-major, gate rows
 *                                  [0, H) then up rows [H, 2H))
 *     act     = silu(gate) * up   (silu(z) = z / (1 + exp(-z)))
 *     y       = W2[e] act         (W2 [E, D, H], output-major)
 * and out[t] = sum over the token's k slots of weight * y. The library runs
 * it as: route (per-expert histogram, prefix sum, stable index maps) ->
 * grouped GEMM1 with the SwiGLU epilogue -> grouped GEMM2 with the
 * routing-weight epilogue -> combine into out.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers (HIP device memory) unless the
 *     comment says "host". Tensors are dense and row-major (last dim
 *     contiguous). bf16 tensors hold IEEE bfloat16 bit patterns (uint16).
 *   - The caller owns every buffer. The library never allocates device
 *     memory inside these calls and keeps no state between them (the one
 *     exception is the static scratch array of moe_ffn_forward_noalloc).
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously; no call synchronizes the host except where stated.
 *   - Return value: MOE_FFN_OK (0) or a negative MOE_FFN_E* code; no
 *     exception crosses the ABI. moe_ffn_strerror() names a code.
 *   - Calls on distinct streams with distinct workspaces and outputs are
 *     independent; concurrent calls that share a workspace race.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_API __attribute__((visibility("default")))

/* Data paths (Prime Flash MoE, introduction: a bf16 path and an MXFP8 path
 * of the same structure). MOE_FFN_MXFP4 is the MXFP4-weight path of
 * "GC-MoE on SM120" (scale formats): expert weights as 4-bit E2M1 codes in
 * blocks of 32 along K, each block with one UE8M0 power-of-two scale, two
 * codes per byte with the even K index in the low nibble; x and the
 * activation stay MX-fp8 (e4m3 codes, e8m0 scales) as in MOE_FFN_MXFP8.
 * SPLIT (and AUTO) only. */
enum { MOE_FFN_BF16 = 0, MOE_FFN_MXFP8 = 1, MOE_FFN_MXFP4 = 2 };

/* Pipelines (same page, introduction and section 6): FUSED runs GEMM1,
 * SwiGLU and GEMM2 in one kernel and never writes the activation; the down
 * projection is then split over H slices whose partial rows are reduced
 * into an fp32 accumulator. SPLIT writes the activation once and runs the
 * down projection as a plain grouped GEMM. AUTO resolves to FUSED for bf16
 * passes bound by launch latency (up to 16 MB of expert weights streamed,
 * one expert's weights per 32 routed rows, with D a multiple of 256 and H of
 * 128) and for MX-fp8 passes whose fused blocks (expected 32-row m-tiles
 * times H/128) fit one round of the device's compute units (D a multiple
 * of 512, H of 128), where it measured faster on MI355X, and to SPLIT
 * otherwise. */
enum { MOE_FFN_AUTO = 0, MOE_FFN_FUSED = 1, MOE_FFN_SPLIT = 2 };

enum {
    MOE_FFN_OK = 0,
    MOE_FFN_EINVAL_SHAPE = -1,  /* T < 0, D/H/E/topk < 1, D or H not a multiple of 64
                                   (bf16) or of 128 (MXFP8, MXFP4), topk > E or > 64,
                                   E > 8192, or sizes that overflow */
    MOE_FFN_EINVAL_PTR = -2,    /* a required pointer is NULL or not 16-byte aligned */
    MOE_FFN_EUNSUPPORTED = -3,  /* dtype or mode unknown, or the pair not built */
    MOE_FFN_EWORKSPACE = -4,    /* workspace NULL, misaligned (256 B) or too small */
    MOE_FFN_EHIP = -5,          /* a HIP launch reported an error */
    MOE_FFN_ESCRATCH = -6       /* moe_ffn_forward_noalloc: the problem needs more
                                   than MOE_FFN_NOALLOC_SCRATCH_BYTES of scratch */
};

/* Problem descriptor (plain C; every pointer is caller-owned).
 *   T, D, H, E, topk : tokens, hidden dim, FFN intermediate dim, experts, k.
 *   dtype            : MOE_FFN_BF16, MOE_FFN_MXFP8 or MOE_FFN_MXFP4.
 *   x_scale, w1_scale, w2_scale : MXFP8 and MXFP4 (NULL for bf16). e8m0 bytes
 *                      (value 2^(byte-127)), one per 32 contiguous elements
 *                      along the contraction dim (Prime Flash MoE, section
 *                      7): x_scale [T, D/32], w1_scale [E, 2H, D/32],
 *                      w2_scale [E, D, H/32], row-major.
 *   workspace        : device scratch of at least moe_ffn_workspace_bytes(),
 *                      256-byte aligned. Its contents on entry are ignored. */
typedef struct moe_ffn_problem {
    int32_t T, D, H, E, topk;
    int32_t dtype;
    const void* x_scale;
    const void* w1_scale;
    const void* w2_scale;
    void* workspace;
    size_t workspace_bytes;
} moe_ffn_problem;

/* Bytes of workspace moe_ffn_forward needs for this problem and mode
 * (AUTO resolves as moe_ffn_forward would). Host only; 0 on invalid input. */
MOE_FFN_API size_t moe_ffn_workspace_bytes(const moe_ffn_problem* p, int mode);

/* Host-only check of shapes, dtype and mode (no pointers are checked, no
 * GPU call is made). Returns MOE_FFN_OK or the error moe_ffn_forward would
 * return for the same shapes. */
MOE_FFN_API int moe_ffn_validate(const moe_ffn_problem* p, int mode);

/* The pipeline AUTO resolves to for this problem (MOE_FFN_FUSED or
 * MOE_FFN_SPLIT); a negative code on invalid input. Host only. */
MOE_FFN_API int moe_ffn_resolve_mode(const moe_ffn_problem* p, int mode);

/* The kernel family moe_ffn_forward runs for GEMM1 (gemm = 1, with the
 * activation) or GEMM2 (gemm = 2, with the routing weight) on this problem in
 * the pipeline `mode` resolves to, as a static NUL-terminated name (owned by
 * the library, never freed): "dma_kmajor_kernel", "dma_skinny_kernel",
 * "big_gemm_kernel<128>", "big_gemm_kernel<256>", "gemm1_swiglu_kernel",
 * "gemm2_weight_kernel", "mx_kmajor_kernel", "mx_gemm1_kernel",
 * "mx_gemm2_kernel", "fused_dma_kernel", "fused_bf16_kernel",
 * "mx_fused_kernel", or "none" for
 * T = 0. NULL on an invalid problem, mode or gemm. Host only: it evaluates
 * the same dispatch rules as the launch, which depend on the shapes only
 * (the routing itself is not known before the route step), except for
 * E == 1: a single group of few rows streams its weights through the decode
 * kernels while the prefill kernels would get fewer tiles than half the
 * current device's compute units (256 on MI355X; 256 is also assumed when
 * no device is visible). Not defined by the pages; it exists so that
 * callers and tests can see which path a shape takes. */
MOE_FFN_API const char* moe_ffn_gemm_kernel(const moe_ffn_problem* p, int mode, int gemm);

/* The forward pass.
 *   x            : bf16 [T, D], or e4m3 codes [T, D] for MXFP8 and MXFP4.
 *   w1           : bf16 [E, 2H, D] (gate rows then up rows per expert), or
 *                  e4m3 codes for MXFP8, or packed e2m1 codes [E, 2H, D/2]
 *                  for MXFP4.
 *   w2           : bf16 [E, D, H], or e4m3 codes for MXFP8, or packed e2m1
 *                  codes [E, D, H/2] for MXFP4.
 *   topk_ids     : int32 [T, topk]; an id outside [0, E) is a dropped route
 *                  that contributes nothing.
 *   topk_weights : fp32 [T, topk], used as given (not renormalized).
 *   out          : bf16 [T, D]; fully overwritten in every mode.
 * Enqueues route, GEMM and combine kernels on `stream`; T == 0 is a
 * successful no-op. */
MOE_FFN_API int moe_ffn_forward(const moe_ffn_problem* p, const void* x, const void* w1,
                                const void* w2, const int32_t* topk_ids,
                                const float* topk_weights, void* out, int mode, void* stream);

/* moe_ffn_forward, additionally recording caller-created HIP events
 * (hipEvent_t, passed as void*) on `stream` at the boundaries of its four
 * kernel stages, for per-kernel timing without a host synchronization:
 *   events[0] before the route step        events[1] after it
 *   events[2] after stage 2 (SPLIT: GEMM1 + SwiGLU; FUSED: nothing, the
 *             route step clears the fp32 accumulator)
 *   events[3] after stage 3 (SPLIT: GEMM2 + weight; FUSED: fused kernel)
 *   events[4] after stage 4 (SPLIT: combine;        FUSED: fp32 -> bf16, or
 *             nothing where the fused kernel converts each completed row)
 * n_events must be 5 (or 0, which makes it moe_ffn_forward). The events
 * stay owned by the caller. */
MOE_FFN_API int moe_ffn_forward_events(const moe_ffn_problem* p, const void* x, const void* w1,
                                       const void* w2, const int32_t* topk_ids,
                                       const float* topk_weights, void* out, int mode,
                                       void* stream, void* const* events, int n_events);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_ffn_forward with the workspace taken from a static device array of
 * the library instead of p->workspace (which is ignored, as is
 * p->workspace_bytes). The array is MOE_FFN_NOALLOC_SCRATCH_BYTES (64 MiB)
 * per device; each GPU the library runs on holds it from the first call on
 * that device until the process ends. The call allocates nothing and calls
 * no allocating routine. A problem whose workspace (moe_ffn_workspace_bytes
 * for the mode AUTO resolves to) exceeds the array returns MOE_FFN_ESCRATCH
 * before anything is enqueued; 64 MiB holds the decode-shaped passes (the
 * 64-token, 32-expert, D=6144, H=2048 split pass needs about 10 MB) and the
 * fused pipeline up to about 4M tokens x D of fp32 accumulator. Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be ordered
 * by the caller. The pass writes every scratch region before reading it, so
 * what an earlier call left there does not matter. The current device must
 * be the one `stream` belongs to. Other arguments as for moe_ffn_forward. */
#define MOE_FFN_NOALLOC_SCRATCH_BYTES (64ll << 20)
MOE_FFN_API int moe_ffn_forward_noalloc(const moe_ffn_problem* p, const void* x, const void* w1,
                                        const void* w2, const int32_t* topk_ids,
                                        const float* topk_weights, void* out, int mode,
                                        void* stream);

/* The router ahead of the pass (Prime Flash MoE, section 1 "The
 * computation": the pass starts from each token's top-k experts and their
 * normalized routing weights): softmax over each token's E logits, the k
 * most probable experts, most probable first with ties to the lower expert
 * id, and their probabilities renormalized to sum to 1. Softmax is strictly
 * increasing, so the order is that of the fp32 logits themselves and the
 * ids are exact; weights are within a few fp32 ulps of
 * exp(l_j - l_max) / sum over the picks of exp(l_i - l_max).
 *   logits       : fp32 [T, E], 4-byte aligned. -inf ranks after every
 *                  finite logit (a masked expert: picked only if fewer
 *                  than k are finite, with weight 0); -0 equals +0; a NaN
 *                  ranks below everything else (NaNs by id) and, if
 *                  picked, makes the token's weights NaN. Each token needs
 *                  at least one finite logit for finite weights.
 *   topk_ids     : int32 [T, topk] (output).
 *   topk_weights : fp32 [T, topk] (output).
 * 1 <= topk <= min(E, 64), E <= 8192. T == 0 is a successful no-op. */
MOE_FFN_API int moe_ffn_router(const float* logits, int32_t T, int32_t E, int32_t topk,
                               int32_t* topk_ids, float* topk_weights, void* stream);

/* moe_ffn_forward_events starting from router logits: the router above
 * writes topk_ids / topk_weights (outputs here, [T, topk] each, 16-byte
 * aligned) and the route step reads them; on the multi-kernel route path
 * the router kernel also builds the route's per-segment expert histogram,
 * so the ids are read back only once. The same workspace as
 * moe_ffn_forward. events[0..1] bracket router and route together;
 * n_events is 0 or 5 as for moe_ffn_forward_events. */
MOE_FFN_API int moe_ffn_forward_logits(const moe_ffn_problem* p, const void* x, const void* w1,
                                       const void* w2, const float* logits, int32_t* topk_ids,
                                       float* topk_weights, void* out, int mode, void* stream,
                                       void* const* events, int n_events);

/* One shared expert next to the routed ones ("GC-MoE on SM120", section
 * 4.7: a shared expert runs on every token, and its output is added into
 * the same fp32 sum that folds the token's k routed slots):
 *     out[t] = sum_j w[t,j] * y(t, ids[t,j]) + W2s (silu(W1s_gate x_t) * W1s_up x_t)
 *   shared_w1 : bf16 [2Hs, D] (gate rows, then up rows), 16-byte aligned.
 *   shared_w2 : bf16 [D, Hs].
 *   Hs        : the shared expert's intermediate size, a multiple of 64.
 * The shared expert runs first, as a grouped GEMM of one group of all T
 * tokens; the combine (split) or the accumulator conversion (fused) adds
 * its rows. bf16 only (MXFP8 returns MOE_FFN_EUNSUPPORTED). The workspace
 * must hold moe_ffn_shared_workspace_bytes(); events as for
 * moe_ffn_forward_events, with events[0..1] bracketing the shared expert
 * and the route step together. */
MOE_FFN_API size_t moe_ffn_shared_workspace_bytes(const moe_ffn_problem* p, int32_t Hs, int mode);
MOE_FFN_API int moe_ffn_forward_shared(const moe_ffn_problem* p, const void* x, const void* w1,
                                       const void* w2, const int32_t* topk_ids,
                                       const float* topk_weights, const void* shared_w1,
                                       const void* shared_w2, int32_t Hs, void* out, int mode,
                                       void* stream, void* const* events, int n_events);

/* Activation variant ("Porting Block-Scaled GEMM Kernels from Blackwell
 * to Rubin", section 5.3: gate and up scaled by the expert's global scale
 * alpha, clamped in the gpt-oss style -- the gate from above only, up on
 * both sides -- then up * silu(gate); "GC-MoE on SM120", section 4.8: the
 * route weight multiplies gate and up before the activation):
 *     s   = alpha[e] * (weight_before_act ? w : 1)
 *     act = silu(min(s*gate, limit)) * clamp(s*up, -limit, limit)   (CLAMPED)
 *     act = silu(s*gate) * (s*up)                                  (SWIGLU)
 *     y   = W2[e] act, summed with weight (weight_before_act ? 1 : w).
 *   kind              : MOE_FFN_ACT_SWIGLU or MOE_FFN_ACT_CLAMPED_SWIGLU.
 *   limit             : the clamp bound (finite, > 0) for CLAMPED.
 *   alpha             : fp32 [E] device array of per-expert scales, or NULL
 *                       (1.0 for every expert); 4-byte aligned.
 *   weight_before_act : 0 or 1. */
enum { MOE_FFN_ACT_SWIGLU = 0, MOE_FFN_ACT_CLAMPED_SWIGLU = 1 };
typedef struct moe_ffn_activation {
    int32_t kind;
    float limit;
    const float* alpha;
    int32_t weight_before_act;
} moe_ffn_activation;

/* moe_ffn_forward_events with an activation variant. bf16 only, on the
 * split pipeline: AUTO runs SPLIT (size the workspace with
 * moe_ffn_workspace_bytes(p, MOE_FFN_SPLIT)); FUSED or MXFP8 return
 * MOE_FFN_EUNSUPPORTED. */
MOE_FFN_API int moe_ffn_forward_act(const moe_ffn_problem* p, const void* x, const void* w1,
                                    const void* w2, const int32_t* topk_ids,
                                    const float* topk_weights, const moe_ffn_activation* act,
                                    void* out, int mode, void* stream, void* const* events,
                                    int n_events);

/* Workspace bytes moe_ffn_route needs (host only; 0 on invalid input). */
MOE_FFN_API size_t moe_ffn_route_workspace_bytes(int32_t T, int32_t topk, int32_t E);

/* The permutation step on its own (the sorted order the grouped GEMMs read:
 * Prime Flash MoE, section 1, the `offs` group offsets of the grouped GEMM
 * formulation, and section 8, routing and sorting). With P = T*topk and
 * pairs p = t*topk + j:
 *   counts         int32 [E]   : valid pairs routed to each expert.
 *   offsets        int32 [E+1] : exclusive prefix sum of counts.
 *   sorted_to_pair int32 [P]   : the pairs of expert 0, then expert 1, ...,
 *                                ascending p inside each expert (a stable
 *                                sort); entries from offsets[E] on are -1.
 *   pair_to_sorted int32 [P]   : the inverse map; -1 for dropped routes.
 * The result is unique, so it is bit-exact against any stable sort. */
MOE_FFN_API int moe_ffn_route(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_to_pair,
                              int32_t* pair_to_sorted, void* workspace, size_t workspace_bytes,
                              void* stream);

/* MX-fp8 quantization of fp32 rows along the last dim (Prime Flash MoE,
 * section 7: e4m3 data with one e8m0 scale per 32 contiguous K elements;
 * the scale rule reads "Porting Block-Scaled GEMM Kernels from Blackwell to
 * Rubin", section 6.2: the scale is amax/448 rounded up to a power of two,
 * i.e. s = the smallest integer with amax <= 448 * 2^s, clamped to
 * [-127, 127], s = -127 for an all-zero block; codes = e4m3(v * 2^-s) with
 * round-to-nearest-even, saturating at +-448).
 *   src    : fp32 [rows, K], K a multiple of 32.
 *   codes  : uint8 [rows, K] e4m3 codes.   scales : uint8 [rows, K/32].
 * The same rule requantizes the SwiGLU output inside the MXFP8 pass. */
MOE_FFN_API int moe_ffn_mx_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                                    uint8_t* scales, void* stream);

/* MXFP4 quantization of fp32 rows along the last dim, for expert weights
 * ("GC-MoE on SM120", scale formats: E2M1 codes with a UE8M0 exponent per
 * 32 contiguous elements). The pages give no fp4 scale rule; this reads the
 * MX-fp8 rule above with E2M1's largest magnitude 6 in place of 448:
 * s = the smallest integer with amax <= 6 * 2^s, clamped to [-127, 127]
 * (-127 for an all-zero block); codes = e2m1(v * 2^-s), nearest value with
 * ties to the even code, saturating at +-6.
 *   src    : fp32 [rows, K], K a multiple of 32, 16-byte aligned.
 *   codes  : uint8 [rows, K/2], two codes per byte, even K index in the low
 *            nibble, 4-byte aligned.
 *   scales : uint8 [rows, K/32].
 * Asynchronous on `stream`; MOE_FFN_EINVAL_SHAPE / _PTR on bad arguments. */
MOE_FFN_API int moe_ffn_mxfp4_quantize(const float* src, int64_t rows, int32_t K, uint8_t* codes,
                                       uint8_t* scales, void* stream);

/* A static string naming `code`. */
MOE_FFN_API const char* moe_ffn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
