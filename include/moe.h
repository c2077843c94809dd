/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts layer.
 *
 * What the layer computes.  "Mixture-of-Experts kernel engineering on Amazon
 * SageMaker AI" (summary text, fused-MoE definition) describes a fused MoE
 * as one batched GPU operation that merges token routing, data shuffling
 * and the expert networks, in place of sequential per-expert loops.  The
 * expert GEMM there is C = A.B with A the tokens [M,K] and B the expert
 * weights [K,N]; its Swap-AB passage (Figure 1) computes the transpose
 * C^T[N,M] = B^T[N,K].A^T[K,M], so expert weights are held output-major
 * with the reduction dimension contiguous.  This library keeps that layout:
 *
 *   x        bf16 [M,K]      tokens, row-major
 *   w_router bf16 [E,K]      router weights
 *   w1       [E,2N,K]        per expert: rows [0,N) gate, rows [N,2N) up
 *   w2       [E,K,N]         per expert: down projection
 *   out      bf16 [M,K]
 *
 *   out[t] = sum_{j<topk} w[t,j] * W2[e_tj] . (silu(W1g[e_tj].x_t) * (W1u[e_tj].x_t))
 *
 * with (e_t, w_t) the top-k experts of softmax(x_t.W_r^T + bias) and their
 * probabilities renormalised over the k picked (ties to the lower expert id,
 * slots in descending order).  FP8 follows the same page's FP8 passage
 * ("tensor-quantized" models: one fp32 scale per expert weight tensor);
 * activations are quantised per token at run time.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the size_t* of moe_fused_forward, which is a host pointer.  The library
 *     never allocates or frees device memory and is re-entrant; calls on
 *     different streams may overlap as long as their buffers do not.  The
 *     one exception is moe_fused_forward_noalloc, whose scratch is a static
 *     device array of the library (one per GPU, see there).
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the default stream).  The library never synchronises the host.
 *   - Arguments are validated before any HIP call, so every error path is
 *     testable on a host without a GPU: a call that returns an error has
 *     enqueued nothing.  MOE_ERR_HIP reports a launch failure
 *     (hipGetLastError after the launches).
 *   - Device pointers must be 16-byte aligned; tensors are dense row-major
 *     with no strides.
 *   - M == 0 is a valid no-op returning MOE_OK.
 */
#ifndef MOE_LAYER_MOE_H
#define MOE_LAYER_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null required pointer, negative size, topk out of [1,E], misalignment */
    MOE_ERR_UNSUPPORTED = 2, /* a size outside the supported envelope (see each call) */
    MOE_ERR_WORKSPACE = 3,   /* workspace smaller than the size the query returned */
    MOE_ERR_HIP = 4          /* a HIP launch failed */
} moe_status;

typedef enum {
    MOE_BF16 = 0,              /* w1/w2 bf16; w1_scale/w2_scale must be NULL */
    MOE_FP8_E4M3 = 1,          /* w1/w2 OCP E4M3FN codes (uint8) with fp32 per-expert
                                  scales w1_scale [E], w2_scale [E] */
    MOE_FP8_E4M3_ROWWISE = 2,  /* e4m3 codes with fp32 per-channel scales: one per
                                  output row, w1_scale [E,2N] (gate rows, then up
                                  rows), w2_scale [E,K] (a scheme the pages do not
                                  describe: the per-tensor one, per row) */
    MOE_MXFP4_E2M1 = 3         /* OCP MXFP4 weights (also beyond the pages): e2m1
                                  codes two per byte, the even element in the low
                                  nibble, w1 [E,2N,K/2], w2 [E,K,N/2]; one E8M0 scale
                                  byte (2^(e-127)) per 32 elements of a row,
                                  w1_scale [E,2N,K/32], w2_scale [E,K,N/32] (uint8
                                  arrays); activations are quantised per token to
                                  e4m3 as for MOE_FP8_E4M3 */
} moe_dtype;

/* Kernel family used by the expert GEMMs; results agree up to fp32
 * summation order whichever is picked. */
typedef enum {
    MOE_REGIME_AUTO = 0,    /* DECODE while M*topk <= 8*E (bf16: at most 8
                               token-slots per expert on average),
                               M*topk <= 16*E (e4m3) or M*topk <= 24*E
                               (MXFP4), else PREFILL: the measured crossovers */
    MOE_REGIME_DECODE = 1,  /* Swap-AB: weight rows on the MFMA row dimension;
                               blocks of 16, 32 or 64 sorted rows sized from
                               the expected rows per expert */
    MOE_REGIME_PREFILL = 2  /* full MFMA tiles of token rows x weight rows
                               (blocks of 128 or 256 sorted rows; 256 for
                               MXFP4) */
} moe_regime;

/* Supported envelope: 1 <= E <= 256, 1 <= topk <= min(E,16), K >= 1 and
 * N >= 1; moe_fused_forward additionally needs K and N multiples of 128
 * (of 256, and K <= 16384, for MOE_MXFP4_E2M1),
 * M*topk < 2^30, (M*topk + 256*E) * N * b < 2^31 with b = 2 for bf16 and
 * 1 otherwise (the sorted activation rows GEMM2 reads), M*K*2 < 2^31 and
 * 2*N*K*2 < 2^31 (one expert's W1). */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16

/*
 * moe_topk -- router: logits, top-k selection and routing weights.
 *
 * Source: "Mixture-of-Experts kernel engineering on Amazon SageMaker AI"
 * (summary text, fused-MoE definition: token routing is part of the fused
 * op); "AI混合专家模型性能优化全链路解析", chapter 1 (experts are chosen by
 * top-k over the router logits).
 *
 *   x            bf16 [M,K]
 *   w_router     bf16 [E,K]
 *   router_bias  fp32 [E] added to every token's logits, or NULL
 *   topk_ids     out int32 [M,topk]: the topk largest logits, descending,
 *                equal logits ordered by ascending expert id
 *   topk_weights out fp32 [M,topk]: exp(l_j - l_0) / sum_j' exp(l_j' - l_0)
 *   logits       out fp32 [M,E] (required): each logit is the fp32 rounding
 *                of an fp64-accumulated dot product plus bias
 *
 * Errors: INVALID_ARG for null pointers (x, w_router, topk_ids,
 * topk_weights, logits), M < 0, K < 1, topk < 1 or topk > E;
 * UNSUPPORTED for E > 256 or topk > 16.
 */
moe_status moe_topk(const void *x, const void *w_router, const float *router_bias,
                    int M, int K, int E, int topk,
                    int32_t *topk_ids, float *topk_weights, float *logits,
                    void *stream);

/*
 * moe_align -- expert-sorted, block-padded permutation of the token slots.
 *
 * Source: "Mixture-of-Experts kernel engineering on Amazon SageMaker AI"
 * (summary text: data shuffling is part of the fused op; the FP8 passage's
 * scheduling around variable token bucketing); "Amazon SageMaker AI上的混合
 * 专家模型内核工程优化", section on H200 bottlenecks (per-expert batch sizes
 * change dynamically).
 *
 * Slot p = t*topk + j (token t, slot j) is sorted stably by expert id, so
 * each expert's slots are contiguous and ascending in p; each expert's
 * segment is padded to a multiple of block_m with the sentinel M*topk.
 *
 *   topk_ids       int32 [M,topk], each in [0,E)
 *   sorted_ids     out int32 [cap], cap = M*topk + E*(block_m-1); entries at
 *                  and past num_padded hold the sentinel
 *   block_expert   out int32 [cap / block_m]: expert owning each block of
 *                  block_m sorted rows, -1 past the last used block
 *   expert_offsets out int32 [E+1]: padded segment starts, [E] = num_padded
 *   num_padded     out int32 [1]
 *
 * Errors: INVALID_ARG for null pointers, M < 0, topk < 1, E < 1 or
 * block_m < 1; UNSUPPORTED for E > 256, block_m > 1024 or M*topk >= 2^30.
 * Ids outside [0,E) are a caller error; they are clamped into range on the
 * device so no access goes out of bounds, and the result is unspecified.
 */
moe_status moe_align(const int32_t *topk_ids, int M, int topk, int E, int block_m,
                     int32_t *sorted_ids, int32_t *block_expert,
                     int32_t *expert_offsets, int32_t *num_padded, void *stream);

/*
 * moe_align_ex -- moe_align with a caller workspace, for large batches: the
 * same outputs, bit for bit.  Source: as moe_align (the fused op's data
 * shuffling; per-expert batch sizes that change from call to call).  Above 2048 token-slots it runs over many
 * workgroups -- per 1024-slot chunk a count of the slots of each expert,
 * one scan that turns the counts into the padded segment starts and each
 * chunk's first position per expert, then per chunk the stable scatter --
 * instead of one workgroup walking all chunks, and keeps the chunk counts in
 * the workspace.  The fused layer runs this align on its own workspace.
 *
 *   topk_ids ... num_padded   as moe_align
 *   workspace        device buffer of at least *workspace_bytes bytes
 *                    (256-byte aligned), or NULL to query: the call stores the
 *                    required size (256 bytes up to 2048 slots, where
 *                    the buffer is not used) in *workspace_bytes,
 *                    enqueues nothing and returns MOE_OK
 *   workspace_bytes  host pointer: in = size of `workspace`, out = required
 *
 * Errors: as moe_align, plus INVALID_ARG for a null workspace_bytes or a
 * workspace not 256-byte aligned; WORKSPACE if *workspace_bytes is below the
 * required size.
 */
moe_status moe_align_ex(const int32_t *topk_ids, int M, int topk, int E, int block_m,
                        int32_t *sorted_ids, int32_t *block_expert,
                        int32_t *expert_offsets, int32_t *num_padded, void *workspace,
                        size_t *workspace_bytes, void *stream);

/*
 * moe_quant_rows_e4m3 -- per-row dynamic FP8 quantisation of bf16 rows, the
 * step the fused forward applies to the tokens before GEMM1 in the e4m3 path.
 *
 * Source: "Mixture-of-Experts kernel engineering on Amazon SageMaker AI"
 * (summary text, FP8 passage: FP8 tensor scaling is one of the steps fused
 * into the single pass); "Amazon SageMaker AI上的混合专家模型内核工程优化",
 * section 2 (scale factors recomputed dynamically at inference time).
 *
 *   x      bf16 [M,K]
 *   q      out uint8 [M,K]: OCP E4M3FN code of x/s, round to nearest even,
 *          magnitudes clamped to 448
 *   scale  out fp32 [M]: s = amax_k |x[t,k]| / 448 (one correctly rounded
 *          fp32 division), 1 when the row is all zero
 *
 * Errors: INVALID_ARG for null pointers, M < 0 or K < 1; UNSUPPORTED for
 * M*K >= 2^31.
 */
moe_status moe_quant_rows_e4m3(const void *x, int M, int K, uint8_t *q, float *scale,
                               void *stream);

/*
 * moe_fused_forward -- the whole layer: router, permutation, GEMM1 with the
 * SiLU*up epilogue, GEMM2 with the routing-weighted un-permute, combine.
 *
 * Source: "Mixture-of-Experts kernel engineering on Amazon SageMaker AI"
 * (summary text: fused-MoE definition; decode-phase passage and Figure 1,
 * Swap-AB; FP8 passage: FP8 tensor scaling, matrix multiplication and
 * expert aggregation fused, for per-tensor FP8 models).
 *
 *   x, w_router, router_bias   as moe_topk
 *   w1        [E,2N,K] bf16 or e4m3 (dtype); MXFP4: [E,2N,K/2] bytes, two
 *             e2m1 codes each (even element in the low nibble)
 *   w2        [E,K,N]  bf16 or e4m3; MXFP4: [E,K,N/2] bytes
 *   w1_scale  per dtype: fp32 [E] (MOE_FP8_E4M3), fp32 [E,2N]
 *             (MOE_FP8_E4M3_ROWWISE), uint8 E8M0 [E,2N,K/32] (MOE_MXFP4_E2M1)
 *             or NULL (MOE_BF16); w2_scale likewise fp32 [E], fp32 [E,K],
 *             uint8 [E,K,N/32] or NULL.  The element type follows dtype, so
 *             the parameters are untyped.
 *   out       out bf16 [M,K]
 *   workspace device buffer of at least *workspace_bytes bytes (256-byte
 *             aligned), or NULL to query: with workspace == NULL the call
 *             stores the required size in *workspace_bytes, enqueues
 *             nothing and returns MOE_OK.  The size depends only on
 *             (dtype, M, K, N, E, topk).
 *   workspace_bytes  host pointer: in = size of `workspace`, out = required
 *
 * FP8: x is quantised per token to e4m3 with scale amax/448; the SiLU*up
 * activation per token-slot likewise; GEMM accumulation is fp32.
 *
 * After the call completes (in stream order) the workspace holds the
 * layer's own routing at the offsets moe_fused_plan reports: logits fp32
 * [M,E], topk_ids int32 [M,topk], topk_weights fp32 [M,topk], sorted_ids
 * int32 [sorted_rows], block_expert int32 [max_blocks], expert_offsets int32
 * [E+1] and num_padded int32 [1], each with the meaning moe_topk and
 * moe_align give it (block size block_m of the plan).  These are the values
 * the GEMMs consumed, so a caller can check or reuse them.
 *
 * Errors: as moe_topk, plus INVALID_ARG for null w1/w2/out/workspace_bytes,
 * N < 1, a bad dtype, scales given for bf16 or missing for fp8;
 * UNSUPPORTED for K or N not a multiple of 128 or the size limits above
 * (MXFP4 also: K or N not a multiple of 256, K > 16384, or, on the decode
 * kernels, N that cannot be split into GEMM2 reduction ranges of at most 8192
 * multiples of 256);
 * WORKSPACE if *workspace_bytes is below the required size.
 */
moe_status moe_fused_forward(const void *x, const void *w_router, const float *router_bias,
                             const void *w1, const void *w2,
                             const void *w1_scale, const void *w2_scale,
                             int dtype, int M, int K, int N, int E, int topk,
                             void *out, void *workspace, size_t *workspace_bytes,
                             void *stream);

/* moe_fused_forward with the GEMM kernel family chosen by the caller
 * (moe_regime).  Used to cross-check the Swap-AB decode kernels against the
 * full-tile kernels on identical inputs (C^T = B^T.A^T, Figure 1 of the
 * page above). */
moe_status moe_fused_forward_ex(const void *x, const void *w_router, const float *router_bias,
                                const void *w1, const void *w2,
                                const void *w1_scale, const void *w2_scale,
                                int dtype, int M, int K, int N, int E, int topk,
                                int regime, void *out, void *workspace,
                                size_t *workspace_bytes, void *stream);

/* moe_fused_forward_ex instrumented with timing events: `events` is a host
 * array of 8 hipEvent_t handles created by the caller.  events[0] is
 * recorded on `stream` before the first launch and events[i] after stage i:
 * 1 router logits, 2 top-k (+ token quantisation), 3 align, 4 GEMM1 +
 * SiLU*up, 5 activation quantisation (recorded with nothing before it on
 * the bf16 path), 6 GEMM2, 7 combine.  Used by the benchmark to time each
 * kernel on the stream it runs on.  Errors as moe_fused_forward_ex, plus
 * INVALID_ARG for a NULL `events` when workspace is non-NULL. */
moe_status moe_fused_forward_timed(const void *x, const void *w_router, const float *router_bias,
                                   const void *w1, const void *w2,
                                   const void *w1_scale, const void *w2_scale,
                                   int dtype, int M, int K, int N, int E, int topk,
                                   int regime, void *out, void *workspace,
                                   size_t *workspace_bytes, void *stream,
                                   void *const *events);

/*
 * moe_plan / moe_fused_plan -- the launch plan moe_fused_forward_ex takes for
 * a shape: the kernel family (the Swap-AB decode kernels or full tiles,
 * "Mixture-of-Experts kernel engineering on Amazon SageMaker AI", decode-
 * phase passage and Figure 1), the block size of the expert-sorted rows, the
 * reduction splits, the workspace size and where in the workspace the
 * routing outputs of the call live (see moe_fused_forward).  The plan
 * depends only on (dtype, M, K, N, E, topk, regime); the query makes no HIP
 * call.
 *
 * Errors: INVALID_ARG for a NULL plan and the argument errors of
 * moe_fused_forward_ex that concern these values; UNSUPPORTED as there.
 */
typedef struct {
    int32_t regime;        /* kernel family used: MOE_REGIME_DECODE or MOE_REGIME_PREFILL */
    int32_t block_m;       /* rows per block of the sorted list */
    int32_t sorted_rows;   /* entries of sorted_ids: M*topk + E*(block_m-1) */
    int32_t max_blocks;    /* entries of block_expert: sorted_rows / block_m */
    int32_t gemm2_splits;  /* GEMM2 reduction split into fp32 partial rows */
    int32_t logit_splits;  /* router reduction split (fp64 partials) */
    int32_t fused_decode;  /* 1: one or two tokens with bf16 weights, the router
                              (logits, top-k, align) computed inside the GEMM1 launch:
                              three launches instead of five */
    int32_t reserved;      /* zero */
    uint64_t workspace_bytes;
    uint64_t logits_offset;          /* byte offsets into the workspace */
    uint64_t topk_ids_offset;
    uint64_t topk_weights_offset;
    uint64_t sorted_ids_offset;
    uint64_t block_expert_offset;
    uint64_t expert_offsets_offset;
    uint64_t num_padded_offset;
} moe_plan;

moe_status moe_fused_plan(int dtype, int M, int K, int N, int E, int topk, int regime,
                          moe_plan *plan);

/*
 * moe_fused_graph_create / _launch / _destroy -- moe_fused_forward_ex
 * captured once into a HIP graph, for callers that re-run the layer on fixed
 * buffers (serving loops): each moe_fused_graph_launch is one graph launch
 * instead of the layer's six to eight kernel launches.
 * ("AI混合专家模型性能优化全链路解析" §3.1 captures the expert computation in
 * a graph to cut launch overhead; this is the HIP form of that step.)
 *
 *   arguments    as moe_fused_forward_ex; workspace_bytes is the size of the
 *                caller's workspace (not a pointer: no size query here)
 *   stream       create: the stream the one eager call runs on
 *   graph        out: the handle (NULL on error)
 *
 * Create runs the layer once eagerly on `stream` (this loads every kernel of
 * the sequence and computes `out`), then captures the same launch sequence
 * on a stream of its own and instantiates the graph.  The graph is bound to
 * the pointers given: a launch recomputes out from whatever x, the weights
 * and the scales hold when it runs, using the same workspace; launches that
 * overlap with each other or with other users of that workspace race.
 * Launch enqueues the graph on `stream` (asynchronous).  Destroy releases
 * the graph (NULL is a no-op); the caller keeps every buffer.
 *
 * Errors: create -- as moe_fused_forward_ex (checked before any HIP call),
 * INVALID_ARG for a NULL graph pointer, NULL workspace or M == 0, WORKSPACE
 * when workspace_bytes is below the required size, HIP when the capture or
 * instantiation fails; launch -- INVALID_ARG for a NULL handle, HIP when the
 * launch fails.
 */
typedef struct moe_graph_s *moe_graph;
moe_status moe_fused_graph_create(const void *x, const void *w_router, const float *router_bias,
                                  const void *w1, const void *w2,
                                  const void *w1_scale, const void *w2_scale,
                                  int dtype, int M, int K, int N, int E, int topk, int regime,
                                  void *out, void *workspace, size_t workspace_bytes,
                                  void *stream, moe_graph *graph);
moe_status moe_fused_graph_launch(moe_graph graph, void *stream);
moe_status moe_fused_graph_destroy(moe_graph graph);

/*
 * moe_fused_forward_noalloc -- moe_fused_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, no allocation,
 * no allocating library call.  The scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library; every GPU the library runs
 * on holds its own copy until the process ends.  Its device address is
 * looked up (hipGetSymbolAddress) on the first call on each device, with
 * that device current.
 *
 *   arguments as moe_fused_forward (regime automatic), without workspace
 *
 * The scratch keeps the last call's contents; every value the layer reads
 * from it is written earlier in the same call.  Calls that overlap on one
 * GPU (different streams, or different host threads) share the one array
 * and race: the caller must order them, e.g. on a single stream.  The
 * routing outputs of the last call can be read at the offsets
 * moe_fused_plan reports, relative to the array.
 *
 * Errors: as moe_fused_forward; WORKSPACE when the shape needs more than
 * MOE_NOALLOC_SCRATCH_BYTES (moe_fused_plan reports the size); HIP when the
 * array's address cannot be obtained; UNSUPPORTED on a device ordinal >= 64.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
moe_status moe_fused_forward_noalloc(const void *x, const void *w_router,
                                     const float *router_bias, const void *w1, const void *w2,
                                     const void *w1_scale, const void *w2_scale, int dtype,
                                     int M, int K, int N, int E, int topk, void *out,
                                     void *stream);

/* Static, NUL-terminated name of a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_MOE_H */
