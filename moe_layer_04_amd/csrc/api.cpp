// api.cpp -- the C ABI of include/moe.h: argument validation (before any HIP
// call), the workspace layout, the choice of kernel family and the launch
// sequence of the fused MoE layer.
//
// Launch sequence of moe_fused_forward (all on the caller's stream, no host
// synchronisation, grids sized from host-known upper bounds so no device
// value is read back):
//   1 router logits (fp64 dot products) (+ x -> e4m3)
//   2 top-k + weights                         3 align (sorted rows, block owners)
//     (2-3 are one single-workgroup launch for up to 1024 token-slots)
//   4 GEMM1 + SiLU*up
//   5 (e4m3) per-row activation quantisation  6 GEMM2 * routing weight, scattered
//   7 combine into bf16 out
#include <cmath>
#include <hip/hip_runtime.h>
#include <mutex>
#include <new>
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"
#include "launch.hpp"
#include "tuning.hpp"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kDecodeBlock = moe::kDecodeRows;
constexpr int kPrefillBlock = moe::kPrefillRows;
constexpr size_t kAlign = 256;
bool misaligned(const void* p) { return p && ((uintptr_t)p & 15u); }

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    int regime = MOE_REGIME_DECODE;
    int block = kDecodeBlock;
    int cap = 0;         // rows of the sorted list: M*topk + E*(block-1)
    int max_blocks = 0;  // cap / block: entries of block_expert
    // Launch grids cover at most this many blocks: summed over the experts
    // that received rows, ceil(c_e / block) <= floor(slots / block) +
    // (number of such experts), and that number is <= min(E, slots).
    int grid_blocks = 0;
    int nsplit = 1;      // GEMM2 reduction split (decode)
    int lsplit = 1;      // router-logit reduction split (fp64 partials in lpart)
    bool fused = false;  // bf16, one or two tokens: the two-launch decode
    size_t lpart = 0;
    size_t logits = 0, ids = 0, wts = 0, sorted = 0, bexp = 0, offs = 0, npad = 0;
    size_t inv = 0;  // FP8 activations: sorted position of each slot
    bool align_multi = false;  // the multi-workgroup align (scratch achunk, atot)
    size_t achunk = 0, atot = 0;
    size_t xq = 0, xs = 0, amax = 0, act = 0, actq = 0, as = 0, ypart = 0, total = 0;
};

// every dtype with e4m3-quantised activations (the e4m3 and MXFP4 weights)
bool is_fp8(int dtype) {
    return dtype == MOE_FP8_E4M3 || dtype == MOE_FP8_E4M3_ROWWISE || dtype == MOE_MXFP4_E2M1;
}

Plan make_plan(int dtype, int M, int K, int N, int E, int topk, int regime) {
    Plan p;
    const long slots = (long)M * topk;
    // the automatic choice routes one or two tokens with bf16 weights inside
    // the GEMM1 launch; a forced family keeps the separate routing kernels
    p.fused = regime == MOE_REGIME_AUTO && dtype == MOE_BF16 &&
              moe::decode_fused_fits(M, K, N, E, topk);
    if (regime == MOE_REGIME_AUTO) {
        const long rows = dtype == MOE_BF16           ? moe::tune::kDecodeMaxRowsPerExpert
                          : dtype == MOE_MXFP4_E2M1 ? moe::tune::kMxDecodeMaxRowsPerExpert
                                                      : moe::tune::kFp8DecodeMaxRowsPerExpert;
        regime = slots <= rows * E ? MOE_REGIME_DECODE : MOE_REGIME_PREFILL;
    }
    p.regime = regime;
    p.block = (regime == MOE_REGIME_DECODE) ? kDecodeBlock : kPrefillBlock;
    // full tiles: 128-row token blocks when the experts receive few rows
    // (tuning.hpp); those kernels are built for K % 256 == 0.  MXFP4 weights
    // have 256-row tiles only.
    const long small_rows = dtype == MOE_BF16 ? moe::tune::kPrefillSmallTileMaxRows
                                              : moe::tune::kPrefillFp8SmallTileMaxRows;
    if (regime == MOE_REGIME_PREFILL && K % 256 == 0 && dtype != MOE_MXFP4_E2M1 &&
        slots <= small_rows * (slots < E ? slots : E))
        p.block = moe::kPrefillSmallRows;
    // larger decode blocks when experts receive more rows (sized in tuning.hpp)
    if (regime == MOE_REGIME_DECODE) p.block = moe::tune::decode_block_rows(slots, E);
    // the routing GEMM1 gives every routed expert one 16-row block
    if (p.block != kDecodeBlock) p.fused = false;
    p.cap = (int)(slots + (long)E * (p.block - 1));
    p.max_blocks = p.cap / p.block;
    {
        const long bound = slots / p.block + (slots < E ? slots : E);
        p.grid_blocks = (int)(bound < p.max_blocks ? bound : p.max_blocks);
    }
    if (regime == MOE_REGIME_DECODE) {
        // GEMM2's reduction split: the rule and its measurements are in tuning.hpp
        const long est_blocks = slots < E ? slots : E;
        const int mx = dtype == MOE_MXFP4_E2M1;
        const long tiles = est_blocks * (K / (mx ? 256 : 128));  // output rows per workgroup
        // weight bytes per output row of a wave's tile, per reduction element
        // (bf16: 32 rows x 2 B; e4m3: 32 x 1 B; MXFP4: 64 rows x 1/2 B)
        const long row_bytes = dtype == MOE_BF16 ? 64 : 32;
        // each split's reduction length stays a multiple of the kernels' step
        const int gran = mx ? 256 : 128;
        if (tiles < moe::tune::kDecodeSplitUnsplitTiles)
            while (tiles * p.nsplit < moe::tune::kDecodeSplitTargetTiles && p.nsplit < 16 &&
                   (N / (p.nsplit * 2)) % gran == 0 &&
                   row_bytes * (N / (p.nsplit * 2)) >= moe::tune::kDecodeSplitMinWaveBytes)
                p.nsplit *= 2;
        if (mx)
            while (N / p.nsplit > moe::tune::kMxMaxSplitLen && p.nsplit < 16 &&
                   (N / (p.nsplit * 2)) % gran == 0)
                p.nsplit *= 2;
    } else {
        p.nsplit = moe::prefill_gemm2_splits(K, N, p.grid_blocks, is_fp8(dtype) ? 128 : 64);
    }
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += round_up(bytes);
        return at;
    };
    p.logits = take((size_t)M * E * 4);
    // the fused top-k + align kernel reads finished logits: split only when
    // the separate top-k kernel runs
    p.lsplit = moe::topk_align_fits(M, topk) ? 1 : moe::router_logit_splits(M, K, E);
    if (p.lsplit > 1) p.lpart = take((size_t)p.lsplit * M * E * 8);
    p.ids = take((size_t)slots * 4);
    p.wts = take((size_t)slots * 4);
    p.sorted = take((size_t)p.cap * 4);
    p.bexp = take((size_t)p.max_blocks * 4);
    p.offs = take((size_t)(E + 1) * 4);
    p.npad = take(4);
    p.align_multi = !moe::topk_align_fits(M, topk) && moe::align_multi_fits((int)slots);
    if (p.align_multi) {
        p.achunk = take((size_t)moe::align_chunks((int)slots) * E * 4);
        p.atot = take((size_t)E * 4);
    }
    if (is_fp8(dtype)) {
        p.xq = take((size_t)M * K);
        p.xs = take((size_t)M * 4);
        p.amax = take((size_t)p.cap * 4);
        p.inv = take((size_t)slots * 4);
        p.act = take((size_t)p.cap * N * 4);
        p.actq = take((size_t)p.cap * N);
        p.as = take((size_t)p.cap * 4);
    } else {
        p.act = take((size_t)p.cap * N * 2);
    }
    if (p.fused) p.nsplit = 1;  // GEMM2 and the combine in one launch: no partial rows
    else p.ypart = take((size_t)p.nsplit * slots * K * 4);
    p.total = o;
    return p;
}

}  // namespace

MOE_API const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

static moe_status finish_launches() {
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_topk(const void* x, const void* w_router, const float* router_bias, int M,
                            int K, int E, int topk, int32_t* topk_ids, float* topk_weights,
                            float* logits, void* stream) {
    if (M < 0 || K < 1 || E < 1 || topk < 1 || topk > E) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || topk > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if ((long)M * K >= (1L << 31) || (long)E * K >= (1L << 31)) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_weights || !logits) return MOE_ERR_INVALID_ARG;
    if (misaligned(x) || misaligned(w_router) || misaligned(router_bias) ||
        misaligned(topk_ids) || misaligned(topk_weights) || misaligned(logits))
        return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    // no workspace here: the logits are finished by the logits kernel itself
    moe::launch_router_logits(x, w_router, router_bias, M, K, E, logits, nullptr, nullptr, 1,
                              nullptr, s);
    moe::launch_router_topk(logits, M, E, topk, topk_ids, topk_weights, nullptr, 1, nullptr, s);
    return finish_launches();
}

MOE_API moe_status moe_quant_rows_e4m3(const void* x, int M, int K, uint8_t* q, float* scale,
                                       void* stream) {
    if (M < 0 || K < 1) return MOE_ERR_INVALID_ARG;
    if ((long)M * K >= (1L << 31)) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!x || !q || !scale || misaligned(x) || misaligned(q) || misaligned(scale))
        return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    moe::launch_quant_rows(x, M, K, q, scale, (hipStream_t)stream);
    return finish_launches();
}

static moe_status align_check(const int32_t* topk_ids, int M, int topk, int E, int block_m,
                              int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* expert_offsets, int32_t* num_padded) {
    if (M < 0 || topk < 1 || E < 1 || block_m < 1) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || block_m > 1024 || (long)M * topk >= (1L << 30))
        return MOE_ERR_UNSUPPORTED;
    if (!sorted_ids || !block_expert || !expert_offsets || !num_padded ||
        (M > 0 && !topk_ids))
        return MOE_ERR_INVALID_ARG;
    if (misaligned(topk_ids) || misaligned(sorted_ids) || misaligned(block_expert) ||
        misaligned(expert_offsets) || misaligned(num_padded))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

MOE_API moe_status moe_align(const int32_t* topk_ids, int M, int topk, int E, int block_m,
                             int32_t* sorted_ids, int32_t* block_expert,
                             int32_t* expert_offsets, int32_t* num_padded, void* stream) {
    const moe_status st = align_check(topk_ids, M, topk, E, block_m, sorted_ids, block_expert,
                                      expert_offsets, num_padded);
    if (st != MOE_OK) return st;
    const int n = M * topk;
    const int cap = n + E * (block_m - 1);
    (void)hipGetLastError();
    moe::launch_align(topk_ids, n, E, block_m, cap, sorted_ids, block_expert, expert_offsets,
                      num_padded, nullptr, 0, nullptr, (hipStream_t)stream);
    return finish_launches();
}

MOE_API moe_status moe_align_ex(const int32_t* topk_ids, int M, int topk, int E, int block_m,
                                int32_t* sorted_ids, int32_t* block_expert,
                                int32_t* expert_offsets, int32_t* num_padded, void* workspace,
                                size_t* workspace_bytes, void* stream) {
    if (!workspace_bytes) return MOE_ERR_INVALID_ARG;
    if (M < 0 || topk < 1 || E < 1 || block_m < 1) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || block_m > 1024 || (long)M * topk >= (1L << 30))
        return MOE_ERR_UNSUPPORTED;
    const int n = M * topk;
    const bool multi = moe::align_multi_fits(n);
    // chunk counts [chunks, E], then the experts' totals [E]
    const size_t chunk_bytes = round_up((size_t)moe::align_chunks(n) * E * 4);
    // a non-zero size even where the single-workgroup align uses no
    // scratch, so that a buffer sized from the query is never NULL (which
    // would read as another size query)
    const size_t need = multi ? chunk_bytes + round_up((size_t)E * 4) : kAlign;
    if (!workspace) {
        *workspace_bytes = need;
        return MOE_OK;
    }
    const moe_status st = align_check(topk_ids, M, topk, E, block_m, sorted_ids, block_expert,
                                      expert_offsets, num_padded);
    if (st != MOE_OK) return st;
    if ((uintptr_t)workspace & (kAlign - 1)) return MOE_ERR_INVALID_ARG;
    if (*workspace_bytes < need) return MOE_ERR_WORKSPACE;
    const int cap = n + E * (block_m - 1);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (multi)
        moe::launch_align_multi(topk_ids, n, E, block_m, cap, sorted_ids, block_expert,
                                expert_offsets, num_padded, nullptr, 0, nullptr,
                                (int32_t*)workspace, (int32_t*)((char*)workspace + chunk_bytes),
                                s);
    else
        moe::launch_align(topk_ids, n, E, block_m, cap, sorted_ids, block_expert, expert_offsets,
                          num_padded, nullptr, 0, nullptr, s);
    return finish_launches();
}

// Arguments that fix the plan (dtype, sizes, regime): the checks shared by
// the fused forward and the plan query.
static moe_status fused_shape_check(int dtype, int M, int K, int N, int E, int topk, int regime) {
    if (dtype != MOE_BF16 && !is_fp8(dtype)) return MOE_ERR_INVALID_ARG;
    if (regime < MOE_REGIME_AUTO || regime > MOE_REGIME_PREFILL) return MOE_ERR_INVALID_ARG;
    if (M < 0 || K < 1 || N < 1 || E < 1 || topk < 1 || topk > E) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || topk > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (K % 128 || N % 128) return MOE_ERR_UNSUPPORTED;
    // MXFP4: 256-deep decode steps and 256-row weight tiles; the decode
    // GEMM1 keeps K/32 scale bytes per row of its waves in LDS (K <= 16384:
    // 64 KB per workgroup)
    if (dtype == MOE_MXFP4_E2M1 && (K % 256 || N % 256 || K > moe::tune::kMxMaxK))
        return MOE_ERR_UNSUPPORTED;
    const long slots = (long)M * topk;
    // 32-bit buffer offsets: the sorted activation rows GEMM2 reads (bf16, or
    // e4m3 codes), the tokens and one expert's W1 must each stay below 2 GiB
    // (the fp32 activation and the partial rows are addressed in 64 bits)
    const long act_bytes = dtype == MOE_BF16 ? 2 : 1;
    if (slots >= (1L << 30) || (slots + (long)E * kPrefillBlock) * N * act_bytes >= (1L << 31) ||
        (long)M * K * 2 >= (1L << 31) || (long)2 * N * K * 2 >= (1L << 31) ||
        (long)E * 2 * N >= (1L << 31))
        return MOE_ERR_UNSUPPORTED;
    const Plan p = make_plan(dtype, M, K, N, E, topk, regime);
    if (p.max_blocks > 65535) return MOE_ERR_UNSUPPORTED;
    // MXFP4 decode GEMM2: a split's scale bytes must fit its LDS copy
    if (dtype == MOE_MXFP4_E2M1 && p.regime == MOE_REGIME_DECODE &&
        N / p.nsplit > moe::tune::kMxMaxSplitLen)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

MOE_API moe_status moe_fused_plan(int dtype, int M, int K, int N, int E, int topk, int regime,
                                  moe_plan* plan) {
    if (!plan) return MOE_ERR_INVALID_ARG;
    const moe_status st = fused_shape_check(dtype, M, K, N, E, topk, regime);
    if (st != MOE_OK) return st;
    const Plan p = make_plan(dtype, M, K, N, E, topk, regime);
    memset(plan, 0, sizeof(*plan));
    plan->regime = p.regime;
    plan->block_m = p.block;
    plan->sorted_rows = p.cap;
    plan->max_blocks = p.max_blocks;
    plan->gemm2_splits = p.nsplit;
    plan->logit_splits = p.lsplit;
    plan->fused_decode = p.fused ? 1 : 0;
    plan->workspace_bytes = p.total;
    plan->logits_offset = p.logits;
    plan->topk_ids_offset = p.ids;
    plan->topk_weights_offset = p.wts;
    plan->sorted_ids_offset = p.sorted;
    plan->block_expert_offset = p.bexp;
    plan->expert_offsets_offset = p.offs;
    plan->num_padded_offset = p.npad;
    return MOE_OK;
}

// Required tensors present and 16-byte aligned.
static bool fused_ptrs_ok(const void* x, const void* w_router, const float* router_bias,
                          const void* w1, const void* w2, const void* w1_scale,
                          const void* w2_scale, const void* out) {
    if (!x || !w_router || !w1 || !w2 || !out) return false;
    return !(misaligned(x) || misaligned(w_router) || misaligned(router_bias) ||
             misaligned(w1) || misaligned(w2) || misaligned(w1_scale) || misaligned(w2_scale) ||
             misaligned(out));
}

static moe_status fused_impl(const void* x, const void* w_router, const float* router_bias,
                             const void* w1, const void* w2, const void* w1_scale,
                             const void* w2_scale, int dtype, int M, int K, int N, int E,
                             int topk, int regime, void* out, void* workspace,
                             size_t* workspace_bytes, void* stream, void* const* events,
                             bool timed) {
    if (!workspace_bytes) return MOE_ERR_INVALID_ARG;
    if (dtype != MOE_BF16 && !is_fp8(dtype)) return MOE_ERR_INVALID_ARG;
    if (dtype == MOE_BF16 && (w1_scale || w2_scale)) return MOE_ERR_INVALID_ARG;
    if (is_fp8(dtype) && (!w1_scale || !w2_scale)) return MOE_ERR_INVALID_ARG;
    {
        const moe_status st = fused_shape_check(dtype, M, K, N, E, topk, regime);
        if (st != MOE_OK) return st;
    }
    const long slots = (long)M * topk;
    const Plan p = make_plan(dtype, M, K, N, E, topk, regime);
    if (!workspace) {
        *workspace_bytes = p.total;
        return MOE_OK;
    }
    if (M == 0) return MOE_OK;
    if (!fused_ptrs_ok(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, out) ||
        ((uintptr_t)workspace & (kAlign - 1)))
        return MOE_ERR_INVALID_ARG;
    if (*workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
    if (timed && !events) return MOE_ERR_INVALID_ARG;

    char* ws = (char*)workspace;
    float* logits = (float*)(ws + p.logits);
    int32_t* ids = (int32_t*)(ws + p.ids);
    float* wts = (float*)(ws + p.wts);
    int32_t* sorted = (int32_t*)(ws + p.sorted);
    int32_t* bexp = (int32_t*)(ws + p.bexp);
    int32_t* offs = (int32_t*)(ws + p.offs);
    int32_t* npad = (int32_t*)(ws + p.npad);
    float* ypart = (float*)(ws + p.ypart);
    const int nslots = (int)slots;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    auto mark = [&](int i) {
        if (timed) (void)hipEventRecord((hipEvent_t)events[i], s);
    };

    const bool fp8 = is_fp8(dtype);
    // per-channel scales: row r of expert e's W1 / W2 reads its own scale
    const int rowwise = dtype == MOE_FP8_E4M3_ROWWISE ? 1 : 0;
    uint8_t* xq = fp8 ? (uint8_t*)(ws + p.xq) : nullptr;
    float* xs = fp8 ? (float*)(ws + p.xs) : nullptr;
    // FP8: GEMM1's epilogue folds each row's |act| max into amax, which the
    // routing clears on the way
    uint32_t* amax = fp8 ? (uint32_t*)(ws + p.amax) : nullptr;
    const int amax_words = fp8 ? p.cap : 0;
    int32_t* inv = fp8 ? (int32_t*)(ws + p.inv) : nullptr;
    mark(0);
    if (p.fused) {
        // router, top-k, align and GEMM1 + SiLU*up in one launch, then GEMM2
        // and the combine in another
        void* act = ws + p.act;
        moe::launch_decode_route_gemm1_bf16(x, w_router, router_bias, w1, M, K, N, E, topk, p.cap,
                                            logits, ids, wts, sorted, bexp, offs, npad, act, s);
        for (int i = 1; i <= 5; ++i) mark(i);
        moe::launch_decode_gemm2_combine_bf16(act, w2, wts, sorted, bexp, M, K, N, E, topk, p.cap,
                                              out, s);
        mark(6);
        mark(7);
        return finish_launches();
    }
    if (moe::topk_align_fits(M, topk)) {
        // the FP8 token codes go with top-k + align when the tokens are few
        // and short (a wave per token there; a workgroup per token otherwise)
        const bool q_late = fp8 && M <= moe::tune::kLateQuantRows && K <= moe::tune::kLateQuantCols;
        moe::launch_router_logits(x, w_router, router_bias, M, K, E, logits,
                                  q_late ? nullptr : xq, xs, 1, nullptr, s);
        mark(1);
        moe::launch_topk_align(logits, x, M, K, E, topk, ids, wts, q_late ? xq : nullptr, xs,
                               p.block, p.cap, sorted, bexp, offs, npad, amax, amax_words, inv,
                               s);
        mark(2);
    } else {
        double* lpart = p.lsplit > 1 ? (double*)(ws + p.lpart) : nullptr;
        moe::launch_router_logits(x, w_router, router_bias, M, K, E, logits, xq, xs, p.lsplit,
                                  lpart, s);
        mark(1);
        moe::launch_router_topk(logits, M, E, topk, ids, wts, lpart, p.lsplit, router_bias, s);
        mark(2);
        if (p.align_multi)
            moe::launch_align_multi(ids, nslots, E, p.block, p.cap, sorted, bexp, offs, npad,
                                    amax, amax_words, inv, (int32_t*)(ws + p.achunk),
                                    (int32_t*)(ws + p.atot), s);
        else
            moe::launch_align(ids, nslots, E, p.block, p.cap, sorted, bexp, offs, npad, amax,
                              amax_words, inv, s);
    }
    mark(3);
    if (fp8) {
        float* act = (float*)(ws + p.act);
        uint8_t* actq = (uint8_t*)(ws + p.actq);
        float* as = (float*)(ws + p.as);
        const bool mx = dtype == MOE_MXFP4_E2M1;
        const bool tiles = p.regime == MOE_REGIME_PREFILL;
        if (tiles && mx)
            moe::launch_gemm1_prefill_mx(xq, xs, w1, (const uint8_t*)w1_scale, sorted, bexp, npad,
                                         M, topk, nslots, K, N, p.grid_blocks, act, amax, s);
        else if (tiles)
            moe::launch_gemm1_prefill_fp8(xq, xs, w1, (const float*)w1_scale, rowwise, sorted, bexp, npad, M,
                                          topk, nslots, K, N, p.grid_blocks, p.block, act, amax,
                                          s);
        else if (mx)
            moe::launch_gemm1_decode_mxfp4(xq, xs, w1, (const uint8_t*)w1_scale, sorted, bexp,
                                           npad, M, topk, nslots, K, N, p.grid_blocks,
                                           p.block / kDecodeBlock, act, amax, s);
        else
            moe::launch_gemm1_decode_fp8(xq, xs, w1, (const float*)w1_scale, rowwise, sorted, bexp, npad, M,
                                         topk, nslots, K, N, p.grid_blocks, p.block / kDecodeBlock,
                                         act, amax, s);
        mark(4);
        moe::launch_act_quant(act, amax, inv, nslots, N, actq, as, s);
        mark(5);
        if (tiles && mx)
            moe::launch_gemm2_prefill_mx(actq, as, w2, (const uint8_t*)w2_scale, wts, sorted, bexp,
                                         npad, p.cap, nslots, K, N, p.nsplit, p.grid_blocks, ypart,
                                         s);
        else if (tiles)
            moe::launch_gemm2_prefill_fp8(actq, as, w2, (const float*)w2_scale, rowwise, wts, sorted, bexp,
                                          npad, p.cap, nslots, K, N, p.nsplit, p.grid_blocks,
                                          p.block, ypart, s);
        else if (mx)
            moe::launch_gemm2_decode_mxfp4(actq, as, w2, (const uint8_t*)w2_scale, wts, sorted,
                                           bexp, npad, p.cap, nslots, K, N, p.nsplit,
                                           p.grid_blocks, p.block / kDecodeBlock, ypart, s);
        else
            moe::launch_gemm2_decode_fp8(actq, as, w2, (const float*)w2_scale, rowwise, wts, sorted, bexp,
                                         npad, p.cap, nslots, K, N, p.nsplit, p.grid_blocks,
                                         p.block / kDecodeBlock, ypart, s);
        mark(6);
    } else {
        void* act = ws + p.act;
        if (p.regime == MOE_REGIME_DECODE)
            moe::launch_gemm1_decode_bf16(x, w1, sorted, bexp, npad, M, topk, nslots, K, N,
                                          p.grid_blocks, p.block / kDecodeBlock, act, s);
        else
            moe::launch_gemm1_prefill_bf16(x, w1, sorted, bexp, npad, M, topk, nslots, K, N,
                                           p.grid_blocks, p.block, act, s);
        mark(4);
        mark(5);
        if (p.regime == MOE_REGIME_DECODE)
            moe::launch_gemm2_decode_bf16(act, w2, wts, sorted, bexp, npad, p.cap, nslots, K, N,
                                          p.nsplit, p.grid_blocks, p.block / kDecodeBlock, ypart,
                                          s);
        else
            moe::launch_gemm2_prefill_bf16(act, w2, wts, sorted, bexp, npad, p.cap, nslots, K, N,
                                           p.nsplit, p.grid_blocks, p.block, ypart, s);
        mark(6);
    }
    moe::launch_combine(ypart, M, K, topk, p.nsplit, out, s);
    mark(7);
    return finish_launches();
}

MOE_API moe_status moe_fused_forward_ex(const void* x, const void* w_router,
                                        const float* router_bias, const void* w1,
                                        const void* w2, const void* w1_scale,
                                        const void* w2_scale, int dtype, int M, int K, int N,
                                        int E, int topk, int regime, void* out,
                                        void* workspace, size_t* workspace_bytes,
                                        void* stream) {
    return fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, dtype, M, K, N, E,
                      topk, regime, out, workspace, workspace_bytes, stream, nullptr, false);
}

MOE_API moe_status moe_fused_forward_timed(const void* x, const void* w_router,
                                           const float* router_bias, const void* w1,
                                           const void* w2, const void* w1_scale,
                                           const void* w2_scale, int dtype, int M, int K,
                                           int N, int E, int topk, int regime, void* out,
                                           void* workspace, size_t* workspace_bytes,
                                           void* stream, void* const* events) {
    return fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, dtype, M, K, N, E,
                      topk, regime, out, workspace, workspace_bytes, stream, events, true);
}

MOE_API moe_status moe_fused_forward(const void* x, const void* w_router,
                                     const float* router_bias, const void* w1, const void* w2,
                                     const void* w1_scale, const void* w2_scale, int dtype,
                                     int M, int K, int N, int E, int topk, void* out,
                                     void* workspace, size_t* workspace_bytes, void* stream) {
    return moe_fused_forward_ex(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, dtype, M, K,
                                N, E, topk, MOE_REGIME_AUTO, out, workspace, workspace_bytes,
                                stream);
}

// ---------------------------------------------------------------------------
// The fused forward captured once into a HIP graph, for callers that replay
// the layer on fixed buffers (serving loops): one graph launch per call
// instead of the six to eight kernel launches.  The capture runs on a
// library-created stream; the layer issues no allocation, host
// synchronisation or memset, so its launch sequence is captured whole.
// ---------------------------------------------------------------------------
struct moe_graph_s {
    hipGraphExec_t exec = nullptr;
};

MOE_API moe_status moe_fused_graph_create(const void* x, const void* w_router,
                                          const float* router_bias, const void* w1,
                                          const void* w2, const void* w1_scale,
                                          const void* w2_scale, int dtype, int M, int K, int N,
                                          int E, int topk, int regime, void* out,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          moe_graph* graph) {
    if (!graph) return MOE_ERR_INVALID_ARG;
    *graph = nullptr;
    // every argument check of the eager call, before any HIP call
    {
        size_t need = 0;
        const moe_status st = fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale,
                                         dtype, M, K, N, E, topk, regime, out, nullptr, &need,
                                         stream, nullptr, false);
        if (st != MOE_OK) return st;
        if (M == 0) return MOE_ERR_INVALID_ARG;  // nothing to capture
        if (!workspace) return MOE_ERR_INVALID_ARG;
        if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
    }
    // one eager call on the caller's stream: validates the pointers and loads
    // every kernel the sequence uses before capture
    size_t have = workspace_bytes;
    {
        const moe_status st = fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale,
                                         dtype, M, K, N, E, topk, regime, out, workspace, &have,
                                         stream, nullptr, false);
        if (st != MOE_OK) return st;
    }
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_HIP;
    hipGraph_t g = nullptr;
    moe_status st = MOE_OK;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        st = MOE_ERR_HIP;
    } else {
        st = fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, dtype, M, K, N, E,
                        topk, regime, out, workspace, &have, cs, nullptr, false);
        // the capture always ends, whatever the layer returned
        if (hipStreamEndCapture(cs, &g) != hipSuccess && st == MOE_OK) st = MOE_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    if (st == MOE_OK && (!g || hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess))
        st = MOE_ERR_HIP;
    if (g) (void)hipGraphDestroy(g);
    (void)hipStreamDestroy(cs);
    (void)hipGetLastError();
    if (st != MOE_OK) {
        if (exec) (void)hipGraphExecDestroy(exec);
        return st;
    }
    moe_graph h = new (std::nothrow) moe_graph_s;
    if (!h) {
        (void)hipGraphExecDestroy(exec);
        return MOE_ERR_HIP;
    }
    h->exec = exec;
    *graph = h;
    return MOE_OK;
}

MOE_API moe_status moe_fused_graph_launch(moe_graph graph, void* stream) {
    if (!graph || !graph->exec) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hipGraphLaunch(graph->exec, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_fused_graph_destroy(moe_graph graph) {
    if (!graph) return MOE_OK;
    const hipError_t e = graph->exec ? hipGraphExecDestroy(graph->exec) : hipSuccess;
    delete graph;
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The fused forward without a caller workspace, for callers that cannot
// allocate device memory.  Its scratch is a file-scope device array: every
// GPU the library runs on holds one copy (kNoAllocScratchBytes) until the
// process ends.  In host code `scratch` only names the symbol; the device
// address of the current GPU's copy comes from hipGetSymbolAddress, taken
// once per device on the first call there and kept in g_scratch.
// ---------------------------------------------------------------------------
namespace moe {
// external linkage (hidden by the library's default visibility), so the
// runtime registers it under a stable name for hipGetSymbolAddress
__device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];
}  // namespace moe

namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
}  // namespace

MOE_API moe_status moe_fused_forward_noalloc(const void* x, const void* w_router,
                                             const float* router_bias, const void* w1,
                                             const void* w2, const void* w1_scale,
                                             const void* w2_scale, int dtype, int M, int K,
                                             int N, int E, int topk, void* out, void* stream) {
    // the plan's size first: argument errors and oversized shapes are
    // reported before any HIP call
    size_t need = 0;
    {
        const moe_status st = fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale,
                                         dtype, M, K, N, E, topk, MOE_REGIME_AUTO, out, nullptr,
                                         &need, stream, nullptr, false);
        if (st != MOE_OK) return st;
    }
    if (need > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
    if (M == 0) return MOE_OK;
    if (!fused_ptrs_ok(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, out))
        return MOE_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
    if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        g_scratch_rc[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(moe::scratch));
        g_scratch[dev] = g_scratch_rc[dev] == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_rc[dev] != hipSuccess || !g_scratch[dev]) return MOE_ERR_HIP;
    size_t have = kNoAllocScratchBytes;
    return fused_impl(x, w_router, router_bias, w1, w2, w1_scale, w2_scale, dtype, M, K, N, E,
                      topk, MOE_REGIME_AUTO, out, g_scratch[dev], &have, stream, nullptr, false);
}
