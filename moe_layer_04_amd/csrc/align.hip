// align.hip -- moe_align on gfx950: the expert-sorted, block-padded
// permutation of token slots ("data shuffling" of the fused MoE in
// "Mixture-of-Experts kernel engineering on Amazon SageMaker AI", summary
// text; per-expert batch sizes that change from call to call, "Amazon
// SageMaker AI上的混合专家模型内核工程优化", H200 bottleneck section).
//
// Slot p = t*topk + j is sorted stably by expert; each expert's segment is
// padded to a multiple of the block size with the sentinel n = M*topk.
// One 1024-thread workgroup runs the align body of routing.hpp.
#include "routing.hpp"

namespace moe {

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int n, int E, int B, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_padded,
    uint32_t* __restrict__ zero_buf, int zero_words, int32_t* __restrict__ inv) {
    __shared__ AlignShared sh;
    align_body(sh, ids, n, E, B, cap, sorted_ids, block_expert, expert_offsets, num_padded,
               zero_buf, zero_words, inv);
}

// ---------------------------------------------------------------------------
// Top-k and align of a batch of at most kRouteSmallMaxTokens tokens and
// kRouteSmallMaxSlots token-slots in one workgroup (one launch instead of two): the top-k of every token (a
// wave per token) with the picked ids kept in LDS, then the align body over
// them; for the FP8 path with few tokens also the per-token e4m3 rows (a
// wave per token).  The arithmetic is that of the separate kernels, so ids,
// weights and codes are identical.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAlignThreads) void topk_align_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int K, int E,
    int topk, int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    uint8_t* __restrict__ xq, float* __restrict__ xscale, int B, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_padded,
    uint32_t* __restrict__ zero_buf, int zero_words, int32_t* __restrict__ inv) {
    __shared__ int32_t sid[kRouteSmallMaxSlots];
    __shared__ AlignShared sh;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    if (xq)
        for (int t = wave; t < M; t += kAlignWaves)
            quant_row_wave(x + (size_t)t * K, K, xq + (size_t)t * K, xscale + t);
    for (int t = wave; t < M; t += kAlignWaves)
        topk_wave(logits + (size_t)t * E, E, topk, topk_ids + (size_t)t * topk,
                  topk_weights + (size_t)t * topk, sid + t * topk);
    __syncthreads();
    align_body(sh, sid, M * topk, E, B, cap, sorted_ids, block_expert, expert_offsets,
               num_padded, zero_buf, zero_words, inv);
}

void launch_align(const int32_t* ids, int n, int E, int B, int cap, int32_t* sorted_ids,
                  int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
                  uint32_t* zero_buf, int zero_words, int32_t* inv, hipStream_t s) {
    align_kernel<<<1, kAlignThreads, 0, s>>>(ids, n, E, B, cap, sorted_ids, block_expert,
                                             expert_offsets, num_padded, zero_buf, zero_words,
                                             inv);
}

bool topk_align_fits(int M, int topk) {
    // each wave handles M / 16 tokens one after another: only for few tokens
    return M <= kRouteSmallMaxTokens && (long)M * topk <= kRouteSmallMaxSlots;
}

void launch_topk_align(const float* logits, const void* x, int M, int K, int E, int topk,
                       int32_t* ids, float* w, uint8_t* xq, float* xscale, int B, int cap,
                       int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                       int32_t* num_padded, uint32_t* zero_buf, int zero_words, int32_t* inv,
                       hipStream_t s) {
    topk_align_kernel<<<1, kAlignThreads, 0, s>>>(
        logits, (const uint16_t*)x, M, K, E, topk, ids, w, xq, xscale, B, cap, sorted_ids,
        block_expert, expert_offsets, num_padded, zero_buf, zero_words, inv);
}

}  // namespace moe
