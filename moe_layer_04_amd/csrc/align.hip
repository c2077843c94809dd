// align.hip -- moe_align on gfx950: the expert-sorted, block-padded
// permutation of token slots ("data shuffling" of the fused MoE in
// "Mixture-of-Experts kernel engineering on Amazon SageMaker AI", summary
// text; per-expert batch sizes that change from call to call, "Amazon
// SageMaker AI上的混合专家模型内核工程优化", H200 bottleneck section).
//
// Slot p = t*topk + j is sorted stably by expert; each expert's segment is
// padded to a multiple of the block size with the sentinel n = M*topk.
// One 1024-thread workgroup runs the align body of routing.hpp; for more
// than 2048 slots three launches spread the same work over a workgroup per
// 1024-slot chunk (below), with an identical result.
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
    __shared__ float swt[kRouteSmallMaxSlots];
    __shared__ float slog[kRouteSmallMaxTokens * MOE_KERNEL_MAX_EXPERTS];
    __shared__ AlignShared sh;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int tid = (int)threadIdx.x;
    // The batch's logits go to LDS in one pass, and each token's picks stay
    // in LDS until all are done: a wave takes several tokens in turn, and
    // with global loads and stores per token every token would wait for the
    // previous one's stores (one counter tracks both) and for its own load.
    {
        constexpr int kPer = kRouteSmallMaxTokens * MOE_KERNEL_MAX_EXPERTS / kAlignThreads;
        const int n = M * E;
        float v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + j * kAlignThreads;
            v[j] = i < n ? logits[i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + j * kAlignThreads;
            if (i < n) slog[i] = v[j];
        }
    }
    if (xq)
        for (int t = wave; t < M; t += kAlignWaves)
            quant_row_wave(x + (size_t)t * K, K, xq + (size_t)t * K, xscale + t);
    __syncthreads();
    if (E <= 16) {
        // four tokens per wave at once, one per 16-lane row
        for (int t0 = 4 * wave; t0 < M; t0 += 4 * kAlignWaves) {
            const int t = t0 + (lane_id() >> 4);
            const bool valid = t < M;
            const int tt = valid ? t : 0;
            topk_row16(slog + tt * E, valid, E, topk, sid + tt * topk, swt + tt * topk);
        }
    } else {
        for (int t = wave; t < M; t += kAlignWaves)
            topk_wave(slog + t * E, E, topk, sid + t * topk, swt + t * topk, nullptr);
    }
    __syncthreads();
    for (int i = tid; i < M * topk; i += kAlignThreads) {
        topk_ids[i] = sid[i];
        topk_weights[i] = swt[i];
    }
    align_body(sh, sid, M * topk, E, B, cap, sorted_ids, block_expert, expert_offsets,
               num_padded, zero_buf, zero_words, inv);
}

// ---------------------------------------------------------------------------
// The same top-k + align for one or two tokens in a single wave (no
// workgroup barriers, a 64-thread launch); the align is align_wave.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void topk_align_wave_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int K, int E,
    int topk, int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    uint8_t* __restrict__ xq, float* __restrict__ xscale, int B, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_padded,
    uint32_t* __restrict__ zero_buf, int zero_words, int32_t* __restrict__ inv) {
    __shared__ int32_t sid[kWave];
    __shared__ int cnt[MOE_KERNEL_MAX_EXPERTS];
    __shared__ int off[MOE_KERNEL_MAX_EXPERTS + 1];
    if (xq)
        for (int t = 0; t < M; ++t)
            quant_row_wave(x + (size_t)t * K, K, xq + (size_t)t * K, xscale + t);
    for (int t = 0; t < M; ++t)
        topk_wave(logits + (size_t)t * E, E, topk, topk_ids + (size_t)t * topk,
                  topk_weights + (size_t)t * topk, sid + t * topk);
    __syncthreads();  // one wave: orders the LDS writes above before the reads below
    align_wave(sid, M * topk, E, B, cap, cnt, off, sorted_ids, block_expert, expert_offsets,
               num_padded, zero_buf, zero_words, inv);
}

// ---------------------------------------------------------------------------
// The same permutation for large batches over many workgroups, in three
// launches.  The slots are cut into chunks of kAlignThreads, as the single
// workgroup walks them; (1) a workgroup per chunk counts its slots per
// expert; (2) one workgroup adds the counts up, scans the padded totals into
// the experts' offsets and gives every (chunk, expert) its first position:
// the expert's offset plus that expert's slots in earlier chunks -- exactly
// the running count the single workgroup carries from chunk to chunk; (3) a
// workgroup per chunk places its slots at that base plus their rank inside
// the chunk (the same ballot ranks), and all workgroups share the sentinel
// and block-owner writes.  The result is identical to align_kernel's.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ chunk_cnt) {
    __shared__ int cnt[MOE_KERNEL_MAX_EXPERTS];
    const int tid = (int)threadIdx.x;
    const int c = (int)blockIdx.x;
    for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;
    __syncthreads();
    const int p = c * kAlignThreads + tid;
    if (p < n) atomicAdd(&cnt[min(max(ids[p], 0), E - 1)], 1);  // counts are order-free
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) chunk_cnt[(size_t)c * E + e] = cnt[e];
}

// One workgroup; chunk_cnt [nchunk,E] becomes the chunk bases; cnt_total [E]
// receives each expert's slot count.
__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(
    int nchunk, int E, int B, int32_t* __restrict__ chunk_cnt, int32_t* __restrict__ cnt_total,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_padded) {
    __shared__ int tot[MOE_KERNEL_MAX_EXPERTS];
    __shared__ int off[MOE_KERNEL_MAX_EXPERTS + 1];
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    // per expert: exclusive prefix of its counts over the chunks (in place)
    for (int e = tid; e < E; e += kAlignThreads) {
        int run = 0;
        for (int c = 0; c < nchunk; ++c) {
            const int v = chunk_cnt[(size_t)c * E + e];
            chunk_cnt[(size_t)c * E + e] = run;
            run += v;
        }
        tot[e] = run;
    }
    __syncthreads();
    if (wave == 0) {
        int v[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            v[i] = (e < E) ? (tot[e] + B - 1) / B * B : 0;
            sum += v[i];
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int base = incl - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            if (e < E) off[e] = base;
            base += v[i];
        }
        if (lane == kWave - 1) off[E] = incl;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += kAlignThreads) expert_offsets[e] = off[e];
    for (int e = tid; e < E; e += kAlignThreads) cnt_total[e] = tot[e];
    if (tid == 0) *num_padded = off[E];
    for (int i = tid; i < nchunk * E; i += kAlignThreads) chunk_cnt[i] += off[i % E];
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int n, int E, int B, int cap,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ cnt_total,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, uint32_t* __restrict__ zero_buf, int zero_words,
    int32_t* __restrict__ inv) {
    __shared__ int cnt[MOE_KERNEL_MAX_EXPERTS];
    __shared__ int off[MOE_KERNEL_MAX_EXPERTS + 1];
    __shared__ int wc[kAlignWaves][MOE_KERNEL_MAX_EXPERTS];
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int c = (int)blockIdx.x;
    const int nthreads = (int)gridDim.x * kAlignThreads;
    const int gtid = c * kAlignThreads + tid;
    for (int i = gtid; i < zero_words; i += nthreads) zero_buf[i] = 0u;
    for (int e = tid; e < E; e += kAlignThreads) cnt[e] = cnt_total[e];
    for (int e = tid; e <= E; e += kAlignThreads) off[e] = expert_offsets[e];
    for (int i = tid; i < kAlignWaves * MOE_KERNEL_MAX_EXPERTS; i += kAlignThreads)
        (&wc[0][0])[i] = 0;
    __syncthreads();
    const int npad = off[E];
    // sentinels and block owners, shared by all workgroups
    for (int i = gtid; i < cap; i += nthreads) {
        bool pad = (i >= npad);
        if (!pad) {
            int lo = 0, hi = E - 1;  // last e with off[e] <= i
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            pad = (i - off[lo]) >= cnt[lo];
        }
        if (pad) sorted_ids[i] = n;
    }
    for (int b = gtid; b < cap / B; b += nthreads) {
        const int i = b * B;
        int owner = -1;
        if (i < npad) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        block_expert[b] = owner;
    }
    // this chunk's slots: rank among earlier slots of the same expert
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int p = c * kAlignThreads + tid;
    const bool valid = p < n;
    const int e = valid ? min(max(ids[p], 0), E - 1) : 0;
    uint64_t match = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool on = (e >> bit) & 1;
        const uint64_t bb = __ballot(valid && on);
        match &= on ? bb : ~bb;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && (match >> lane) == 1ull) wc[wave][e] = __popcll(match);  // last lane of its group
    __syncthreads();
    if (valid) {
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wc[w][e];
        const int pos = chunk_base[(size_t)c * E + e] + before + rank;
        sorted_ids[pos] = p;
        if (inv) inv[p] = pos;
    }
}

static_assert(kAlignThreads == 1024, "align_chunks counts chunks of 1024 slots");

bool align_multi_fits(int n) { return n > kAlignMultiMinSlots; }

void launch_align_multi(const int32_t* ids, int n, int E, int B, int cap, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
                        uint32_t* zero_buf, int zero_words, int32_t* inv, int32_t* chunk_cnt,
                        int32_t* cnt_total, hipStream_t s) {
    const int nchunk = align_chunks(n);
    align_count_kernel<<<nchunk, kAlignThreads, 0, s>>>(ids, n, E, chunk_cnt);
    align_scan_kernel<<<1, kAlignThreads, 0, s>>>(nchunk, E, B, chunk_cnt, cnt_total,
                                                  expert_offsets, num_padded);
    align_scatter_kernel<<<nchunk, kAlignThreads, 0, s>>>(ids, n, E, B, cap, chunk_cnt, cnt_total,
                                                          expert_offsets, sorted_ids, block_expert,
                                                          zero_buf, zero_words, inv);
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
    // one wave does the top-k of the tokens one after another: only for one
    // or two tokens (M = 1: 0.9 us faster; M = 8: 6.7 us slower than a wave
    // per token in the workgroup version)
    if (M <= 2 && (long)M * topk <= kWave) {
        topk_align_wave_kernel<<<1, kWave, 0, s>>>(
            logits, (const uint16_t*)x, M, K, E, topk, ids, w, xq, xscale, B, cap, sorted_ids,
            block_expert, expert_offsets, num_padded, zero_buf, zero_words, inv);
        return;
    }
    topk_align_kernel<<<1, kAlignThreads, 0, s>>>(
        logits, (const uint16_t*)x, M, K, E, topk, ids, w, xq, xscale, B, cap, sorted_ids,
        block_expert, expert_offsets, num_padded, zero_buf, zero_words, inv);
}

}  // namespace moe
